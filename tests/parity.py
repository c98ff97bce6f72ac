"""Parity helpers shared by the GPU tests (comparison logic only)."""
from __future__ import annotations

import numpy as np

import oracle as O

REL_TOL = 1e-2  # max |err| <= 1e-2 * RMS(reference), fp32 accumulation


def rms(a) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def assert_close_rms(got, ref, what: str, rel: float = REL_TOL, extra=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = rel * rms(ref) + extra
    worst = float(err.max()) if err.size else 0.0
    assert np.all(err <= bound), (
        f"{what}: max|err|={worst:.3e} > {rel:g}*RMS={bound:.3e} at "
        f"{np.unravel_index(int(np.argmax(err - bound)), err.shape)}")
    return worst / max(rms(ref), 1e-300)


def bf16_half_ulp(ref):
    """Half a bf16 unit in the last place at each reference value."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def assert_bf16_output_close(got_bits, ref_o, what: str):
    """bf16 output vs the oracle's unrounded fp64 value: the kernel's own
    final rounding (half a bf16 ulp) is allowed on top of 1e-2 * RMS."""
    got = O.bf16_to_f64(np.asarray(got_bits).view(np.uint16))
    ref = np.asarray(ref_o, dtype=np.float64)
    err = np.abs(got - ref)
    bound = REL_TOL * rms(ref) + bf16_half_ulp(ref)
    assert np.all(err <= bound), (
        f"{what}: max excess {float((err - bound).max()):.3e}, max|err|={float(err.max()):.3e}, "
        f"RMS={rms(ref):.3e}")
    return float(err.max()) / max(rms(ref), 1e-300)


def check_routing(gpu_logits, gpu_idx, gpu_w, ref_logits, K, norm_topk=True,
                  max_near_ties=0):
    """Routing parity, decomposed:
    (i)   |logits_gpu - logits_oracle| <= 1e-2 * RMS(logits_oracle);
    (ii)  the oracle's selection and weights applied to the GPU's own logits
          reproduce the GPU's indices exactly and its weights to 1e-5;
    (iii) GPU indices equal the oracle's for every token whose oracle margin
          (K-th minus (K+1)-th logit) exceeds 2 * max logit error.
    Tokens under the margin are certified near-ties; returns their list."""
    gl = np.asarray(gpu_logits, dtype=np.float64)
    rl = np.asarray(ref_logits, dtype=np.float64)
    T, E = rl.shape
    assert_close_rms(gl, rl, "router logits")
    err = float(np.abs(gl - rl).max()) if gl.size else 0.0
    gi = np.asarray(gpu_idx)
    gw = np.asarray(gpu_w, dtype=np.float64)
    near = []
    for t in range(T):
        sel = O.select_topk(gl[t], K)
        assert sel.tolist() == gi[t].tolist(), (t, sel, gi[t])
        wref = O.topk_weights(gl[t], sel, norm_topk)
        assert np.allclose(gw[t], wref, rtol=1e-5, atol=1e-7), (t, gw[t], wref)
        order = np.lexsort((np.arange(E), -rl[t]))
        margin = np.inf if K == E else rl[t, order[K - 1]] - rl[t, order[K]]
        if margin > 2 * err:
            assert order[:K].tolist() == gi[t].tolist(), (t, order[:K], gi[t], margin, err)
        else:
            near.append(t)
    assert len(near) <= max_near_ties, f"near-ties {near} exceed {max_near_ties}"
    return near
