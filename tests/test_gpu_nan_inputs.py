"""GPU: tokens whose activations hold NaN.

A NaN logit ranks as -infinity in the top-K, so every path still selects K
distinct experts in [0, E) for such a token (its output is NaN), the prefill
grouping stays a permutation, and the other tokens of the batch are computed
as usual: they are compared with the oracle.
"""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _layer(w, seed=0):
    from int4_expert_ffn_int8_amd.layer import MoeLayer
    router = synth.router_tensors(w, 0, seed)
    experts = [synth.expert_tensors(w, 0, e, seed) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"], seed) if w["n_shared"] else None
    L = MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                 router, experts, shared)
    return L, router, experts, shared


def _poison(xb, rows):
    x = xb.copy()
    for t in rows:
        x[t, ::7] = 0x7FC0  # bf16 quiet NaN in every 7th column
    return x


def _check_selection(idx, K, E):
    idx = np.asarray(idx)
    assert ((idx >= 0) & (idx < E)).all(), idx
    for row in idx:
        assert len(set(row.tolist())) == K, row


def _check_good_tokens(w, router, experts, shared, x_bits, good, out_bits):
    o_ref = O.moe_block(w, router, lambda e: experts[e], x_bits[good], shared=shared)
    assert_bf16_output_close(out_bits[good], o_ref, "tokens without NaN")


def test_fused_decode_with_nan_token():
    # (two tokens of K + shared = 3 pairs fit the fused path's 8 pairs)
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0)
    L, router, experts, shared = _layer(w)
    fb = L.fused_buffers(2)
    xb = _poison(synth.tokens(w, 11, T=2), [0])
    print("fused decode, NaN token 0", flush=True)
    L.decode_fused(dev(xb), fb)
    torch.cuda.synchronize()
    _check_selection(fb["idx"].cpu().numpy(), w["K"], w["E"])
    assert L.fused_error_word(fb) == 0
    out = fb["out"].cpu().numpy().view(np.uint16)
    _check_good_tokens(w, router, experts, shared, xb, [1], out)


def test_three_call_decode_with_nan_token():
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(1)
    L, router, experts, shared = _layer(w, seed=1)
    b = L.buffers(3)
    xb = _poison(synth.tokens(w, 12, T=3, seed=1), [1])
    print("three-call decode, NaN token 1", flush=True)
    L.forward(dev(xb), b)
    torch.cuda.synchronize()
    _check_selection(b["idx"].cpu().numpy(), w["K"], w["E"])
    out = b["out"].cpu().numpy().view(np.uint16)
    _check_good_tokens(w, router, experts, shared, xb, [0, 2], out)


def test_prefill_with_nan_tokens():
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0, H=256, E=64, K=4, I=128, r=4, n_shared=1)
    L, router, experts, shared = _layer(w, seed=2)
    T = 300
    bad = [0, 77, 299]
    xb = _poison(synth.tokens(w, 13, T=T, seed=2), bad)
    b = L.buffers(T, prefill=True)
    print("prefill, NaN tokens", bad, flush=True)
    L.forward(dev(xb), b)
    torch.cuda.synchronize()
    gi = b["idx"].cpu().numpy()
    _check_selection(gi, w["K"], w["E"])
    counts, offsets, perm = O.group_pairs(gi, w["E"])
    assert b["counts"].cpu().numpy().tolist() == counts.tolist()
    assert b["perm"].cpu().numpy()[:T * w["K"]].tolist() == perm.tolist()
    good = [t for t in range(T) if t not in bad]
    out = b["out"].cpu().numpy().view(np.uint16)
    _check_good_tokens(w, router, experts, shared, xb, good, out)
