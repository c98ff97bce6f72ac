"""GPU parity of the unmerged LoRA delta on every path, through the C ABI.

The LoRA delta of a normal expert is about 1% of its output, small enough to
hide inside the 1e-2 * RMS block tolerance.  So the delta is isolated:

* LoRA-only experts (every group scale and bias 0, B scaled up): the output
  is the LoRA chain alone, lambda B_d A_d (silu(lambda B_g A_g x) *
  lambda B_u A_u x), so a dropped, squared or misplaced lambda, or a wrong
  LoRA operand, moves the whole output;
* B = 0 experts: the base alone, so a LoRA term that leaks into the base
  shows;
* lambda = 0.5 and 2 on LoRA-only experts, through the fused block
  (moe_block_decode and moe_block_decode_exec), the three-call decode path
  and the prefill path.

[P1] Recover-LoRA paragraph and [P3] "三件套" bullets: the adapter stays
unmerged and its delta is added at inference.

Also here: the fused block at 3 and 4 tokens with one routed expert per
token (its largest token count).
"""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close, assert_close_rms, check_routing, rms

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


def _experts(w, seed, mode):
    """Routed experts + shared expert of layer 0; mode 'lora_only' zeroes the
    base and scales B by 50, 'b_zero' zeroes every B, 'plain' keeps them."""
    experts = [synth.expert_tensors(w, 0, e, seed) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"], seed) if w["n_shared"] else None
    for ex in experts + ([shared] if shared is not None else []):
        for p in ("gate", "up", "down"):
            if mode == "lora_only":
                ex[f"s_{p}"] = np.zeros_like(ex[f"s_{p}"])
                ex[f"b_{p}"] = np.zeros_like(ex[f"b_{p}"])
                ex[f"B_{p}"] = synth.f32_to_bf16_bits(O.bf16_to_f64(ex[f"B_{p}"]) * 50.0)
            elif mode == "b_zero":
                ex[f"B_{p}"] = np.zeros_like(ex[f"B_{p}"])
    return experts, shared


def _layer(w, seed=0, mode="plain"):
    from int4_expert_ffn_int8_amd.layer import MoeLayer
    router = synth.router_tensors(w, 0, seed)
    experts, shared = _experts(w, seed, mode)
    L = MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                 router, experts, shared)
    return L, router, experts, shared


def _check_lora_only_is_lora(w, experts, shared, x_bits, idx):
    """The LoRA-only outputs must not be ~0 (they are the whole signal)."""
    x = O.bf16_to_f64(x_bits)
    y = O.expert_forward(experts[int(idx[0, 0])], x[:1], w["lora_scale"])
    assert rms(y) > 1e-3


# ---------------------------------------------------------------------------
# fused block (the decode bench path), 35B shape
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode,lam", [("lora_only", 1.0), ("lora_only", 0.5),
                                      ("lora_only", 2.0), ("b_zero", 2.0)])
def test_fused_block_lora_isolated_35b(mode, lam):
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(1, lora_scale=lam)
    L, router, experts, shared = _layer(w, seed=2, mode=mode)
    fb = L.fused_buffers(1)
    for step in range(2):
        print(f"fused 35b {mode} lam={lam} step={step}", flush=True)
        xb = synth.tokens(w, 20 + step, seed=2)
        L.decode_fused(dev(xb), fb)
        torch.cuda.synchronize()
        o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                                   return_parts=True)
        assert fb["idx"].cpu().numpy().tolist() == parts["idx"].tolist()
        assert np.allclose(fb["w"].cpu().numpy(), parts["w"], rtol=1e-5, atol=1e-7)
        if mode == "lora_only":
            _check_lora_only_is_lora(w, experts, shared, xb, parts["idx"])
        assert_bf16_output_close(_bits(fb["out"]), o_ref, f"fused {mode} lam={lam}")
    assert L.fused_error_word(fb) == 0


@pytest.mark.parametrize("mode,lam", [("lora_only", 0.5), ("lora_only", 2.0), ("b_zero", 1.0)])
def test_fused_exec_lora_isolated_35b(mode, lam):
    # prediction-as-routing: given experts (unrelated to the router's choice)
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(1, lora_scale=lam)
    L, router, experts, shared = _layer(w, seed=3, mode=mode)
    fb = L.fused_buffers(1)
    rng = np.random.default_rng(77)
    for step in range(2):
        print(f"exec 35b {mode} lam={lam} step={step}", flush=True)
        xb = synth.tokens(w, 30 + step, seed=3)
        given = rng.permutation(w["E"])[:w["K"]].reshape(1, -1).astype(np.int32)
        L.decode_fused(dev(xb), fb, exec_idx=dev(given))
        torch.cuda.synchronize()
        o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                                   return_parts=True, exec_idx=given)
        assert fb["idx"].cpu().numpy().tolist() == given.tolist()
        assert np.allclose(fb["w"].cpu().numpy(), parts["w"], rtol=1e-5, atol=1e-7)
        assert_bf16_output_close(_bits(fb["out"]), o_ref, f"exec {mode} lam={lam}")
    assert L.fused_error_word(fb) == 0


@pytest.mark.parametrize("wid,K,T", [(0, 1, 3), (0, 1, 4), (1, 1, 4), (1, 1, 3), (0, 3, 2)])
def test_fused_block_largest_token_counts(wid, K, T):
    # T (K + shared) reaches the fused path's 8 pairs: 4 tokens x (1 + 1)
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(wid, K=K, lora_scale=0.5)
    L, router, experts, shared = _layer(w, seed=4)
    fb = L.fused_buffers(T)
    for step in range(2):
        print(f"fused wid={wid} K={K} T={T} step={step}", flush=True)
        xb = synth.tokens(w, 50 + step, T=T, seed=4)
        L.decode_fused(dev(xb), fb)
        torch.cuda.synchronize()
        o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                                   return_parts=True)
        assert fb["idx"].cpu().numpy().tolist() == parts["idx"].tolist()
        assert np.allclose(fb["w"].cpu().numpy(), parts["w"], rtol=1e-5, atol=1e-7)
        assert_bf16_output_close(_bits(fb["out"]), o_ref, f"fused K={K} T={T}")
    assert L.fused_error_word(fb) == 0


# ---------------------------------------------------------------------------
# three-call decode path
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wid,lam", [(0, 0.5), (0, 2.0), (1, 2.0)])
def test_three_call_lora_only_lambda(wid, lam):
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(wid, lora_scale=lam)
    L, router, experts, shared = _layer(w, seed=5, mode="lora_only")
    T = 3
    xb = synth.tokens(w, 7, T=T, seed=5)
    b = L.buffers(T)
    L.forward(dev(xb), b)
    torch.cuda.synchronize()
    o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                               return_parts=True)
    near = check_routing(b["logits"].cpu().numpy(), b["idx"].cpu().numpy(),
                         b["w"].cpu().numpy(), parts["logits"], w["K"])
    assert not near
    gi = b["idx"].cpu().numpy()
    _check_lora_only_is_lora(w, experts, shared, xb, gi)
    x = O.bf16_to_f64(xb)
    y_ref = np.zeros((T, w["K"] + w["n_shared"], w["H"]))
    for t in range(T):
        for k in range(w["K"]):
            y_ref[t, k] = O.expert_forward(experts[gi[t, k]], x[t:t + 1], lam)[0]
        if w["n_shared"]:
            y_ref[t, w["K"]] = O.expert_forward(shared, x[t:t + 1], lam)[0]
    assert_close_rms(b["y"].cpu().numpy(), y_ref, f"three-call y lam={lam}")
    assert_bf16_output_close(_bits(b["out"]), o_ref, f"three-call out lam={lam}")


# ---------------------------------------------------------------------------
# prefill path
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wid,T,lam", [(0, 90, 0.5), (0, 90, 2.0), (1, 300, 2.0)])
def test_prefill_lora_only_lambda(wid, T, lam):
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(wid, lora_scale=lam)
    L, router, experts, shared = _layer(w, seed=6, mode="lora_only")
    xb = synth.tokens(w, 8, T=T, seed=6)
    b = L.buffers(T, prefill=True)
    L.forward(dev(xb), b)
    torch.cuda.synchronize()
    o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                               return_parts=True)
    near = check_routing(b["logits"].cpu().numpy(), b["idx"].cpu().numpy(),
                         b["w"].cpu().numpy(), parts["logits"], w["K"], max_near_ties=2)
    gi = b["idx"].cpu().numpy()
    _check_lora_only_is_lora(w, experts, shared, xb, gi)
    x = O.bf16_to_f64(xb)
    y_ref = np.zeros((T, w["K"] + w["n_shared"], w["H"]))
    for e in np.unique(gi):
        rows, ks = np.nonzero(gi == e)
        y_ref[rows, ks] = O.expert_forward(experts[int(e)], x[rows], lam)
    if w["n_shared"]:
        y_ref[:, w["K"]] = O.expert_forward(shared, x, lam)
    assert_close_rms(b["y"].cpu().numpy(), y_ref, f"prefill y lam={lam}")
    ok = [t for t in range(T) if t not in near]
    assert_bf16_output_close(_bits(b["out"])[ok], o_ref[ok], f"prefill out lam={lam}")
