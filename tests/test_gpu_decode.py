"""GPU parity of the decode path (router, expert GEMV, combine) against the
CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synth
from parity import (assert_bf16_output_close, assert_close_rms, check_routing, rms)

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _layer(w, seed=0, layer=0, experts=None, shared=None, router=None):
    from int4_expert_ffn_int8_amd.layer import MoeLayer
    router = router or synth.router_tensors(w, layer, seed)
    if experts is None:
        experts = [synth.expert_tensors(w, layer, e, seed) for e in range(w["E"])]
    if shared is None and w["n_shared"]:
        shared = synth.expert_tensors(w, layer, w["E"], seed)
    L = MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                 router, experts, shared, norm_topk=w.get("norm_topk", 1))
    return L, router, experts, shared


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


def _run_block(w, L, router, experts, shared, x_bits, max_near_ties=0):
    from int4_expert_ffn_int8_amd.layer import dev
    T = x_bits.shape[0]
    x = dev(x_bits)
    b = L.buffers(T)
    L.forward(x, b)
    torch.cuda.synchronize()
    o_ref, parts = O.moe_block(w, router, lambda e: experts[e], x_bits, shared=shared,
                               return_parts=True)
    gl = b["logits"].cpu().numpy()
    gi = b["idx"].cpu().numpy()
    gw = b["w"].cpu().numpy()
    near = check_routing(gl, gi, gw, parts["logits"], w["K"], bool(w.get("norm_topk", 1)),
                         max_near_ties)
    # expert outputs for the GPU's own selection
    y = b["y"].cpu().numpy()
    xf = O.bf16_to_f64(x_bits)
    y_ref = np.zeros_like(y, dtype=np.float64)
    for t in range(T):
        for k in range(w["K"]):
            y_ref[t, k] = O.expert_forward(experts[gi[t, k]], xf[t:t + 1], w["lora_scale"])[0]
        if w["n_shared"]:
            y_ref[t, w["K"]] = O.expert_forward(shared, xf[t:t + 1], w["lora_scale"])[0]
    rel_y = assert_close_rms(y, y_ref, "expert outputs y")
    if w["n_shared"]:
        g = b["sw"].cpu().numpy()[:T]
        assert np.allclose(g, parts["g"], rtol=1e-5, atol=1e-6)
    # whole block vs the oracle's own routing (tokens without near-ties)
    ok = [t for t in range(T) if t not in near]
    rel_o = assert_bf16_output_close(_bits(b["out"])[ok], o_ref[ok], "block output")
    return dict(rel_y=rel_y, rel_o=rel_o, near=near, b=b)


def test_tiny_block_decode_seed0():
    w = synth.workload(0)
    L, router, experts, shared = _layer(w)
    r = _run_block(w, L, router, experts, shared, synth.tokens(w, 0))
    print("tiny block rel err y %.2e out %.2e" % (r["rel_y"], r["rel_o"]))


def test_tiny_block_decode_several_tokens_and_seeds():
    for seed in (1, 2):
        w = synth.workload(0)
        L, router, experts, shared = _layer(w, seed=seed)
        _run_block(w, L, router, experts, shared, synth.tokens(w, 1, T=7, seed=seed))


def test_block_decode_35b_shape():
    w = synth.workload(1)
    L, router, experts, shared = _layer(w)
    for step in range(3):
        r = _run_block(w, L, router, experts, shared, synth.tokens(w, step))
        print("35b-shaped block step %d rel err y %.2e out %.2e" % (step, r["rel_y"], r["rel_o"]))


def test_decode_no_shared_expert_k8():
    w = synth.workload(2)  # E=128, K=8, no shared expert
    L, router, experts, shared = _layer(w)
    _run_block(w, L, router, experts, shared, synth.tokens(w, 0, T=2))


def test_lora_only_path():
    # base off (scale = bias = 0): the output is the LoRA chain alone, which
    # is ~1% of a normal output and would hide inside the block tolerance
    w = synth.workload(0)
    experts = [synth.expert_tensors(w, 0, e) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"])
    for ex in experts + [shared]:
        for p in ("gate", "up", "down"):
            ex[f"s_{p}"] = np.zeros_like(ex[f"s_{p}"])
            ex[f"b_{p}"] = np.zeros_like(ex[f"b_{p}"])
            ex[f"B_{p}"] = synth.f32_to_bf16_bits(O.bf16_to_f64(ex[f"B_{p}"]) * 50.0)
    L, router, _, _ = _layer(w, experts=experts, shared=shared)
    r = _run_block(w, L, router, experts, shared, synth.tokens(w, 0, T=3))
    assert rms(r["b"]["y"].cpu().numpy()) > 0


def test_lora_zero_b_equals_base():
    w = synth.workload(0)
    experts = [synth.expert_tensors(w, 0, e) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"])
    for ex in experts + [shared]:
        for p in ("gate", "up", "down"):
            ex[f"B_{p}"] = np.zeros_like(ex[f"B_{p}"])
    L, router, _, _ = _layer(w, experts=experts, shared=shared)
    _run_block(w, L, router, experts, shared, synth.tokens(w, 0, T=2))


def test_exact_router_inputs_bit_exact():
    # integer x and one power-of-two scale per row: every partial sum is an
    # exact fp32 value, so the GPU logits must equal the oracle's bit for bit
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    rng = np.random.default_rng(11)
    w = synth.workload(1)
    E, H, K = w["E"], w["H"], w["K"]
    rq = rng.integers(-127, 128, (E, H)).astype(np.int8)
    rs = np.repeat((2.0 ** rng.integers(-12, -6, (E, 1))).astype(np.float32), H // 64, axis=1)
    xi = rng.integers(-4, 5, (3, H)).astype(np.float32)
    xb = synth.f32_to_bf16_bits(xi)
    d = B.dims(H, w["I"], E, K, w["r"], 0)
    T = 3
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws = torch.empty((B.moe_workspace_bytes(d, T, False),), dtype=torch.uint8, device="cuda")
    B.moe_route(d, dev(rq), dev(rs), None, None, dev(xb), T, None, idx, wt, None, logits, None,
                None, None, ws)
    torch.cuda.synchronize()
    ref = O.router_logits(rq, rs, xb)
    assert np.array_equal(logits.cpu().numpy().astype(np.float64), ref)
    for t in range(T):
        assert idx.cpu().numpy()[t].tolist() == O.select_topk(ref[t], K).tolist()


def test_router_ties_and_zero_input():
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    H, E = 64, 8
    codes = [1, 2, 2, 0, 2, -1, 2, 0]
    rq = np.array([[c] * H for c in codes], np.int8)
    rs = np.full((E, 1), 1.0 / 64, np.float32)
    x = np.stack([np.full(H, 0x3F80, np.uint16), np.zeros(H, np.uint16)])
    for K in (1, 3, 8):
        d = B.dims(H, 64, E, K, 0, 0)
        T = 2
        logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        wt = torch.empty((T, K), dtype=torch.float32, device="cuda")
        ws = torch.empty((B.moe_workspace_bytes(d, T, False),), dtype=torch.uint8, device="cuda")
        B.moe_route(d, dev(rq), dev(rs), None, None, dev(x), T, None, idx, wt, None, logits,
                    None, None, None, ws)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
        # token 0: logits (1,2,2,0,2,-1,2,0) -> 1,2,4,6 then 0,3,7 then 5
        assert gi[0].tolist() == [1, 2, 4, 6, 0, 3, 7, 5][:K]
        # token 1: all logits 0 -> ascending indices, equal weights
        assert gi[1].tolist() == list(range(K))
        assert np.allclose(wt.cpu().numpy()[1], 1.0 / K, rtol=1e-6)


def test_empty_batch_is_noop():
    from int4_expert_ffn_int8_amd import binding as B
    w = synth.workload(0)
    L, *_ = _layer(w)
    b = L.buffers(0)
    x = torch.empty((0, w["H"]), dtype=torch.int16, device="cuda")
    L.forward(x, b)
    torch.cuda.synchronize()


def test_run_to_run_bitwise_stable():
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(1)
    L, *_ = _layer(w)
    x = dev(synth.tokens(w, 4))
    b = L.buffers(1)
    outs = []
    for _ in range(3):
        L.forward(x, b)
        torch.cuda.synchronize()
        outs.append((b["y"].cpu().numpy().copy(), b["out"].cpu().numpy().copy()))
    for y, o in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(o, outs[0][1])
