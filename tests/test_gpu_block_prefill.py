"""GPU parity of moe_block_prefill (route + grouped expert GEMMs + combine in
one call, the expert outputs kept in the workspace as fp16 with one
power-of-two exponent per row, taken from the bound the packer stores in
each blob) against the CPU oracle, and against the three-call path on the
same inputs, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close, check_routing

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


def _check_block(w, L, router, experts, shared, x_bits, bias=None, max_near_ties=0,
                 residual_bits=None, norm=False):
    """Run the three-call path and moe_block_prefill on the same input: the
    routing must agree bit for bit (same kernels), both outputs must match the
    oracle (tokens off a certified near-tie), and the optional norm output
    must be the RMSNorm of the block output."""
    from int4_expert_ffn_int8_amd.layer import dev
    T = x_bits.shape[0]
    x = dev(x_bits)
    bias_d = dev(bias) if bias is not None else None
    res = dev(residual_bits) if residual_bits is not None else None
    b = L.buffers(T, prefill=True)
    L.forward(x, b, bias=bias_d, residual=res)
    pb = L.block_prefill_buffers(T)
    nout = torch.empty((T, w["H"]), dtype=torch.int16, device="cuda") if norm else None
    L.block_prefill(x, pb, bias=bias_d, residual=res, norm_out=nout)
    torch.cuda.synchronize()
    gi = b["idx"].cpu().numpy()
    ref_logits = O.router_logits(router["router_q"], router["router_s"], x_bits, bias)
    near = check_routing(b["logits"].cpu().numpy(), gi, b["w"].cpu().numpy(), ref_logits,
                         w["K"], True, max_near_ties)
    np.testing.assert_array_equal(pb["idx"].cpu().numpy(), gi)
    np.testing.assert_array_equal(pb["w"].cpu().numpy().view(np.uint32),
                                  b["w"].cpu().numpy().view(np.uint32))
    o_ref = O.moe_block(w, router, lambda e: experts[e], x_bits, bias=bias, shared=shared)
    if residual_bits is not None:
        o_ref = o_ref + O.bf16_to_f64(residual_bits)
    ok = [t for t in range(T) if t not in near]
    got = pb["out"].cpu().numpy().view(np.uint16)
    rel = assert_bf16_output_close(got[ok], o_ref[ok], "moe_block_prefill output")
    assert_bf16_output_close(b["out"].cpu().numpy().view(np.uint16)[ok], o_ref[ok],
                             "three-call prefill output")
    if norm:
        ref_n = O.rmsnorm(O.bf16_to_f64(got), 1e-6)
        assert_bf16_output_close(nout.cpu().numpy().view(np.uint16), ref_n,
                                 "moe_block_prefill norm output")
    return dict(rel=rel, near=near, pb=pb, b=b)


def test_block_prefill_tiny_ragged():
    w = synth.workload(0)
    L, router, experts, shared = _layer(w)
    xb = synth.tokens(w, 0, T=37, seed=3)
    _check_block(w, L, router, experts, shared, xb)


def test_block_prefill_residual_and_norm_output():
    # the stack wiring: out = bf16(residual + block(x)), norm_out = RMSNorm(out)
    w = synth.workload(0)
    L, router, experts, shared = _layer(w, seed=2)
    xb = synth.tokens(w, 1, T=130, seed=2)
    rb = synth.tokens(w, 2, T=130, seed=2)
    _check_block(w, L, router, experts, shared, xb, residual_bits=rb, norm=True)


@pytest.mark.parametrize("lam", [0.5, 2.0, -1.0])
def test_block_prefill_lora_scale(lam):
    # the packed bound combines the base and LoRA parts with |lambda|
    w = synth.workload(0, lora_scale=lam)
    L, router, experts, shared = _layer(w, seed=4)
    xb = synth.tokens(w, 3, T=100, seed=4)
    _check_block(w, L, router, experts, shared, xb)


def test_block_prefill_large_activations():
    # inputs scaled far beyond N(0, 1): the per-row exponents follow, nothing
    # overflows the fp16 outputs
    w = synth.workload(0)
    L, router, experts, shared = _layer(w, seed=6)
    xf = O.bf16_to_f64(synth.tokens(w, 4, T=70, seed=6)) * 3.0e4
    xb = O.round_bf16(xf)
    _check_block(w, L, router, experts, shared, xb)


def test_block_prefill_3300_tokens_zipf():
    w = synth.workload(4)
    L, router, experts, shared = _layer(w)
    xb = synth.tokens(w, 0)
    r = _check_block(w, L, router, experts, shared, xb, bias=synth.zipf_bias(w), max_near_ties=3)
    print("block prefill 3300: rel err %.2e, near ties %s" % (r["rel"], r["near"]))


def test_block_prefill_8b_shape_3300_tokens_zipf():
    w = synth.workload(5)
    L, router, experts, shared = _layer(w)
    xb = synth.tokens(w, 0)
    r = _check_block(w, L, router, experts, shared, xb, bias=synth.zipf_bias(w), max_near_ties=3)
    print("block prefill 8B-shaped 3300: rel err %.2e, near ties %s" % (r["rel"], r["near"]))


def test_block_prefill_repeatable_and_graph_replays():
    # fixed-order reductions throughout: two eager calls give the same bits,
    # and graph replays with eager calls between them give those bits too
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(4)
    L, router, experts, shared = _layer(w, seed=5)
    T = 700
    x = dev(synth.tokens(w, 9, T=T, seed=5))
    bias = dev(synth.zipf_bias(w))
    pb = L.block_prefill_buffers(T)
    L.block_prefill(x, pb, bias=bias)
    torch.cuda.synchronize()
    eager = {k: pb[k].clone() for k in ("idx", "w", "out")}
    L.block_prefill(x, pb, bias=bias)
    torch.cuda.synchronize()
    for k in eager:
        assert torch.equal(pb[k], eager[k]), ("repeat", k)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.block_prefill(x, pb, bias=bias)
    for rep in range(3):
        for k in eager:
            pb[k].zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(pb[k], eager[k]), (rep, k)
        L.block_prefill(x, pb, bias=bias)
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(pb[k], eager[k]), ("eager", rep, k)


def test_block_prefill_empty_batch_and_small_workspace():
    from int4_expert_ffn_int8_amd import binding as B
    w = synth.workload(0)
    L, router, experts, shared = _layer(w)
    pb = L.block_prefill_buffers(0)
    L.block_prefill(torch.empty((0, w["H"]), dtype=torch.int16, device="cuda"), pb)  # no-op
    T = 8
    pb = L.block_prefill_buffers(T)
    pb["ws"] = pb["ws"][:-256]
    with pytest.raises(B.MoeError):
        L.block_prefill(torch.zeros((T, w["H"]), dtype=torch.int16, device="cuda"), pb)


def test_block_prefill_through_pool_matches_resident():
    # moe_block_prefill with the routed experts behind a slot pool over a
    # pinned host copy: cold (every expert read from the host copy, the down
    # GEMM's output bound included) and warm give the resident bits
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev, pack_experts
    w = synth.workload(0)
    L, router, experts, shared = _layer(w, seed=21)
    T = 300
    xb = synth.tokens(w, 4, T=T, seed=21)
    x = dev(xb)
    pb0 = L.block_prefill_buffers(T)
    L.block_prefill(x, pb0)
    torch.cuda.synchronize()
    out_res = pb0["out"].cpu().numpy().copy()
    o_ref = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared)
    touched = np.unique(pb0["idx"].cpu().numpy()).astype(np.int32)
    E, nb = w["E"], B.moe_expert_blob_bytes(w["H"], w["I"], w["r"])
    host = torch.from_numpy(pack_experts(w["H"], w["I"], w["r"], experts)).pin_memory()
    slots = torch.empty((1, 8, nb), dtype=torch.uint8, device="cuda")
    table = torch.empty((1, E), dtype=torch.int32, device="cuda")
    counters = torch.zeros(2, dtype=torch.int64, device="cuda")
    pool = B.MoePool(1, E, 8, nb, slots, table, host)
    try:
        ex = pool.layer(0, counters)
        for phase in ("cold", "warm"):
            if phase == "warm":
                pool.update(touched.reshape(1, -1))
                pool.wait_layer(0)
            pb = L.block_prefill_buffers(T)
            L.block_prefill(x, pb, routed=ex)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(pb["out"].cpu().numpy(), out_res, err_msg=phase)
        assert_bf16_output_close(out_res.view(np.uint16), o_ref, "pooled block prefill output")
    finally:
        pool.close()
