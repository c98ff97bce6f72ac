"""GPU parity of the prefill path: MFMA router GEMM, pair grouping
(histogram / scan / stable scatter) and the grouped int4 MFMA GEMMs with the
LoRA chunk, against the CPU oracle through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close, assert_close_rms, check_routing

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _layer(w, seed=0, experts=None, shared=None, router=None):
    from int4_expert_ffn_int8_amd.layer import MoeLayer
    router = router or synth.router_tensors(w, 0, seed)
    if experts is None:
        experts = [synth.expert_tensors(w, 0, e, seed) for e in range(w["E"])]
    if shared is None and w["n_shared"]:
        shared = synth.expert_tensors(w, 0, w["E"], seed)
    L = MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                 router, experts, shared)
    return L, router, experts, shared


def _oracle_y(w, experts, shared, x_bits, idx):
    """Oracle expert outputs for the given selection, grouped per expert."""
    T, K = idx.shape
    x = O.bf16_to_f64(x_bits)
    y = np.zeros((T, K + w["n_shared"], w["H"]))
    for e in np.unique(idx):
        rows, ks = np.nonzero(idx == e)
        y[rows, ks] = O.expert_forward(experts[int(e)], x[rows], w["lora_scale"])
    if w["n_shared"]:
        y[:, K] = O.expert_forward(shared, x, w["lora_scale"])
    return y


def _run_prefill(w, L, router, experts, shared, x_bits, bias=None, max_near_ties=0,
                 check_block=True):
    from int4_expert_ffn_int8_amd.layer import dev
    T = x_bits.shape[0]
    b = L.buffers(T, prefill=True)
    L.forward(dev(x_bits), b, bias=dev(bias) if bias is not None else None)
    torch.cuda.synchronize()
    ref_logits = O.router_logits(router["router_q"], router["router_s"], x_bits, bias)
    gi = b["idx"].cpu().numpy()
    near = check_routing(b["logits"].cpu().numpy(), gi, b["w"].cpu().numpy(), ref_logits,
                         w["K"], True, max_near_ties)
    # grouping of the GPU's own selection: bit-exact
    counts, offsets, perm = O.group_pairs(gi, w["E"])
    assert b["counts"].cpu().numpy().tolist() == counts.tolist()
    assert b["offsets"].cpu().numpy().tolist() == offsets.tolist()
    assert b["perm"].cpu().numpy()[:T * w["K"]].tolist() == perm.tolist()
    # expert outputs for the GPU's selection
    y = b["y"].cpu().numpy()
    y_ref = _oracle_y(w, experts, shared, x_bits, gi)
    rel = assert_close_rms(y, y_ref, "prefill expert outputs y")
    if check_block:
        o_ref, parts = O.moe_block(w, router, lambda e: experts[e], x_bits, bias=bias,
                                   shared=shared, return_parts=True)
        ok = [t for t in range(T) if t not in near]
        assert_bf16_output_close(b["out"].cpu().numpy().view(np.uint16)[ok], o_ref[ok],
                                 "prefill block output")
    return dict(b=b, rel=rel, near=near, idx=gi)


def test_prefill_tiny_ragged():
    # T*K = 74 pairs over 16 experts: many groups, ragged tiles, shared group
    w = synth.workload(0)
    L, router, experts, shared = _layer(w)
    _run_prefill(w, L, router, experts, shared, synth.tokens(w, 0, T=37))


def test_prefill_multi_tile_groups_router_gemm():
    # T >= 64 switches the router to the MFMA GEMM; 600 tokens over 16
    # experts give groups spanning several 128-row tiles plus tails
    w = synth.workload(0)
    L, router, experts, shared = _layer(w, seed=3)
    r = _run_prefill(w, L, router, experts, shared, synth.tokens(w, 2, T=600, seed=3),
                     max_near_ties=2)
    print("tiny prefill T=600 rel err %.2e, near ties %s" % (r["rel"], r["near"]))


def test_prefill_equals_decode_path():
    # path invariance: the grouped GEMM path and the GEMV path agree (both
    # are also held to the oracle)
    w = synth.workload(0)
    L, router, experts, shared = _layer(w, seed=5)
    from int4_expert_ffn_int8_amd.layer import dev
    xb = synth.tokens(w, 1, T=12, seed=5)
    r = _run_prefill(w, L, router, experts, shared, xb)
    bd = L.buffers(12, prefill=False)
    L.forward(dev(xb), bd)
    torch.cuda.synchronize()
    assert np.array_equal(bd["idx"].cpu().numpy(), r["idx"])
    y_ref = _oracle_y(w, experts, shared, xb, r["idx"])
    assert_close_rms(bd["y"].cpu().numpy(), y_ref, "decode y")
    yp, yd = r["b"]["y"].cpu().numpy(), bd["y"].cpu().numpy()
    assert_close_rms(yp, yd, "prefill vs decode y")


@pytest.mark.parametrize("H,I", [(256, 64), (64, 128)])
def test_prefill_k_not_multiple_of_128(H, I):
    # the expert GEMMs take K in chunks of 128: a last chunk of 64 is padded
    # with zero activations and zero weights
    w = synth.workload(0, H=H, I=I)
    L, router, experts, shared = _layer(w, seed=11)
    _run_prefill(w, L, router, experts, shared, synth.tokens(w, 3, T=90, seed=11), max_near_ties=2)


def test_prefill_no_shared_k8_no_lora():
    w = synth.workload(2, r=0)
    L, router, experts, shared = _layer(w)
    _run_prefill(w, L, router, experts, shared, synth.tokens(w, 0, T=150), max_near_ties=2)


@pytest.mark.parametrize("T", [40, 700])
def test_prefill_k6_e200_pairs_straddle_histogram_chunks(T):
    # K = 6 does not divide the 1024-pair histogram chunks, so at T = 700 the
    # pairs of token 170 fall in two chunks; E = 200 is not a multiple of 64.
    # T = 40 takes the GEMV router, T = 700 the MFMA router GEMM.
    w = synth.workload(0, H=256, E=200, K=6, I=128, r=4, n_shared=1)
    L, router, experts, shared = _layer(w, seed=11)
    _run_prefill(w, L, router, experts, shared, synth.tokens(w, 3, T=T, seed=11),
                 max_near_ties=2)


def test_prefill_fewer_pairs_than_experts():
    w = synth.workload(1)
    L, router, experts, shared = _layer(w)
    _run_prefill(w, L, router, experts, shared, synth.tokens(w, 7, T=5))


def test_prefill_lora_only():
    w = synth.workload(0)
    experts = [synth.expert_tensors(w, 0, e) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"])
    for ex in experts + [shared]:
        for p in ("gate", "up", "down"):
            ex[f"s_{p}"] = np.zeros_like(ex[f"s_{p}"])
            ex[f"b_{p}"] = np.zeros_like(ex[f"b_{p}"])
            ex[f"B_{p}"] = synth.f32_to_bf16_bits(O.bf16_to_f64(ex[f"B_{p}"]) * 50.0)
    L, router, _, _ = _layer(w, experts=experts, shared=shared)
    _run_prefill(w, L, router, experts, shared, synth.tokens(w, 0, T=70), max_near_ties=1)


def test_router_gemm_exact_inputs_bit_exact():
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    rng = np.random.default_rng(12)
    w = synth.workload(1)
    E, H, K, T = w["E"], w["H"], w["K"], 130
    rq = rng.integers(-127, 128, (E, H)).astype(np.int8)
    rs = np.repeat((2.0 ** rng.integers(-12, -6, (E, 1))).astype(np.float32), H // 64, axis=1)
    sq = rng.integers(-127, 128, (H,)).astype(np.int8)
    ss = np.full(H // 64, 2.0 ** -9, np.float32)
    xb = synth.f32_to_bf16_bits(rng.integers(-4, 5, (T, H)).astype(np.float32))
    d = B.dims(H, w["I"], E, K, w["r"], 1)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, K), dtype=torch.float32, device="cuda")
    sw = torch.empty((T,), dtype=torch.float32, device="cuda")
    ws = torch.empty((B.moe_workspace_bytes(d, T, False),), dtype=torch.uint8, device="cuda")
    B.moe_route(d, dev(rq), dev(rs), dev(sq), dev(ss), dev(xb), T, None, idx, wt, sw, logits,
                None, None, None, ws)
    torch.cuda.synchronize()
    ref = O.router_logits(rq, rs, xb)
    assert np.array_equal(logits.cpu().numpy().astype(np.float64), ref)
    g_ref = O.shared_gate(sq.reshape(1, -1), ss.reshape(1, -1), xb)
    assert np.allclose(sw.cpu().numpy(), g_ref, rtol=1e-6)


def test_prefill_3300_tokens_zipf():
    # the skewed prefill workload at full size: 3300 tokens, 256 experts,
    # top-4, Zipf(1.1) rank bias on the router logits
    w = synth.workload(4)
    L, router, experts, shared = _layer(w)
    xb = synth.tokens(w, 0)
    bias = synth.zipf_bias(w)
    r = _run_prefill(w, L, router, experts, shared, xb, bias=bias, max_near_ties=3)
    counts = r["b"]["counts"].cpu().numpy()
    print("prefill 3300: rel err %.2e, experts used %d, largest group %d, near ties %s"
          % (r["rel"], (counts > 0).sum(), counts.max(), r["near"]))


def test_prefill_3300_tokens_repeatable_bits():
    # every reduction on the prefill path has a fixed order (K-split partials
    # summed in split order, grouping counts by integer atomics, stable
    # scatter), so two calls on the same input give the same bits
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(4)
    L, router, experts, shared = _layer(w)
    x = dev(synth.tokens(w, 0))
    bias = dev(synth.zipf_bias(w))
    b = L.buffers(w["T"], prefill=True)
    runs = []
    for _ in range(2):
        L.forward(x, b, bias=bias)
        torch.cuda.synchronize()
        runs.append({k: b[k].cpu().numpy().copy() for k in ("logits", "idx", "w", "perm", "y", "out")})
    for k in runs[0]:
        np.testing.assert_array_equal(runs[1][k].view(np.uint8), runs[0][k].view(np.uint8), err_msg=k)


def test_prefill_graph_replays_match_eager():
    # the whole prefill block captured in a HIP graph: nothing on the path is
    # cleared with a memset node (the grouping histogram is zeroed by the
    # router kernel), so every replay, with eager calls in between, gives the
    # eager bits
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(4)  # 35B-shaped layer with the Zipf(1.1) router bias
    L, router, experts, shared = _layer(w, seed=5)
    T = 700  # MFMA router GEMM, several histogram chunks
    x = dev(synth.tokens(w, 9, T=T, seed=5))
    bias = dev(synth.zipf_bias(w))
    b = L.buffers(T, prefill=True)
    L.forward(x, b, bias=bias)
    torch.cuda.synchronize()
    eager = {k: b[k].clone() for k in ("idx", "perm", "y", "out")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(x, b, bias=bias)
    for rep in range(3):
        for k in eager:
            b[k].zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(b[k], eager[k]), (rep, k)
        L.forward(x, b, bias=bias)  # eager work between replays
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(b[k], eager[k]), ("eager", rep, k)


def test_prefill_8b_shape_3300_tokens_zipf():
    # the second prefill workload: 8B-shaped layer (128 experts, top-8, no
    # shared expert), 3300 tokens, Zipf(1.1) rank bias; group sizes differ
    # from the 35B-shaped case (twice the pairs over half the experts)
    w = synth.workload(5)
    L, router, experts, shared = _layer(w)
    assert shared is None
    xb = synth.tokens(w, 0)
    bias = synth.zipf_bias(w)
    r = _run_prefill(w, L, router, experts, shared, xb, bias=bias, max_near_ties=3)
    counts = r["b"]["counts"].cpu().numpy()
    assert counts.sum() == w["T"] * w["K"]
    print("prefill 8B-shaped 3300: rel err %.2e, experts used %d, largest group %d, near ties %s"
          % (r["rel"], (counts > 0).sum(), counts.max(), r["near"]))


def test_prefill_through_pool_cold_and_warm_match_resident():
    # prefill with the routed experts behind an HBM slot pool over a pinned
    # host master copy: cold (no expert resident: the GEMMs read the host
    # copy) and warm (the touched experts filled into slots) give the same
    # bits as the all-resident layer, match the oracle, and the lookups are
    # counted
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev, pack_experts
    w = synth.workload(0)
    L, router, experts, shared = _layer(w, seed=21)
    xb = synth.tokens(w, 4, T=300, seed=21)
    x = dev(xb)
    b0 = L.buffers(300, prefill=True)
    L.forward(x, b0)
    torch.cuda.synchronize()
    y_res = b0["y"].cpu().numpy().copy()
    out_res = b0["out"].cpu().numpy().copy()
    o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                               return_parts=True)
    counts = b0["counts"].cpu().numpy()
    touched = np.nonzero(counts)[0].astype(np.int32)

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
                n = pool.update(touched.reshape(1, -1))
                assert n == min(len(touched), 8)
                pool.wait_layer(0)
            counters.zero_()
            b = L.buffers(300, prefill=True)
            L.forward(x, b, routed=ex)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(b["y"].cpu().numpy(), y_res, err_msg=phase)
            np.testing.assert_array_equal(b["out"].cpu().numpy(), out_res, err_msg=phase)
            # and against the oracle on the same inputs
            gi = b["idx"].cpu().numpy()
            near = check_routing(b["logits"].cpu().numpy(), gi, b["w"].cpu().numpy(),
                                 parts["logits"], w["K"], True, max_near_ties=2)
            assert_close_rms(b["y"].cpu().numpy(), _oracle_y(w, experts, shared, xb, gi),
                             f"pooled prefill y ({phase})")
            ok = [t for t in range(300) if t not in near]
            assert_bf16_output_close(b["out"].cpu().numpy().view(np.uint16)[ok], o_ref[ok],
                                     f"pooled prefill output ({phase})")
            hits, lookups = (int(v) for v in counters.cpu().numpy())
            assert lookups == len(touched)
            assert hits == (0 if phase == "cold" else min(len(touched), 8))
    finally:
        pool.close()
