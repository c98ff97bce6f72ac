"""GPU: moe_block_decode_noalloc (library-owned scratch, no allocation)
against moe_block_decode on the same inputs, through the C ABI: the same
bits, and the oracle's bound.  Two calls in a row, the second with a smaller
input; error_out reports no timed-out wait."""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _layer(w, seed):
    from int4_expert_ffn_int8_amd.layer import MoeLayer
    router = synth.router_tensors(w, 0, seed)
    experts = [synth.expert_tensors(w, 0, e, seed) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"], seed) if w["n_shared"] else None
    L = MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                 router, experts, shared)
    return L, router, experts, shared


def _noalloc(L, x, T, flags=0, eps=1e-6):
    from int4_expert_ffn_int8_amd import binding as B
    idx = torch.full((T, L.K), -1, dtype=torch.int32, device="cuda")
    wt = torch.zeros((T, L.K), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, L.H), dtype=torch.int16, device="cuda")
    err = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    B.moe_block_decode_noalloc(L.d, L.gate_q, L.gate_s, L.sgate_q, L.sgate_s, L.experts,
                               L.shared_blob, x, T, flags, eps, idx, wt, out, err)
    return idx, wt, out, err


@pytest.mark.parametrize("first,second", [((1, 1, 4, 0), (0, 1, 2, 0)),
                                          ((0, 4, 1, 1), (0, 1, 1, 1))])
def test_noalloc_matches_block_decode_twice(first, second):
    # (workload, T, K, stack flags): the second call has the smaller input
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    for n, (wid, T, K, stack) in enumerate((first, second)):
        print(f"noalloc call {n}: workload {wid} T={T} K={K} stack={stack}", flush=True)
        w = synth.workload(wid, K=K)
        L, router, experts, shared = _layer(w, seed=10 + n)
        xb = synth.tokens(w, 60 + n, T=T, seed=10 + n)
        x = dev(xb)
        flags = (B.DECODE_NORM_INPUT | B.DECODE_RESIDUAL) if stack else 0
        idx, wt, out, err = _noalloc(L, x, T, flags)
        fb = L.fused_buffers(T)
        L.decode_fused(x, fb, flags=flags)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(idx, fb["idx"]) and torch.equal(wt, fb["w"])
        assert torch.equal(out, fb["out"])
        bits = out.cpu().numpy().view(np.uint16)
        if stack:
            ref_bits, parts = O.stack_layer(w, router, lambda e: experts[e], xb, shared=shared,
                                            eps=1e-6, return_parts=True)
            ref = O.bf16_to_f64(xb) + parts["o"]
        else:
            ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                                     return_parts=True)
        assert idx.cpu().numpy().tolist() == parts["idx"].tolist()
        assert_bf16_output_close(bits, ref, f"noalloc call {n}")


def test_noalloc_repeated_calls_in_one_graph_and_eager():
    # the scratch keeps its control words consistent across calls: eager calls
    # and graph replays in any interleaving give the same bits
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0)
    L, *_ = _layer(w, seed=3)
    x = dev(synth.tokens(w, 5, T=2, seed=3))
    idx0, wt0, out0, err0 = _noalloc(L, x, 2)
    torch.cuda.synchronize()
    from int4_expert_ffn_int8_amd import binding as B
    idx = torch.empty_like(idx0)
    wt = torch.empty_like(wt0)
    out = torch.empty_like(out0)
    err = torch.empty_like(err0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_block_decode_noalloc(L.d, L.gate_q, L.gate_s, L.sgate_q, L.sgate_s, L.experts,
                                   L.shared_blob, x, 2, 0, 1e-6, idx, wt, out, err)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out0) and torch.equal(idx, idx0) and int(err.item()) == 0, rep
        _, _, o2, e2 = _noalloc(L, x, 2)
        torch.cuda.synchronize()
        assert torch.equal(o2, out0) and int(e2.item()) == 0
