"""GPU parity of the fused single-launch decode block (moe_block_decode)."""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close, assert_close_rms, check_routing

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _layer(w, seed=0, layer=0):
    from int4_expert_ffn_int8_amd.layer import MoeLayer
    router = synth.router_tensors(w, layer, seed)
    experts = [synth.expert_tensors(w, layer, e, seed) for e in range(w["E"])]
    shared = synth.expert_tensors(w, layer, w["E"], seed) if w["n_shared"] else None
    L = MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                 router, experts, shared)
    return L, router, experts, shared


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("wid,T", [(0, 1), (0, 2), (1, 1), (2, 1)])
def test_fused_block_matches_oracle_over_consecutive_launches(wid, T):
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(wid)
    L, router, experts, shared = _layer(w)
    fb = L.fused_buffers(T)
    for step in range(4):  # same workspace: the counters must reset each launch
        xb = synth.tokens(w, step, T=T)
        L.decode_fused(dev(xb), fb)
        torch.cuda.synchronize()
        o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                                   return_parts=True)
        gi = fb["idx"].cpu().numpy()
        gw = fb["w"].cpu().numpy()
        assert gi.tolist() == parts["idx"].tolist(), (step, gi, parts["idx"])
        assert np.allclose(gw, parts["w"], rtol=1e-5, atol=1e-7)
        assert_bf16_output_close(_bits(fb["out"]), o_ref, f"fused block step {step}")
    assert L.fused_error_word(fb) == 0


def test_fused_agrees_with_three_call_path():
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(1)
    L, router, experts, shared = _layer(w, seed=4)
    fb = L.fused_buffers(1)
    b = L.buffers(1)
    for step in range(3):
        x = dev(synth.tokens(w, step, seed=4))
        L.decode_fused(x, fb)
        L.forward(x, b)
        torch.cuda.synchronize()
        assert np.array_equal(fb["idx"].cpu().numpy(), b["idx"].cpu().numpy())
        a = O.bf16_to_f64(_bits(fb["out"]))
        c = O.bf16_to_f64(_bits(b["out"]))
        assert_close_rms(a, c, "fused vs three-call", rel=2e-3,
                         extra=np.abs(c) * 2.0 ** -7)


def test_fused_stack_layer_mode():
    # x = bf16(RMSNorm(h)), out = bf16(h + MoE(x)): one layer of the 24-layer
    # stack, against the oracle's stack layer
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(2)
    L, router, experts, shared = _layer(w, layer=3)
    fb = L.fused_buffers(1)
    h = synth.tokens(w, 9)
    L.decode_fused(dev(h), fb, flags=B.DECODE_NORM_INPUT | B.DECODE_RESIDUAL, eps=1e-6)
    torch.cuda.synchronize()
    ref_bits, parts = O.stack_layer(w, router, lambda e: experts[e], h, eps=1e-6,
                                    return_parts=True)
    assert fb["idx"].cpu().numpy().tolist() == parts["idx"].tolist()
    ref = O.bf16_to_f64(h) + parts["o"]
    assert_bf16_output_close(_bits(fb["out"]), ref, "fused stack layer")


def test_fused_graph_replays_match_eager():
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0)
    L, router, experts, shared = _layer(w)
    fb = L.fused_buffers(1)
    x = dev(synth.tokens(w, 3))
    L.decode_fused(x, fb)
    torch.cuda.synchronize()
    eager = fb["out"].clone()
    g = torch.cuda.CUDAGraph()
    out2 = torch.empty_like(fb["out"])
    with torch.cuda.graph(g):
        L.decode_fused(x, fb, out=out2)
    for _ in range(4):
        out2.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out2, eager)
        L.decode_fused(x, fb)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(fb["out"], eager)
    assert L.fused_error_word(fb) == 0


@pytest.mark.parametrize("path", ["fused", "three_call"])
def test_large_activations_keep_full_range(path):
    # x * 2^8 drives the SwiGLU outputs h far above the fp16 range (|h| up to
    # ~1e6); the decode paths store h as fp16 with a power-of-two exponent
    # per 32-column block, so the result must still match the oracle
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0)
    L, router, experts, shared = _layer(w)
    xb = synth.tokens(w, 5, T=2)
    x = O.round_bf16(O.bf16_to_f64(xb) * 256.0)  # exact: power-of-two scaling
    ref, parts = O.moe_block(w, router, lambda e: experts[e], x, shared=shared,
                             return_parts=True)
    _, hid = O.expert_forward(shared, O.bf16_to_f64(x), w["lora_scale"], return_hidden=True)
    assert np.abs(hid).max() > 1e5  # far outside the fp16 range
    if path == "fused":
        fb = L.fused_buffers(2)
        out = L.decode_fused(dev(x), fb)
        idx = fb["idx"]
    else:
        b = L.buffers(2)
        out = L.forward(dev(x), b)
        idx = b["idx"]
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == parts["idx"].tolist()
    assert_bf16_output_close(_bits(out), ref, f"large activations ({path})")
