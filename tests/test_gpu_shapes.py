"""GPU parity at the edges of the supported shapes, against the oracle:
every fused-decode geometry family (including the largest pair count and the
widest intermediate, whose down rows take two h slices per lane), the widest
three-call decode GEMVs (H or I = 4096) and prefill GEMMs with the longest K."""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close, assert_close_rms, check_routing

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


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


def _clear_margin(logits, K):
    """Tokens whose oracle K-th / (K+1)-th logit gap exceeds 1e-3 of the
    logits' RMS (fp32 logits cannot reorder those)."""
    ok = []
    scale = float(np.sqrt(np.mean(logits ** 2)))
    for t in range(logits.shape[0]):
        s = np.sort(logits[t])[::-1]
        if K == logits.shape[1] or s[K - 1] - s[K] > 1e-3 * scale:
            ok.append(t)
    return ok


# H, I, r, E, K, n_shared, T with T (K + n_shared) <= 8 pairs
FUSED = [
    (512, 1024, 16, 16, 3, 1, 2),    # 8 pairs, I 1024
    (1024, 2048, 16, 16, 7, 1, 1),   # 8 pairs, I 2048: two h slices per down lane
    (2048, 2048, 16, 12, 3, 1, 2),   # the largest H and I together
    (256, 256, 8, 8, 2, 0, 4),       # four tokens, no shared expert
    (2048, 128, 4, 16, 4, 1, 1),     # the narrowest I under the widest H (r <= I / 32)
    (512, 512, 16, 16, 1, 1, 3),     # K = 1 with a shared expert, three tokens
    (1024, 512, 16, 32, 1, 0, 4),    # K = 1 alone, four tokens
]


@pytest.mark.parametrize("H,I,r,E,K,S,T", FUSED)
def test_fused_shapes(H, I, r, E, K, S, T):
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0, H=H, I=I, r=r, E=E, K=K, n_shared=S, lora_scale=0.5)
    L, router, experts, shared = _layer(w, seed=11)
    fb = L.fused_buffers(T)
    for step in range(2):
        xb = synth.tokens(w, 40 + step, T=T)
        L.decode_fused(dev(xb), fb)
        torch.cuda.synchronize()
        o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                                   return_parts=True)
        ok = _clear_margin(parts["logits"], K)
        assert len(ok) == T, "seeded inputs hold no near-ties"
        assert fb["idx"].cpu().numpy().tolist() == parts["idx"].tolist()
        assert np.allclose(fb["w"].cpu().numpy(), parts["w"], rtol=1e-5, atol=1e-7)
        assert_bf16_output_close(_bits(fb["out"]), o_ref, f"fused {H}x{I} step {step}")
    assert L.fused_error_word(fb) == 0


def _oracle_y(w, experts, shared, x_bits, idx):
    T, K = idx.shape
    x = O.bf16_to_f64(x_bits)
    y = np.zeros((T, K + w["n_shared"], w["H"]))
    for e in np.unique(idx):
        rows, ks = np.nonzero(idx == e)
        y[rows, ks] = O.expert_forward(experts[int(e)], x[rows], w["lora_scale"])
    if w["n_shared"]:
        y[:, K] = O.expert_forward(shared, x, w["lora_scale"])
    return y


# H, I, r, E, K, n_shared, T: three-call path (decode GEMVs for small T,
# grouped prefill GEMMs for large T)
THREE_CALL = [
    (4096, 1024, 16, 8, 2, 1, 2),     # GEMV: two 2048-column slices per lane over H
    (1024, 4096, 16, 8, 2, 1, 1),     # GEMV: the widest down row
    (4096, 512, 16, 8, 2, 1, 300),    # prefill: gate/up K = 4096 (64 chunks)
    (512, 4096, 8, 8, 3, 0, 200),     # prefill: down K = 4096, no shared expert
]


@pytest.mark.parametrize("H,I,r,E,K,S,T", THREE_CALL)
def test_three_call_wide_shapes(H, I, r, E, K, S, T):
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0, H=H, I=I, r=r, E=E, K=K, n_shared=S, lora_scale=2.0)
    L, router, experts, shared = _layer(w, seed=12)
    xb = synth.tokens(w, 7, T=T)
    prefill = T > 16
    b = L.buffers(T, prefill=prefill)
    L.forward(dev(xb), b)
    torch.cuda.synchronize()
    ref_logits = O.router_logits(router["router_q"], router["router_s"], xb)
    gi = b["idx"].cpu().numpy()
    near = check_routing(b["logits"].cpu().numpy(), gi, b["w"].cpu().numpy(), ref_logits, K)
    assert not near
    if prefill:  # the grouping of the GPU's own selection, bit-exact
        counts, offsets, perm = O.group_pairs(gi, E)
        assert b["counts"].cpu().numpy().tolist() == counts.tolist()
        assert b["offsets"].cpu().numpy().tolist() == offsets.tolist()
        assert b["perm"].cpu().numpy()[:T * K].tolist() == perm.tolist()
    y_ref = _oracle_y(w, experts, shared, xb, gi)
    assert_close_rms(b["y"].cpu().numpy(), y_ref, f"expert outputs {H}x{I} T={T}")
    o_ref = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared)
    assert_bf16_output_close(_bits(b["out"]), o_ref, f"block {H}x{I} T={T}")
