"""GPU: prediction-as-routing.

* moe_block_decode_exec (the fused block with the routed experts given)
  against the oracle's block with the same given experts: executed experts
  bit-exact, weights to fp32 rounding, outputs within the bf16 bound; with
  the router's own top-K as the given experts it reproduces moe_block_decode
  bit for bit; an index outside [0, E) raises the sticky error word.
* A stack in "predict" mode: layers 1 .. L-1 execute the previous step's
  Prerouter predictions.  Pooled (with and without a modeled storage
  latency) and resident stacks agree bit for bit, every layer is checked
  against the oracle's stack layer with the executed experts given, and
  after the first step every lookup of layers 1 .. L-1 is served from a
  slot (the layer waited for its fills).
* The same with routing-feature heads: each head also sees the experts its
  layer executed; its predictions are checked against the oracle's head.
"""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_bf16_output_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


def _layer(w, seed=0, layer=0, norm_topk=1):
    from int4_expert_ffn_int8_amd.layer import MoeLayer
    router = synth.router_tensors(w, layer, seed)
    experts = [synth.expert_tensors(w, layer, e, seed) for e in range(w["E"])]
    shared = synth.expert_tensors(w, layer, w["E"], seed) if w["n_shared"] else None
    L = MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                 router, experts, shared, norm_topk=norm_topk)
    return L, router, experts, shared


def _given(E, K, T, seed):
    """K distinct experts per token, in random order (a stand-in for a
    prediction: unrelated to the router's choice)."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("wid,T,norm", [(0, 1, 1), (0, 2, 1), (0, 2, 0), (1, 1, 1), (2, 1, 1)])
def test_exec_given_experts_match_oracle(wid, T, norm):
    from int4_expert_ffn_int8_amd.layer import dev
    w = dict(synth.workload(wid), norm_topk=norm)
    L, router, experts, shared = _layer(w, norm_topk=norm)
    fb = L.fused_buffers(T)
    for step in range(3):
        print(f"exec wid={wid} T={T} norm={norm} step={step}", flush=True)
        xb = synth.tokens(w, 40 + step, T=T)
        given = _given(w["E"], w["K"], T, seed=100 * wid + step)
        L.decode_fused(dev(xb), fb, exec_idx=dev(given))
        torch.cuda.synchronize()
        o_ref, parts = O.moe_block(w, router, lambda e: experts[e], xb, shared=shared,
                                   return_parts=True, exec_idx=given)
        assert fb["idx"].cpu().numpy().tolist() == given.tolist()
        assert np.allclose(fb["w"].cpu().numpy(), parts["w"], rtol=1e-5, atol=1e-7)
        assert_bf16_output_close(_bits(fb["out"]), o_ref, f"exec block step {step}")
    assert L.fused_error_word(fb) == 0


def test_exec_with_router_topk_is_bit_identical():
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(1)
    L, *_ = _layer(w, seed=2)
    fa, fg = L.fused_buffers(1), L.fused_buffers(1)
    for step in range(3):
        x = dev(synth.tokens(w, 60 + step, seed=2))
        L.decode_fused(x, fa)
        torch.cuda.synchronize()
        L.decode_fused(x, fg, exec_idx=fa["idx"].clone())
        torch.cuda.synchronize()
        assert torch.equal(fg["idx"], fa["idx"])
        assert torch.equal(fg["w"], fa["w"])
        assert torch.equal(fg["out"], fa["out"])


def test_exec_index_out_of_range_sets_error_word():
    # the kernel's own bounds check: the entry is executed as expert 0 and the
    # sticky error word is set; the host sees the flag
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0)
    L, *_ = _layer(w)
    fb = L.fused_buffers(1)
    x = dev(synth.tokens(w, 7))
    L.decode_fused(x, fb, exec_idx=dev(np.array([[1, 0]], np.int32)))
    torch.cuda.synchronize()
    assert L.fused_error_word(fb) == 0
    L.decode_fused(x, fb, exec_idx=dev(np.array([[1, w["E"]]], np.int32)))
    torch.cuda.synchronize()
    assert L.fused_error_word(fb) == 1
    assert fb["idx"].cpu().numpy().tolist() == [[1, 0]]


def _stack_weights(w, layers, seed=0):
    from int4_expert_ffn_int8_amd.layer import dev, pack_experts
    H, I, r, E = w["H"], w["I"], w["r"], w["E"]
    routers = [synth.router_tensors(w, l, seed) for l in range(layers)]
    experts = [[synth.expert_tensors(w, l, e, seed) for e in range(E)] for l in range(layers)]
    shared = [synth.expert_tensors(w, l, E, seed) for l in range(layers)]
    blobs = np.stack([pack_experts(H, I, r, experts[l]) for l in range(layers)])
    shared_dev = dev(np.stack([pack_experts(H, I, r, [shared[l]])[0] for l in range(layers)]))
    return routers, experts, shared, blobs, shared_dev


def test_predict_mode_stack_pool_resident_and_oracle():
    from int4_expert_ffn_int8_amd.layer import MoeStack, dev
    w = synth.workload(0, prerouter_D=64)
    nl, slots, steps, K = 3, 4, 6, w["K"]
    routers, experts, shared, blobs, shared_dev = _stack_weights(w, nl)
    heads = []
    for l in range(nl - 1):
        pt = synth.prerouter_tensors(w, l)
        heads.append((dev(pt["W1"]), dev(pt["W2"])))
    host = torch.from_numpy(blobs).pin_memory()

    def make(**kw):
        return MoeStack(w["H"], w["I"], w["E"], K, w["r"], w["n_shared"], w["lora_scale"],
                        routers, shared_dev, prerouter=heads, pred_k=K, eps=1e-6,
                        exec_mode="predict", **kw)

    resident = make(routed=dev(blobs))
    pooled = make(host_blobs=host, pool_slots=slots)
    delayed = make(host_blobs=host, pool_slots=slots)
    delayed.set_read_delay(20000)  # 20 us per on-demand read and per fill batch
    layer_outs = [torch.empty((1, w["H"]), dtype=torch.int16, device="cuda") for _ in range(nl)]
    prev_pred = None
    base = None
    for step in range(steps):
        print(f"predict stack step {step}", flush=True)
        xb = synth.tokens(w, 300 + step)
        x = dev(xb)
        outs, idx = [], []
        for st in (resident, pooled, delayed):
            o = st.step(x, outs=layer_outs if st is resident else None)
            st.end_step()
            torch.cuda.synchronize()
            outs.append(_bits(o).copy())
            idx.append(st.idx.cpu().numpy().reshape(nl, K).copy())
        np.testing.assert_array_equal(outs[1], outs[0], err_msg=f"pooled step {step}")
        np.testing.assert_array_equal(outs[2], outs[0], err_msg=f"delayed step {step}")
        np.testing.assert_array_equal(idx[1], idx[0])
        np.testing.assert_array_equal(idx[2], idx[0])
        if prev_pred is not None:  # layers >= 1 executed the previous step's predictions
            np.testing.assert_array_equal(idx[0][1:], prev_pred[1:])
        prev_pred = resident.pred.cpu().numpy().reshape(nl, K).copy()
        assert (prev_pred[1:] >= 0).all() and (prev_pred[1:] < w["E"]).all()
        # every layer against the oracle's stack layer, teacher-forced, with
        # the executed experts given where the layer executed a prediction
        h_in = xb
        for l in range(nl):
            given = None if (step == 0 or l == 0) else idx[0][l][None, :]
            _, parts = O.stack_layer(w, routers[l], experts[l].__getitem__, h_in,
                                     shared=shared[l], eps=1e-6, return_parts=True,
                                     exec_idx=given)
            assert parts["idx"].tolist() == [idx[0][l].tolist()], (step, l)
            got = _bits(layer_outs[l]).copy()
            assert_bf16_output_close(got, O.bf16_to_f64(h_in) + parts["o"],
                                     f"predict stack step {step} layer {l}")
            h_in = got
        if step == 0:
            base = pooled.counters.cpu().numpy().copy()
    # after the first step every lookup of layers >= 1 hit a slot
    c = pooled.counters.cpu().numpy() - base
    assert (c[1:, 1] == (steps - 1) * K).all(), c
    np.testing.assert_array_equal(c[1:, 0], c[1:, 1])
    for st in (pooled, delayed):
        st.pool.sync(st.side)
    for st in (resident, pooled, delayed):
        assert st.error_word() == 0


def test_predict_mode_with_feature_heads():
    from int4_expert_ffn_int8_amd.layer import MoeStack, dev
    w = synth.workload(0, prerouter_D=64)
    nl, slots, steps, K, E = 3, 4, 5, w["K"], w["E"]
    routers, experts, shared, blobs, shared_dev = _stack_weights(w, nl)
    ptf = [synth.prerouter_feat_tensors(w, l) for l in range(nl - 1)]
    heads = [(dev(p["W1"]), dev(p["W2"])) for p in ptf]
    host = torch.from_numpy(blobs).pin_memory()

    def make(**kw):
        return MoeStack(w["H"], w["I"], E, K, w["r"], w["n_shared"], w["lora_scale"], routers,
                        shared_dev, prerouter=heads, pred_k=K, eps=1e-6, exec_mode="predict",
                        prerouter_feat=True, **kw)

    resident = make(routed=dev(blobs))
    pooled = make(host_blobs=host, pool_slots=slots)
    layer_outs = [torch.empty((1, w["H"]), dtype=torch.int16, device="cuda") for _ in range(nl)]
    prev_pred = None
    checked = 0
    for step in range(steps):
        print(f"predict+features step {step}", flush=True)
        x = dev(synth.tokens(w, 400 + step))
        o_r = resident.step(x, outs=layer_outs)
        resident.end_step()
        o_p = pooled.step(x)
        pooled.end_step()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(o_p), _bits(o_r), err_msg=f"step {step}")
        idx = resident.idx.cpu().numpy().reshape(nl, K)
        np.testing.assert_array_equal(pooled.idx.cpu().numpy().reshape(nl, K), idx)
        if prev_pred is not None:
            np.testing.assert_array_equal(idx[1:], prev_pred[1:])
        pred = resident.pred.cpu().numpy().reshape(nl, K)
        # each head: oracle on the GPU's layer output and executed experts
        for l in range(nl - 1):
            h = _bits(layer_outs[l])
            _, z_ref = O.prerouter_feat(ptf[l]["W1"], ptf[l]["W2"], h, idx[l][None, :], K)
            order = np.lexsort((np.arange(E), -z_ref[0]))
            margin = z_ref[0, order[K - 1]] - z_ref[0, order[K]]
            if margin > 1e-3 * np.abs(z_ref).max():
                assert pred[l + 1].tolist() == order[:K].tolist(), (step, l)
                checked += 1
        prev_pred = pred.copy()
    assert checked >= (nl - 1) * steps // 2
    pooled.pool.sync(pooled.side)
    assert resident.error_word() == 0 and pooled.error_word() == 0
