"""GPU: decode stacks and the expert pool.

* 24-layer-stack shapes (E=128, K=8, no shared expert): parity is
  teacher-forced per layer -- each layer's GPU input is fed to the oracle's
  stack layer and the GPU output is compared with the result.
* Expert pool: a stack whose routed experts live in a 4-slot LRU pool with
  Prerouter-driven fills must give bit-identical outputs and routing to the
  same stack with every expert resident, and to a pool that never fills
  (every lookup reads the pinned host copy); the slot/lookup counters must
  add up.
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


def _stack_weights(w, layers, seed=0):
    from int4_expert_ffn_int8_amd.layer import dev, pack_experts
    H, I, r, E = w["H"], w["I"], w["r"], w["E"]
    routers = [synth.router_tensors(w, l, seed) for l in range(layers)]
    experts = [[synth.expert_tensors(w, l, e, seed) for e in range(E)] for l in range(layers)]
    shared = ([synth.expert_tensors(w, l, E, seed) for l in range(layers)]
              if w["n_shared"] else None)
    blobs = np.stack([pack_experts(H, I, r, experts[l]) for l in range(layers)])
    shared_dev = (dev(np.stack([pack_experts(H, I, r, [shared[l]])[0] for l in range(layers)]))
                  if shared else None)
    return routers, experts, shared, blobs, shared_dev


def test_stack24_shapes_teacher_forced_per_layer():
    from int4_expert_ffn_int8_amd.layer import MoeStack, dev
    w = synth.workload(2)
    nl = 3
    routers, experts, shared, blobs, shared_dev = _stack_weights(w, nl)
    st = MoeStack(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                  routers, shared_dev, routed=dev(blobs), eps=w["rms_eps"])
    outs = [torch.empty((1, w["H"]), dtype=torch.int16, device="cuda") for _ in range(nl)]
    for step in range(2):
        print(f"stack24 step {step}", flush=True)
        h = dev(synth.tokens(w, 100 + step))
        cur = h
        for l in range(nl):
            st.layer_forward(l, cur, outs[l])
            cur = outs[l]
        torch.cuda.synchronize()
        h_in = synth.tokens(w, 100 + step)
        for l in range(nl):
            ref_bits, parts = O.stack_layer(w, routers[l], experts[l].__getitem__, h_in,
                                            eps=w["rms_eps"], return_parts=True)
            assert st.idx[l].cpu().numpy().tolist() == parts["idx"].tolist(), (step, l)
            got = _bits(outs[l])
            assert_bf16_output_close(got, O.bf16_to_f64(h_in) + parts["o"],
                                     f"stack24 step {step} layer {l}")
            h_in = got  # teacher forcing: the oracle's next input is the GPU's output
    assert st.error_word() == 0


def _pool_stack(w, routers, shared_dev, blobs, heads, pred_k, **kw):
    from int4_expert_ffn_int8_amd.layer import MoeStack
    return MoeStack(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                    routers, shared_dev, prerouter=heads, pred_k=pred_k, eps=1e-6, **kw)


def test_pool_results_do_not_depend_on_residency():
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0, prerouter_D=64)
    nl, slots, pred_k, steps = 3, 4, 2, 8
    routers, _, _, blobs, shared_dev = _stack_weights(w, nl)
    heads = []
    for l in range(nl - 1):
        pt = synth.prerouter_tensors(w, l)
        heads.append((dev(pt["W1"]), dev(pt["W2"])))
    host = torch.from_numpy(blobs).pin_memory()
    resident = _pool_stack(w, routers, shared_dev, blobs, heads, pred_k, routed=dev(blobs))
    pooled = _pool_stack(w, routers, shared_dev, blobs, heads, pred_k, host_blobs=host,
                         pool_slots=slots)
    never = _pool_stack(w, routers, shared_dev, blobs, heads, pred_k, host_blobs=host,
                        pool_slots=slots, max_fills=0)
    for step in range(steps):
        print(f"pool step {step}", flush=True)
        x = dev(synth.tokens(w, 200 + step))
        outs, idx = [], []
        for st in (resident, pooled, never):
            o = st.step(x)
            st.end_step()
            torch.cuda.synchronize()
            outs.append(_bits(o).copy())
            idx.append(st.idx.cpu().numpy().copy())
        np.testing.assert_array_equal(outs[1], outs[0], err_msg=f"pooled step {step}")
        np.testing.assert_array_equal(outs[2], outs[0], err_msg=f"no-fill step {step}")
        np.testing.assert_array_equal(idx[1], idx[0])
        np.testing.assert_array_equal(idx[2], idx[0])
    pooled.pool.sync(pooled.side)
    lookups = steps * nl * w["K"]
    hits_p, look_p = pooled.hit_counts()
    hits_n, look_n = never.hit_counts()
    assert look_p == lookups and look_n == lookups
    assert hits_n == 0
    assert 0 < hits_p <= lookups
    fills, _ = pooled.pool.stats()
    assert fills > 0 and never.pool.stats() == (0, 0)
    # the device table mirrors the planner's table
    for l in range(nl):
        np.testing.assert_array_equal(pooled.table[l].cpu().numpy(), pooled.pool.table(l))
    for st in (resident, pooled, never):
        assert st.error_word() == 0


@pytest.mark.parametrize("mode,feat", [("router", False), ("predict", False), ("predict", True)])
def test_heads_on_their_own_stream_match_serial_heads(mode, feat):
    # Prerouter heads overlapped with the next layers (own stream, the layer
    # buffers reused two layers on) give the same outputs, routes and
    # predictions, bit for bit, as heads issued between the layers
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0, prerouter_D=64)
    nl, pred_k, steps = 5, w["K"], 4
    routers, _, _, blobs, shared_dev = _stack_weights(w, nl)
    gen = synth.prerouter_feat_tensors if feat else synth.prerouter_tensors
    heads = [(dev(p["W1"]), dev(p["W2"])) for p in (gen(w, l) for l in range(nl - 1))]
    stacks = [_pool_stack(w, routers, shared_dev, blobs, heads, pred_k, routed=dev(blobs),
                          exec_mode=mode, prerouter_feat=feat, overlap_heads=ov)
              for ov in (True, False)]
    assert stacks[0].overlap_heads and not stacks[1].overlap_heads
    for step in range(steps):
        x = dev(synth.tokens(w, 300 + step))
        got = []
        for st in stacks:
            o = st.step(x)
            torch.cuda.synchronize()
            got.append((_bits(o).copy(), st.idx.cpu().numpy().copy(), st.pred.cpu().numpy().copy()))
        for a, b in zip(got[0], got[1]):
            np.testing.assert_array_equal(a, b, err_msg=f"{mode} feat={feat} step {step}")
        assert (got[0][2][1:] >= 0).all()  # every head predicted
    for st in stacks:
        assert st.error_word() == 0
