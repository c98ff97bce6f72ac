"""GPU parity of the Prerouter head against the CPU oracle."""
import numpy as np
import pytest

import oracle as O
import synth
from parity import assert_close_rms

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _run(W1, W2, h, K):
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    D, H = W1.shape
    E = W2.shape[0]
    T = h.shape[0]
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    z = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = torch.empty((B.prerouter_workspace_bytes(D, E, T),), dtype=torch.uint8, device="cuda")
    B.prerouter_predict(dev(W1), dev(W2), H, D, E, K, dev(h), T, idx, z, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), z.cpu().numpy()


def test_prerouter_35b_shape():
    w = synth.workload(3)
    pr = synth.prerouter_tensors(w, 5)
    h = synth.tokens(w, 3, T=4)
    idx, z = _run(pr["W1"], pr["W2"], h, w["K"])
    pred, z_ref = O.prerouter(pr["W1"], pr["W2"], h, w["K"])
    # ranking parity decomposed like the router's (no weights are used)
    assert_close_rms(z, z_ref, "prerouter logits")
    for t in range(h.shape[0]):
        assert O.select_topk(z[t], w["K"]).tolist() == idx[t].tolist()
    err = float(np.abs(z - z_ref).max())
    for t in range(h.shape[0]):
        order = np.lexsort((np.arange(z_ref.shape[1]), -z_ref[t]))
        if z_ref[t, order[3]] - z_ref[t, order[4]] > 2 * err:
            assert order[:4].tolist() == idx[t].tolist()


def test_prerouter_zero_head_predicts_first_indices():
    w = synth.workload(3)
    pr = synth.prerouter_tensors(w, 0)
    W2 = np.zeros_like(pr["W2"])
    idx, z = _run(pr["W1"], W2, synth.tokens(w, 0, T=2), w["K"])
    assert np.all(z == 0) and idx.tolist() == [[0, 1, 2, 3]] * 2


def test_prerouter_feat_35b_shape():
    # routing-feature input: the one-hot of the experts the layer executed
    # (here 4 per token, one token padded with -1) appended to h
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(3)
    pr = synth.prerouter_feat_tensors(w, 7)
    h = synth.tokens(w, 5, T=4)
    prev = np.array([[3, 17, 200, 255], [0, 1, 2, 3], [128, 64, 32, -1], [255, 254, 9, 100]],
                    np.int32)
    D, E, H, K, T = w["prerouter_D"], w["E"], w["H"], w["K"], 4
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    z = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = torch.empty((B.prerouter_workspace_bytes(D, E, T),), dtype=torch.uint8, device="cuda")
    B.prerouter_predict_feat(dev(pr["W1"]), dev(pr["W2"]), H, D, E, K, dev(h), dev(prev), 4, T,
                             idx, z, ws)
    torch.cuda.synchronize()
    idx, z = idx.cpu().numpy(), z.cpu().numpy()
    pred, z_ref = O.prerouter_feat(pr["W1"], pr["W2"], h, prev, K)
    assert_close_rms(z, z_ref, "prerouter (features) logits")
    err = float(np.abs(z - z_ref).max())
    for t in range(T):
        assert O.select_topk(z[t], K).tolist() == idx[t].tolist()
        order = np.lexsort((np.arange(E), -z_ref[t]))
        if z_ref[t, order[K - 1]] - z_ref[t, order[K]] > 2 * err:
            assert order[:K].tolist() == idx[t].tolist()
    # with an empty executed list the head equals the plain one on W1's h part
    idx0 = torch.empty((T, K), dtype=torch.int32, device="cuda")
    z0 = torch.empty((T, E), dtype=torch.float32, device="cuda")
    B.prerouter_predict_feat(dev(pr["W1"]), dev(pr["W2"]), H, D, E, K, dev(h), None, 0, T,
                             idx0, z0, ws)
    plain = synth.prerouter_tensors(w, 7)
    idx1, z1 = _run(plain["W1"], plain["W2"], h, K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(z0.cpu().numpy(), z1)
    np.testing.assert_array_equal(idx0.cpu().numpy(), idx1)
