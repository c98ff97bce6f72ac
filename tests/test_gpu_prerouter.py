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
    ws = torch.zeros((B.prerouter_workspace_bytes(D, E, T),), dtype=torch.uint8, device="cuda")
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
    ws = torch.zeros((B.prerouter_workspace_bytes(D, E, T),), dtype=torch.uint8, device="cuda")
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


def _check_against_oracle(W1, W2, h, K, idx, z, prev=None):
    if prev is None:
        pred, z_ref = O.prerouter(W1, W2, h, K)
    else:
        pred, z_ref = O.prerouter_feat(W1, W2, h, prev, K)
    assert_close_rms(z, z_ref, "prerouter logits")
    err = float(np.abs(z - z_ref).max())
    E = z.shape[1]
    for t in range(h.shape[0]):
        # the kernel's selection is the exact top-K of the logits it returns
        assert O.select_topk(z[t], K).tolist() == idx[t].tolist()
        order = np.lexsort((np.arange(E), -z_ref[t]))
        if K < E and z_ref[t, order[K - 1]] - z_ref[t, order[K]] > 2 * err:
            assert order[:K].tolist() == idx[t].tolist()


# (H, D, E, K, T): one row block smaller than D (H 64: 128-row blocks, D 64),
# E not a multiple of 64, E above 256 (the scan top-K, 4 experts per thread),
# D 4096 (256 row blocks, gathered 16 at a time), H 4096 (two slices a lane)
@pytest.mark.parametrize("H,D,E,K,T", [(64, 64, 100, 3, 2), (256, 128, 300, 8, 3),
                                       (2048, 4096, 1000, 16, 1), (4096, 256, 256, 4, 2),
                                       (512, 192, 1, 1, 1)])
def test_prerouter_shapes(H, D, E, K, T):
    w = synth.workload(0, H=H, E=E, prerouter_D=D)
    pr = synth.prerouter_tensors(w, 1)
    h = synth.tokens(w, 2, T=T)
    idx, z = _run(pr["W1"], pr["W2"], h, K)
    _check_against_oracle(pr["W1"], pr["W2"], h, K, idx, z)


def test_prerouter_feat_small_shape_and_bad_ids():
    # H 256, E 120 (H + E a multiple of 8), ids outside [0, E) ignored
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(0, H=256, E=120, prerouter_D=128)
    pr = synth.prerouter_feat_tensors(w, 2)
    T, K, Kp = 3, 5, 6
    h = synth.tokens(w, 1, T=T)
    prev = np.array([[0, 5, 119, 120, -1, 7], [3, 3, 3, 3, 3, 3], [-5, 1000, 60, 61, 62, 63]],
                    np.int32)
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    z = torch.empty((T, 120), dtype=torch.float32, device="cuda")
    ws = torch.zeros((B.prerouter_workspace_bytes(128, 120, T),), dtype=torch.uint8, device="cuda")
    B.prerouter_predict_feat(dev(pr["W1"]), dev(pr["W2"]), 256, 128, 120, K, dev(h), dev(prev), Kp,
                             T, idx, z, ws)
    torch.cuda.synchronize()
    _check_against_oracle(pr["W1"], pr["W2"], h, K, idx.cpu().numpy(), z.cpu().numpy(), prev)


def test_prerouter_graph_replays_match_eager():
    # one workspace reused by several heads inside a HIP graph: every replay's
    # predictions and logits equal the eager ones (stale hand-off words of
    # earlier launches are never taken for this launch's)
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(3)
    D, E, H, K = w["prerouter_D"], w["E"], w["H"], w["K"]
    heads = [synth.prerouter_tensors(w, l) for l in range(3)]
    hs = [dev(synth.tokens(w, s, T=2)) for s in range(3)]
    W = [(dev(p["W1"]), dev(p["W2"])) for p in heads]
    ws = torch.zeros((B.prerouter_workspace_bytes(D, E, 2),), dtype=torch.uint8, device="cuda")
    idx = torch.empty((3, 2, K), dtype=torch.int32, device="cuda")
    z = torch.empty((3, 2, E), dtype=torch.float32, device="cuda")

    def run():
        for l in range(3):
            B.prerouter_predict(W[l][0], W[l][1], H, D, E, K, hs[l], 2, idx[l], z[l], ws)

    run()
    torch.cuda.synchronize()
    idx_e, z_e = idx.clone(), z.clone()
    for l in range(3):
        _check_against_oracle(heads[l]["W1"], heads[l]["W2"], synth.tokens(w, l, T=2), K,
                              idx_e[l].cpu().numpy(), z_e[l].cpu().numpy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        idx.fill_(-7)
        z.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_e), rep
        assert torch.equal(z, z_e), rep
        run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_e), rep
