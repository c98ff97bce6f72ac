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
