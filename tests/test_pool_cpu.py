"""Host LRU planner of the expert pool (moe_lru_*), no GPU needed.

The planner's rules (include/moe.h, expert pool): executed and predicted
experts that are resident become most recent; fill candidates are the
predicted experts that are not resident, then the executed misses, each once,
at most max_fills per layer; a fill takes a free slot, else the least recently
used slot whose expert was neither executed nor predicted in the step (ties:
lowest slot).  A small Python model of those rules is checked step by step
against the library on random sequences, plus hand-sized cases.
"""
import numpy as np
import pytest

from int4_expert_ffn_int8_amd import binding as B


class LruModel:
    def __init__(self, L, E, S):
        self.E, self.S = E, S
        self.slot_expert = [[-1] * S for _ in range(L)]
        self.last = [[0] * S for _ in range(L)]
        self.clock = 0

    def slot_of(self, l, e):
        return self.slot_expert[l].index(e) if e in self.slot_expert[l] else -1

    def plan(self, executed, predicted, max_fills):
        self.clock += 1
        now, fills = self.clock, []
        for l in range(len(self.slot_expert)):
            prot = set(int(e) for e in executed[l])
            for e in executed[l]:
                s = self.slot_of(l, e)
                if s >= 0:
                    self.last[l][s] = now
            want = []
            for e in (predicted[l] if predicted is not None else []):
                if e < 0:
                    continue
                prot.add(int(e))
                s = self.slot_of(l, e)
                if s >= 0:
                    self.last[l][s] = now
                elif e not in want:
                    want.append(int(e))
            for e in executed[l]:
                if self.slot_of(l, e) < 0 and e not in want:
                    want.append(int(e))
            n = 0
            for e in want:
                if 0 <= max_fills <= n:
                    break
                free = [s for s in range(self.S) if self.slot_expert[l][s] < 0]
                if free:
                    v = free[0]
                else:
                    cand = [s for s in range(self.S) if self.slot_expert[l][s] not in prot]
                    if not cand:
                        break
                    v = min(cand, key=lambda s: (self.last[l][s], s))
                old = self.slot_expert[l][v]
                self.slot_expert[l][v] = e
                self.last[l][v] = now
                prot.add(e)
                fills.append((l, e, v, old))
                n += 1
        return fills

    def table(self, l):
        t = np.full(self.E, -1, np.int32)
        for s, e in enumerate(self.slot_expert[l]):
            if e >= 0:
                t[e] = s
        return t


def test_fills_free_slots_in_candidate_order():
    lru = B.MoeLru(1, 16, 4)
    # predicted first (5, 6), then executed misses (1, 2); each once
    fills = lru.plan([[1, 2, 5]], [[5, 6]])
    assert fills == [(0, 5, 0, -1), (0, 6, 1, -1), (0, 1, 2, -1), (0, 2, 3, -1)]
    t = lru.table(0)
    assert t[5] == 0 and t[6] == 1 and t[1] == 2 and t[2] == 3
    assert (t >= 0).sum() == 4
    assert lru.stats() == (4, 0)


def test_lru_victim_and_protection():
    lru = B.MoeLru(1, 16, 3)
    lru.plan([[0, 1, 2]])                 # slots 0,1,2 <- experts 0,1,2 (step 1)
    lru.plan([[1, 1, 1]])                 # expert 1 used at step 2
    lru.plan([[2, 2, 2]])                 # expert 2 used at step 3
    # step 4: expert 7 misses; expert 0 is least recent and not protected
    fills = lru.plan([[7, 2, 2]])
    assert fills == [(0, 7, 0, 0)]
    # step 5: executed {1, 2} and predicted {9} are protected; 7 (step 4) is
    # the only unprotected resident -> it is evicted for 9; the miss on 3
    # finds every remaining slot protected and is skipped
    fills = lru.plan([[1, 2, 3]], [[9]])
    assert fills == [(0, 9, 0, 7)]
    t = lru.table(0)
    assert t[9] == 0 and t[1] == 1 and t[2] == 2 and t[3] == -1 and t[7] == -1


def test_max_fills_caps_each_layer():
    lru = B.MoeLru(2, 32, 8)
    fills = lru.plan([[0, 1, 2, 3], [4, 5, 6, 7]], [[8, 9], [10, 11]], max_fills=3)
    per_layer = [sum(1 for f in fills if f[0] == l) for l in range(2)]
    assert per_layer == [3, 3]
    assert [f[1] for f in fills if f[0] == 0] == [8, 9, 0]
    assert lru.plan([[0, 1, 2, 3], [4, 5, 6, 7]], max_fills=0) == []


def test_rejects_out_of_range_and_keeps_state():
    lru = B.MoeLru(1, 8, 2)
    with pytest.raises(B.MoeError):
        lru.plan([[8]])
    with pytest.raises(B.MoeError):
        lru.plan([[0]], [[9]])
    assert lru.stats() == (0, 0)
    with pytest.raises(B.MoeError):
        B.MoeLru(1, 8, 9)  # more slots than experts


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_model_on_random_sequences(seed):
    rng = np.random.default_rng(seed)
    L, E, S, K, Kp = 3, 24, 6, 4, 3
    lru, model = B.MoeLru(L, E, S), LruModel(L, E, S)
    for step in range(60):
        # skewed picks so that some experts recur (hits and evictions happen)
        ex = np.stack([rng.choice(E, K, replace=False, p=_zipf(E, rng)) for _ in range(L)])
        pr = None
        if step % 3:
            pr = rng.integers(-1, E, size=(L, Kp)).astype(np.int32)
        mf = int(rng.integers(-1, 5))
        got = lru.plan(ex, pr, max_fills=mf)
        want = model.plan(ex, pr, mf)
        assert got == want, f"step {step}"
        for l in range(L):
            t = lru.table(l)
            np.testing.assert_array_equal(t, model.table(l))
            res = t[t >= 0]
            assert len(set(res.tolist())) == len(res) <= S and res.max(initial=0) < S
    f, e = lru.stats()
    assert f > S * L and e > 0  # the sequence exercised evictions


def _zipf(E, rng):
    w = 1.0 / np.arange(1, E + 1) ** 1.1
    return w / w.sum()


def test_prediction_as_routing_sequence_keeps_every_next_route_resident():
    # In prediction-as-routing the experts executed at step s are the
    # predictions of step s - 1, and each plan gets this step's predictions
    # (the next routes).  With K executed + K predicted <= slots, every next
    # route must be resident after the plan, so every lookup of the next step
    # hits, and the executed experts of the step just finished are never
    # evicted by it.
    rng = np.random.default_rng(5)
    L, E, S, K = 3, 32, 8, 3
    lru = B.MoeLru(L, E, S)
    prev = np.stack([rng.choice(E, K, replace=False) for _ in range(L)]).astype(np.int32)
    lru.plan(prev, None)
    for step in range(40):
        nxt = np.stack([rng.choice(E, K, replace=False) for _ in range(L)]).astype(np.int32)
        before = [lru.table(l).copy() for l in range(L)]
        lru.plan(prev, nxt)
        for l in range(L):
            tab = lru.table(l)
            assert all(tab[e] >= 0 for e in nxt[l]), (step, l)
            # executed experts that were resident stay in their slots
            for e in prev[l]:
                if before[l][e] >= 0:
                    assert tab[e] == before[l][e], (step, l, e)
            assert len(set(tab[tab >= 0].tolist())) == int((tab >= 0).sum())  # one slot each
        prev = nxt
