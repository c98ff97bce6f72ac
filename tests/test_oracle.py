"""Pins for the CPU oracle: hand examples, closed forms, invariants and a
brute-force loop formulation on tiny inputs.  CPU only.

Each pin targets a mistake the oracle could plausibly contain: a dropped LoRA
term, the scale group taken along the wrong axis, a transposed LoRA factor, a
wrong tie-break, a softmax over the wrong set, an off-by-one in the grouping.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "hand_examples.json")))


def bfv(bits):
    """bf16 bits -> Python float, through struct (independent of numpy)."""
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def f2bits(v):
    """Exact bf16 value -> bits (value must be representable)."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    assert u & 0xFFFF == 0, v
    return u >> 16


def const_expert(H, I, r, code, scale, bias, A=None, B=None):
    sb, bb = f2bits(scale), f2bits(bias)
    ex = {}
    for p, (o, i) in {"gate": (I, H), "up": (I, H), "down": (H, I)}.items():
        ex[f"q_{p}"] = np.full((o, i), code, np.uint8)
        ex[f"s_{p}"] = np.full((o, i // 64), sb, np.uint16)
        ex[f"b_{p}"] = np.full((o, i // 64), bb, np.uint16)
        a = (A or {}).get(p, 0.0)
        b = (B or {}).get(p, 0.0)
        ex[f"A_{p}"] = np.full((r, i), f2bits(a), np.uint16)
        ex[f"B_{p}"] = np.full((o, r), f2bits(b), np.uint16)
    return ex


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def test_bf16_rounding_ties_and_values():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8),
                     1 + 2 ** -8 + 2 ** -30, 0.0, 65280.0, 3.0e38])
    got = O.round_bf16(vals)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa -> 1.0
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even -> 1+2^-6
    # just above a tie rounds up
    want = [0x3F80, 0x3F80, 0x3F82, 0xBF80, 0x3F81, 0x0000, 0x477F, 0x7F62]
    assert [int(g) for g in got] == want


def test_bf16_rounding_matches_generator_on_float32_values():
    # two independent implementations (numpy float64 bit cut vs the input
    # generator's uint32 rounding) must agree on float32-representable input
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000)).astype(np.float32)
    assert np.array_equal(O.round_bf16(v.astype(np.float64)), synth.f32_to_bf16_bits(v))


def test_bf16_widen_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    got = O.bf16_to_f64(bits)
    want = np.array([bfv(b) for b in bits])
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# dequantisation
# --------------------------------------------------------------------------
def test_int4_dequant_closed_forms_and_group_axis():
    out, n_in = 3, 192
    q = np.zeros((out, n_in), np.uint8)
    q[:, 64:128] = 15
    s = np.array([[f2bits(0.5), f2bits(0.25), f2bits(2.0)]] * out, np.uint16)
    b = np.array([[f2bits(-1.0), f2bits(0.125), f2bits(3.0)]] * out, np.uint16)
    W = O.dequant_int4_affine(q, s, b)
    # group 0: q=0 -> b ; group 1: q=15 -> 15 s + b ; group 2: q=0 -> b
    assert np.all(W[:, :64] == -1.0)
    assert np.all(W[:, 64:128] == 15 * 0.25 + 0.125)
    assert np.all(W[:, 128:] == 3.0)


def test_int8_dequant_group_axis():
    q = np.tile(np.arange(-64, 64, dtype=np.int8), (2, 1))  # [2,128]
    s = np.array([[0.5, 2.0], [1.0, 0.25]], np.float32)
    W = O.dequant_int8_sym(q, s)
    assert np.array_equal(W[0, :64], 0.5 * np.arange(-64, 0))
    assert np.array_equal(W[0, 64:], 2.0 * np.arange(0, 64))
    assert np.array_equal(W[1, 64:], 0.25 * np.arange(0, 64))


def test_int4_quantiser_round_trip_half_step():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((64, 512)) * 0.05
    w[3, :64] = 0.0  # a constant group (s may be 0)
    q, s_bits, b_bits = O.quantize_int4_affine(w)
    assert q.max() <= 15
    err = np.abs(O.dequant_int4_affine(q, s_bits, b_bits) - w)
    s = O.bf16_to_f64(s_bits)[:, np.arange(512) // 64]
    assert np.all(err <= s / 2 + 1e-12)


def test_int8_quantiser_round_trip_half_step():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((8, 256)) * 0.02
    q, s = O.quantize_int8_sym(w)
    assert np.abs(q.astype(int)).max() <= 127
    err = np.abs(O.dequant_int8_sym(q, s) - w)
    s64 = s.astype(np.float64)[:, np.arange(256) // 64]
    assert np.all(err <= s64 / 2 * (1 + 1e-6))


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def _router_from_codes(codes, scale, H):
    E = len(codes)
    rq = np.array([[c] * H for c in codes], np.int8)
    rs = np.full((E, H // 64), scale, np.float32)
    return rq, rs


def test_router_hand_example_ties():
    g = GOLD["router_ties"]
    rq, rs = _router_from_codes(g["codes"], g["scale"], g["H"])
    x = np.full((1, g["H"]), f2bits(g["x"]), np.uint16)
    l = O.router_logits(rq, rs, x)[0]
    assert list(l) == g["logits"]
    for K in (1, 2, 4):
        sel = O.select_topk(l, K)
        assert list(sel) == g[f"K{K}_idx"]
    assert list(O.topk_weights(l, O.select_topk(l, 2))) == g["K2_w"]
    assert list(O.topk_weights(l, O.select_topk(l, 1))) == g["K1_w"]


def test_router_bias_moves_selection_and_weights():
    # the skewed prefill's per-expert bias enters before both the selection
    # and the softmax: dropping it, or adding it to only one of the two,
    # changes the experts or their weights
    g = GOLD["router_bias"]
    rq, rs = _router_from_codes(g["codes"], g["scale"], g["H"])
    x = np.full((1, g["H"]), f2bits(g["x"]), np.uint16)
    bias = np.array(g["bias"], np.float32)
    l = O.router_logits(rq, rs, x, bias)[0]
    assert list(l) == g["logits"]
    sel = O.select_topk(l, 2)
    assert list(sel) == g["K2_idx"]
    assert np.allclose(O.topk_weights(l, sel), g["K2_w"], rtol=1e-15, atol=0)
    assert np.allclose(O.topk_weights(l, sel, norm_topk=False), g["K2_w_full_softmax"],
                       rtol=1e-15, atol=0)
    # the same through the whole block: two constant experts with different
    # outputs, so the weights show in the block output
    H = g["H"]
    experts = [const_expert(H, 64, 1, 1, 0.015625, 0.0),       # y = sigmoid(1)
               const_expert(H, 64, 1, 1, 0.015625, 0.0,
                            A={"gate": 0.015625}, B={"gate": 1.0}),  # y = 2 sigmoid(2)
               const_expert(H, 64, 1, 0, 0.0, 0.0),
               const_expert(H, 64, 1, 0, 0.0, 0.0)]
    router = {"router_q": rq, "router_s": rs}
    w = dict(H=H, E=4, K=2, lora_scale=1.0)
    o, parts = O.moe_block(w, router, lambda e: experts[e], x, bias=bias, return_parts=True)
    assert parts["idx"].tolist() == [g["K2_idx"]]
    y0 = GOLD["expert_base_only"]["y"]
    y1 = GOLD["expert_lora_gate"]["y"]
    want = g["K2_w"][0] * y0 + g["K2_w"][1] * y1
    assert np.allclose(o, want, rtol=1e-15, atol=0)


def test_router_zero_input():
    w = synth.workload(0)
    r = synth.router_tensors(w, 0)
    x = np.zeros((1, w["H"]), np.uint16)
    l = O.router_logits(r["router_q"], r["router_s"], x)[0]
    assert np.all(l == 0)
    sel = O.select_topk(l, w["K"])
    assert list(sel) == list(range(w["K"]))
    assert np.allclose(O.topk_weights(l, sel), 1.0 / w["K"])
    assert O.shared_gate(r["sgate_q"], r["sgate_s"], x)[0] == 0.5


def test_router_exact_arithmetic_against_fractions():
    # integer x and power-of-two scales: logits are exact rationals
    rng = np.random.default_rng(4)
    E, H = 16, 256
    rq = rng.integers(-127, 128, (E, H)).astype(np.int8)
    rs = (2.0 ** rng.integers(-8, -2, (E, H // 64))).astype(np.float32)
    xi = rng.integers(-8, 9, (2, H))
    x = np.array([[f2bits(float(v)) for v in row] for row in xi], np.uint16)
    l = O.router_logits(rq, rs, x)
    for t in range(2):
        for e in range(E):
            exact = sum(Fraction(float(rs[e, i // 64])) * int(rq[e, i]) * int(xi[t, i])
                        for i in range(H))
            assert Fraction(l[t, e]) == exact


def test_select_topk_brute_force_and_invariants():
    rng = np.random.default_rng(5)
    for trial in range(200):
        E = int(rng.integers(2, 40))
        K = int(rng.integers(1, E + 1))
        # few distinct values so ties are frequent
        l = rng.integers(-3, 4, E).astype(np.float64) * 0.5
        sel = O.select_topk(l, K)
        # brute force: repeatedly take the largest, lowest index first
        remaining = list(range(E))
        want = []
        for _ in range(K):
            best = remaining[0]
            for e in remaining:
                if l[e] > l[best]:
                    best = e
            want.append(best)
            remaining.remove(best)
        assert list(sel) == want
        wts = O.topk_weights(l, sel)
        assert abs(wts.sum() - 1.0) < 1e-12
        # renormalised full softmax equals a softmax over the selected logits
        ls = l[sel]
        direct = np.exp(ls - ls.max()) / np.exp(ls - ls.max()).sum()
        assert np.allclose(wts, direct, rtol=1e-13, atol=0)
        # unnormalised weights are the plain softmax entries
        full = np.exp(l) / np.exp(l).sum()
        assert np.allclose(O.topk_weights(l, sel, norm_topk=False), full[sel],
                           rtol=1e-13, atol=0)
    l = rng.standard_normal(12)
    assert list(O.select_topk(l, 12)) == list(np.argsort(-l, kind="stable"))


# --------------------------------------------------------------------------
# expert FFN
# --------------------------------------------------------------------------
def test_expert_hand_examples():
    g = GOLD["expert_base_only"]
    ex = const_expert(g["H"], g["I"], g["r"], g["code"], g["scale"], g["bias"])
    x = np.ones((1, g["H"]))
    y = O.expert_forward(ex, x, 1.0)
    assert np.allclose(y, g["y"], rtol=1e-15, atol=0)
    assert np.all(O.bf16_value(y) == g["y_bf16"])
    g2 = GOLD["expert_lora_gate"]
    ex2 = const_expert(g2["H"], g2["I"], g2["r"], g2["code"], g2["scale"],
                       g2["bias"], A={"gate": g2["A_gate"]}, B={"gate": g2["B_gate"]})
    y2 = O.expert_forward(ex2, x, 1.0)
    assert np.allclose(y2, g2["y"], rtol=1e-15, atol=0)
    assert np.all(O.bf16_value(y2) == g2["y_bf16"])


def test_block_hand_example_with_shared_expert():
    g1, g2 = GOLD["expert_base_only"], GOLD["expert_lora_gate"]
    H = 64
    routed = const_expert(H, 64, 1, g1["code"], g1["scale"], g1["bias"])
    shared = const_expert(H, 64, 1, g2["code"], g2["scale"], g2["bias"],
                          A={"gate": g2["A_gate"]}, B={"gate": g2["B_gate"]})
    rq, rs = _router_from_codes([1, 1], 0.015625, H)
    router = {"router_q": rq, "router_s": rs,
              "sgate_q": np.zeros((1, H), np.int8),
              "sgate_s": np.ones((1, 1), np.float32)}
    w = dict(H=H, E=2, K=1, lora_scale=1.0)
    x = np.full((1, H), f2bits(1.0), np.uint16)
    o, parts = O.moe_block(w, router, lambda e: routed, x, shared=shared,
                           return_parts=True)
    assert list(parts["idx"][0]) == [0]
    assert parts["g"][0] == 0.5
    assert np.allclose(o, GOLD["block_with_shared"]["o"], rtol=1e-15, atol=0)


def _brute_proj(ex, p, v, lam):
    q, s, b = ex[f"q_{p}"], ex[f"s_{p}"], ex[f"b_{p}"]
    A, B = ex[f"A_{p}"], ex[f"B_{p}"]
    out, n_in = q.shape
    r = A.shape[0]
    Av = [math.fsum(bfv(A[k][i]) * v[i] for i in range(n_in)) for k in range(r)]
    res = []
    for j in range(out):
        terms = [(bfv(s[j][i // 64]) * int(q[j][i]) + bfv(b[j][i // 64])) * v[i]
                 for i in range(n_in)]
        terms += [lam * bfv(B[j][k]) * Av[k] for k in range(r)]
        res.append(math.fsum(terms))
    return res


def _brute_block(w, router, experts, shared, xbits, given=None):
    """Loop formulation of the block for one token, from the definitions.
    given: experts to execute in place of the top-K (prediction-as-routing)."""
    H, E, K, lam = w["H"], w["E"], w["K"], w["lora_scale"]
    x = [bfv(v) for v in xbits]
    logits = []
    for e in range(E):
        logits.append(math.fsum(float(router["router_s"][e][i // 64]) *
                                int(router["router_q"][e][i]) * x[i] for i in range(H)))
    order = sorted(range(E), key=lambda e: (-logits[e], e))[:K] if given is None else list(given)
    m = max(logits)
    den = math.fsum(math.exp(v - m) for v in logits)
    p = [math.exp(logits[e] - m) / den for e in order]
    sp = math.fsum(p)
    p = [v / sp for v in p]

    def ffn(ex):
        ag = _brute_proj(ex, "gate", x, lam)
        au = _brute_proj(ex, "up", x, lam)
        h = [ag[j] / (1 + math.exp(-ag[j])) * au[j] for j in range(len(ag))]
        return _brute_proj(ex, "down", h, lam)

    out = [0.0] * H
    for k, e in enumerate(order):
        y = ffn(experts[e])
        out = [out[i] + p[k] * y[i] for i in range(H)]
    if shared is not None:
        gl = math.fsum(float(router["sgate_s"][0][i // 64]) * int(router["sgate_q"][0][i]) * x[i]
                       for i in range(H))
        g = 1 / (1 + math.exp(-gl))
        y = ffn(shared)
        out = [out[i] + g * y[i] for i in range(H)]
    return order, out


@pytest.mark.parametrize("with_shared", [True, False])
def test_block_matches_brute_force_loops(with_shared):
    # config-0-like but smaller so pure-Python loops finish quickly; random
    # (non-constant) values catch transposed operands and wrong group axes
    w = synth.workload(0, H=128, E=6, K=2, I=64, r=3,
                       n_shared=1 if with_shared else 0)
    router = synth.router_tensors(w, 0, seed=7)
    experts = [synth.expert_tensors(w, 0, e, seed=7) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"], seed=7) if with_shared else None
    x = synth.tokens(w, 0, T=2, seed=7)
    o, parts = O.moe_block(w, router, lambda e: experts[e], x, shared=shared,
                           return_parts=True)
    for t in range(2):
        order, want = _brute_block(w, router, experts, shared, x[t])
        assert list(parts["idx"][t]) == order
        assert np.allclose(o[t], want, rtol=1e-11, atol=1e-11 * np.abs(want).max())


def test_lora_b_zero_reproduces_base_and_base_off_isolates_lora():
    w = synth.workload(0)
    ex = synth.expert_tensors(w, 0, 1)
    x = O.bf16_to_f64(synth.tokens(w, 0, T=3))
    zero_b = dict(ex)
    for p in ("gate", "up", "down"):
        zero_b[f"B_{p}"] = np.zeros_like(ex[f"B_{p}"])
    # base only, written as dense matrices
    Wg = O.dequant_int4_affine(ex["q_gate"], ex["s_gate"], ex["b_gate"])
    Wu = O.dequant_int4_affine(ex["q_up"], ex["s_up"], ex["b_up"])
    Wd = O.dequant_int4_affine(ex["q_down"], ex["s_down"], ex["b_down"])
    base = O.silu(x @ Wg.T) * (x @ Wu.T) @ Wd.T
    assert np.allclose(O.expert_forward(zero_b, x, 1.0), base, rtol=1e-13, atol=0)
    # base off (s = b = 0): only the LoRA chain remains
    off = dict(ex)
    for p in ("gate", "up", "down"):
        off[f"s_{p}"] = np.zeros_like(ex[f"s_{p}"])
        off[f"b_{p}"] = np.zeros_like(ex[f"b_{p}"])
    A = {p: O.bf16_to_f64(ex[f"A_{p}"]) for p in ("gate", "up", "down")}
    B = {p: O.bf16_to_f64(ex[f"B_{p}"]) for p in ("gate", "up", "down")}
    lam = 0.5
    ag = lam * (x @ A["gate"].T) @ B["gate"].T
    au = lam * (x @ A["up"].T) @ B["up"].T
    want = lam * ((O.silu(ag) * au) @ A["down"].T) @ B["down"].T
    assert np.allclose(O.expert_forward(off, x, lam), want, rtol=1e-12, atol=1e-300)


def test_unmerged_equals_merged_dense():
    # independent formulation: merge lambda*B*A into the dense weight
    w = synth.workload(0)
    ex = synth.expert_tensors(w, 0, 2)
    x = O.bf16_to_f64(synth.tokens(w, 3, T=2))
    lam = 0.75
    M = {}
    for p in ("gate", "up", "down"):
        M[p] = (O.dequant_int4_affine(ex[f"q_{p}"], ex[f"s_{p}"], ex[f"b_{p}"]) +
                lam * O.bf16_to_f64(ex[f"B_{p}"]) @ O.bf16_to_f64(ex[f"A_{p}"]))
    want = (O.silu(x @ M["gate"].T) * (x @ M["up"].T)) @ M["down"].T
    got = O.expert_forward(ex, x, lam)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10 * np.abs(want).max())


def test_combine_one_hot_and_no_shared():
    w = synth.workload(0, n_shared=0, K=1)
    router = synth.router_tensors(w, 0)
    x = synth.tokens(w, 0)
    o, parts = O.moe_block(w, router, lambda e: synth.expert_tensors(w, 0, e), x,
                           return_parts=True)
    assert parts["w"][0, 0] == 1.0
    assert np.array_equal(o, parts["y"][:, 0])


# --------------------------------------------------------------------------
# prefill grouping
# --------------------------------------------------------------------------
def test_group_pairs_brute_force():
    rng = np.random.default_rng(6)
    for T, K, E in [(1, 2, 16), (37, 4, 8), (200, 8, 128), (5, 4, 256)]:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
        counts, offsets, perm = O.group_pairs(idx, E)
        assert counts.sum() == T * K and offsets[-1] == T * K and offsets[0] == 0
        assert sorted(perm.tolist()) == list(range(T * K))
        want = []
        for e in range(E):
            for p in range(T * K):
                if idx[p // K][p % K] == e:
                    want.append(p)
        assert perm.tolist() == want
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert len(seg) == counts[e]
            assert np.all(idx.reshape(-1)[seg] == e)


def test_group_pairs_empty():
    counts, offsets, perm = O.group_pairs(np.zeros((0, 4), np.int64), 8)
    assert counts.sum() == 0 and list(offsets) == [0] * 9 and perm.size == 0


# --------------------------------------------------------------------------
# stack wiring and Prerouter
# --------------------------------------------------------------------------
def test_rmsnorm_constant_vector():
    g = GOLD["rmsnorm_constant"]
    v = O.rmsnorm(np.full((1, 64), g["c"]), g["eps"])
    assert np.allclose(v, g["value"], rtol=1e-15, atol=0)


def test_stack_layer_with_zero_block_is_identity():
    w = synth.workload(0, n_shared=0)
    router = synth.router_tensors(w, 0)
    zero = const_expert(w["H"], w["I"], w["r"], 0, 0.0, 0.0)
    h = synth.tokens(w, 5, T=2)
    out = O.stack_layer(w, router, lambda e: zero, h)
    assert np.array_equal(out, h)


def test_stack_layer_hand_example_norm_and_rounding():
    # h' = bf16(h + MoE(bf16(RMSNorm(h)))): a two-valued h whose RMSNorm
    # rounds visibly to bf16, through a constant expert; the block input, the
    # unrounded block output and the layer output all have closed forms
    g = GOLD["stack_layer_norm"]
    H, I = g["H"], g["I"]
    ex = const_expert(H, I, 1, 1, 0.015625, 0.0)
    rq, rs = _router_from_codes([1] * g["E"], 0.015625, H)
    w = dict(H=H, E=g["E"], K=g["K"], lora_scale=1.0)
    h = np.array([[f2bits(g["h_hi"])] * (H // 2) + [f2bits(g["h_lo"])] * (H // 2)], np.uint16)
    out, parts = O.stack_layer(w, {"router_q": rq, "router_s": rs}, lambda e: ex, h,
                               eps=g["eps"], return_parts=True)
    xn = [bfv(v) for v in parts["xn_bits"][0]]
    assert xn == [g["xn_hi"]] * (H // 2) + [g["xn_lo"]] * (H // 2)
    assert parts["idx"].tolist() == [[0]]
    assert np.allclose(parts["o"], g["o"], rtol=1e-14, atol=0)
    assert [bfv(v) for v in out[0]] == [g["out_hi"]] * (H // 2) + [g["out_lo"]] * (H // 2)


def test_prerouter_zero_head_and_brute_force():
    rng = np.random.default_rng(8)
    H, D, E, K = 128, 16, 12, 4
    W1 = synth.f32_to_bf16_bits(rng.standard_normal((D, H)) * 0.1)
    W2 = np.zeros((E, D), np.uint16)
    h = synth.f32_to_bf16_bits(rng.standard_normal((2, H)))
    pred, z = O.prerouter(W1, W2, h, K)
    assert np.all(z == 0) and pred.tolist() == [[0, 1, 2, 3]] * 2
    W2 = synth.f32_to_bf16_bits(rng.standard_normal((E, D)) * 0.1)
    pred, z = O.prerouter(W1, W2, h, K)
    for t in range(2):
        hv = [bfv(v) for v in h[t]]
        a = [math.fsum(bfv(W1[d][i]) * hv[i] for i in range(H)) for d in range(D)]
        a = [v / (1 + math.exp(-v)) for v in a]
        zz = [math.fsum(bfv(W2[e][d]) * a[d] for d in range(D)) for e in range(E)]
        assert np.allclose(z[t], zz, rtol=1e-12, atol=1e-15)
        assert pred[t].tolist() == sorted(range(E), key=lambda e: (-zz[e], e))[:K]


def test_prerouter_feat_pins():
    # Prerouter with routing features (one-hot of the executed experts
    # appended to h): pinned by (1) reduction to the plain head when the
    # feature columns are zero, (2) brute force with explicit sums over the
    # h part plus the selected feature columns, (3) order and padding of the
    # executed list not mattering, (4) a feature column that dominates z.
    rng = np.random.default_rng(31)
    H, D, E, K = 64, 16, 10, 3
    W1h = synth.f32_to_bf16_bits(rng.standard_normal((D, H)) * 0.1)
    W1f = synth.f32_to_bf16_bits(rng.standard_normal((D, E)) * 0.5)
    W2 = synth.f32_to_bf16_bits(rng.standard_normal((E, D)) * 0.1)
    h = synth.f32_to_bf16_bits(rng.standard_normal((2, H)))
    prev = np.array([[1, 4, 7], [0, 9, -1]], np.int32)
    # (1) zero feature columns: the plain head
    W1z = np.concatenate([W1h, np.zeros_like(W1f)], axis=1)
    pz, zz = O.prerouter_feat(W1z, W2, h, prev, K)
    p0, z0 = O.prerouter(W1h, W2, h, K)
    np.testing.assert_array_equal(pz, p0)
    np.testing.assert_allclose(zz, z0, rtol=1e-13, atol=1e-15)
    # (2) brute force
    W1 = np.concatenate([W1h, W1f], axis=1)
    pred, z = O.prerouter_feat(W1, W2, h, prev, K)
    for t in range(2):
        hv = [bfv(v) for v in h[t]]
        sel = [e for e in prev[t] if 0 <= e < E]
        a = [math.fsum([bfv(W1h[d][i]) * hv[i] for i in range(H)] + [bfv(W1f[d][e]) for e in sel])
             for d in range(D)]
        a = [v / (1 + math.exp(-v)) for v in a]
        zb = [math.fsum(bfv(W2[e][d]) * a[d] for d in range(D)) for e in range(E)]
        assert np.allclose(z[t], zb, rtol=1e-12, atol=1e-15)
        assert pred[t].tolist() == sorted(range(E), key=lambda e: (-zb[e], e))[:K]
    # (3) order, padding and repeats of the executed list do not matter (the
    # one-hot is an indicator: an expert executed is 1 however often listed)
    prev2 = np.array([[7, 1, 4, -1], [9, -5, 0, 12]], np.int32)
    p2, z2 = O.prerouter_feat(W1, W2, h, prev2, K)
    np.testing.assert_array_equal(p2, pred)
    np.testing.assert_allclose(z2, z, rtol=1e-13, atol=1e-15)
    prev3 = np.array([[4, 4, 1, 7, 1, 4], [0, 0, 9, 9, 9, -1]], np.int32)
    p3, z3 = O.prerouter_feat(W1, W2, h, prev3, K)
    np.testing.assert_array_equal(p3, pred)
    np.testing.assert_allclose(z3, z, rtol=1e-13, atol=1e-15)
    # (4) a large weight on one feature column into a hidden unit that feeds
    # only expert 5 makes expert 5 the first prediction for tokens that
    # executed expert 2, and changes nothing for tokens that did not
    W1b = W1.copy()
    W1b[0, :] = 0
    W1b[0, H + 2] = synth.f32_to_bf16_bits(np.array([40.0]))[0]
    W2b = np.zeros((E, D), np.uint16)
    W2b[5, 0] = synth.f32_to_bf16_bits(np.array([1.0]))[0]
    pb, zb2 = O.prerouter_feat(W1b, W2b, h, np.array([[2, 3, 4], [3, 4, 6]], np.int32), K)
    assert pb[0, 0] == 5 and zb2[0, 5] > 39
    assert np.all(zb2[1] == 0) and pb[1].tolist() == [0, 1, 2]


# --------------------------------------------------------------------------
# prediction-as-routing: given experts replace the top-K
# --------------------------------------------------------------------------
def test_given_experts_brute_force_loops():
    # the given experts are the two LOWEST-logit experts, in reverse order, so
    # a path that ignored them, re-sorted them or took weights from the top-K
    # would fail
    w = synth.workload(0, H=128, E=6, K=2, I=64, r=3, n_shared=1)
    router = synth.router_tensors(w, 0, seed=9)
    experts = [synth.expert_tensors(w, 0, e, seed=9) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"], seed=9)
    x = synth.tokens(w, 0, T=2, seed=9)
    logits = O.router_logits(router["router_q"], router["router_s"], x)
    given = np.stack([np.argsort(logits[t], kind="stable")[:2][::-1] for t in range(2)])
    for t in range(2):
        assert set(given[t]).isdisjoint(O.select_topk(logits[t], 2))
    o, parts = O.moe_block(w, router, lambda e: experts[e], x, shared=shared,
                           return_parts=True, exec_idx=given)
    assert parts["idx"].tolist() == given.tolist()
    for t in range(2):
        order, want = _brute_block(w, router, experts, shared, x[t], given=given[t])
        assert np.allclose(o[t], want, rtol=1e-11, atol=1e-11 * np.abs(want).max())


def test_given_experts_weights_closed_form():
    # logits 3, 1, 0 (exact): executing experts (2, 1) weighs them by the
    # softmax of their own logits, 1/(1+e) and e/(1+e), renormalised; without
    # renormalisation they keep their full-softmax shares
    H = 64
    rq, rs = _router_from_codes([3, 1, 0], 1.0 / H, H)
    x = np.full((1, H), f2bits(1.0), np.uint16)
    l = O.router_logits(rq, rs, x)[0]
    assert list(l) == [3.0, 1.0, 0.0]
    e = math.e
    w = O.topk_weights(l, [2, 1])
    assert np.allclose(w, [1 / (1 + e), e / (1 + e)], rtol=1e-15, atol=0)
    z = e ** 3 + e + 1
    w = O.topk_weights(l, [2, 1], norm_topk=False)
    assert np.allclose(w, [1 / z, e / z], rtol=1e-15, atol=0)


def test_given_experts_equal_to_topk_reduce_to_router_path():
    w = synth.workload(0)
    router = synth.router_tensors(w, 0, seed=3)
    experts = [synth.expert_tensors(w, 0, e, seed=3) for e in range(w["E"])]
    shared = synth.expert_tensors(w, 0, w["E"], seed=3)
    x = synth.tokens(w, 0, T=3, seed=3)
    o_r, parts = O.moe_block(w, router, lambda e: experts[e], x, shared=shared, return_parts=True)
    o_g = O.moe_block(w, router, lambda e: experts[e], x, shared=shared, exec_idx=parts["idx"])
    np.testing.assert_array_equal(o_g, o_r)
    # a reordering of the given experts changes only the summation order
    o_p = O.moe_block(w, router, lambda e: experts[e], x, shared=shared,
                      exec_idx=parts["idx"][:, ::-1])
    assert np.allclose(o_p, o_r, rtol=1e-13, atol=1e-13 * np.abs(o_r).max())
