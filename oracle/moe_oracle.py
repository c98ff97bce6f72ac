"""Plain, slow, obviously-correct fp64 definition of the MoE block.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark; never by the HIP product path.

Sources (cited by page title and section; the pages print no formulas, so the
arithmetic below is the plainest reading of their prose plus the workload
definition that fixes the FFN form and the routing order):

  [P1] "Edge0开源框架实现35BMoE模型在Mac上流式推理，峰值内存仅2.9GiB"
       (tech.news18a.com) -- Recover-LoRA paragraph; Prerouter paragraph.
  [P2] "SSD 专家卸载 · Prerouter 路由预测" (autoark.ai, Edge0 blog) -- tier
       table; prefill/decode paragraph; Prerouter double-shift paragraph.
  [P3] "iPhone、Mac、Android、Windows 实测横评：Edge0 五大平台谁最能打"
       (2kiu.com) -- model-structure paragraph; "三件套" bullets (affine
       4-bit, group_size 64; prediction heads; unmerged LoRA); quality
       section (router gate and shared-expert gate kept at 8 bit).

Everything is computed in float64.  bf16 inputs are widened exactly; the only
roundings are the ones that define an interface: bf16 block/stack outputs.

Readings where the pages are silent:
  * int4 dequant is affine per 64 consecutive input columns of one output row:
    w = s*q + b, q in {0..15}, s and b bf16.
  * int8 gates are symmetric: w = s*q, fp32 scale per 64 columns.
  * routing selects on logits by the key (-logit, index): ties go to the lower
    index; weights are the full softmax restricted to the selection and
    renormalised (norm_topk), or left unnormalised.
  * experts are SwiGLU: h = silu(gate) * up, y = down(h); each projection adds
    an unmerged LoRA delta lambda * B (A v).
  * shared expert output is scaled by sigmoid(shared-gate logit).
  * stacks: x_l = bf16(RMSNorm(h_l)), h_{l+1} = bf16(h_l + MoE_l(x_l)).
  * prediction-as-routing ([P3] "三件套" Prerouter bullet: the prediction is
    used as the route; [P2] Prerouter paragraph: predicted routes take part
    in the real execution): the given experts replace the top-K selection,
    in the given order; the router still runs, and their weights are the
    same softmax of the router logits restricted to them (renormalised with
    norm_topk).
"""
from __future__ import annotations

import numpy as np

GROUP = 64  # [P3] "三件套" bullets: config.json group_size 64, 4 bits, affine

__all__ = [
    "GROUP", "bf16_to_f64", "round_bf16", "bf16_value", "dequant_int4_affine",
    "dequant_int8_sym", "router_logits", "select_topk", "topk_weights",
    "shared_gate", "silu", "sigmoid", "expert_forward", "moe_block",
    "group_pairs", "rmsnorm", "stack_layer", "prerouter", "prerouter_feat", "quantize_int4_affine",
    "quantize_int8_sym",
]


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); uint16 bits.

    Rounds directly from float64 (no float32 detour): the significand is cut
    to 8 bits with round-half-to-even.  Values are never in the bf16
    subnormal range here; that range is rejected.
    """
    x = np.asarray(x, dtype=np.float64)
    tiny = (x != 0) & (np.abs(x) < 2.0 ** -126)
    if np.any(tiny):
        raise ValueError("bf16 subnormal range not supported by the oracle")
    u = x.view(np.uint64)
    drop = 45  # 52 fraction bits in float64, 7 kept in bf16
    lsb = (u >> np.uint64(drop)) & np.uint64(1)
    r = (u + np.uint64((1 << (drop - 1)) - 1) + lsb) >> np.uint64(drop)
    r = r << np.uint64(drop)
    f32 = r.view(np.float64).astype(np.float32)  # exact: <= 8 significant bits
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(x) -> np.ndarray:
    """float64 value of round_bf16(x)."""
    return bf16_to_f64(round_bf16(x))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


# --------------------------------------------------------------------------
# dequantisation
# --------------------------------------------------------------------------
def dequant_int4_affine(q, s_bits, b_bits) -> np.ndarray:
    """Dense fp64 weights of a 4-bit affine, group-64 projection.

    [P3] "三件套" bullets: the checkpoint is 4-bit affine with group_size 64.
    q: uint8 [out, in] codes 0..15; s_bits, b_bits: bf16 [out, in/64].
    w[j, i] = s[j, i // 64] * q[j, i] + b[j, i // 64].
    """
    q = np.asarray(q)
    out, n_in = q.shape
    s = bf16_to_f64(s_bits)
    b = bf16_to_f64(b_bits)
    assert s.shape == (out, n_in // GROUP) and b.shape == s.shape
    col_group = np.arange(n_in) // GROUP
    return s[:, col_group] * q.astype(np.float64) + b[:, col_group]


def dequant_int8_sym(q, s) -> np.ndarray:
    """Dense fp64 weights of an int8 symmetric, group-64 gate.

    [P3] quality section: each layer's router gate and shared-expert gate are
    kept at 8 bits inside the 4-bit group-64 grid.  Reading: symmetric codes,
    fp32 scale per 64 columns, w[e, i] = s[e, i // 64] * q[e, i].
    """
    q = np.asarray(q)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    col_group = np.arange(q.shape[1]) // GROUP
    return s[:, col_group] * q.astype(np.float64)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def router_logits(rq, rs, x_bits, bias=None) -> np.ndarray:
    """Router logits l = W_r x (+ bias) for every token; [T, E] float64.

    [P2] tier table / [P3] model-structure paragraph: a router picks K of E
    routed experts per token.  The bias is the optional per-expert logit
    offset of the skewed prefill workload.
    """
    W = dequant_int8_sym(rq, rs)
    x = bf16_to_f64(x_bits)
    l = x @ W.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return l


def select_topk(l, K: int) -> np.ndarray:
    """Indices of the K largest logits, ordered by (-logit, index).

    Equal logits go to the lower expert index.  l: [E] (one token).
    """
    l = np.asarray(l, dtype=np.float64)
    order = np.lexsort((np.arange(l.shape[0]), -l))
    return order[:K].astype(np.int64)


def topk_weights(l, sel, norm_topk: bool = True) -> np.ndarray:
    """Routing weights of the selected experts for one token.

    Softmax over all E logits, restricted to the selection; renormalised to
    sum 1 over the selection when norm_topk.
    """
    l = np.asarray(l, dtype=np.float64)
    e = np.exp(l - l.max())
    p = e / e.sum()
    w = p[np.asarray(sel)]
    if norm_topk:
        w = w / w.sum()
    return w


def shared_gate(sq, ss, x_bits) -> np.ndarray:
    """Shared-expert gate g = sigmoid(w_sg . x) per token; [T].

    [P3] quality section: the shared-expert gate is an 8-bit projection.
    """
    w = dequant_int8_sym(sq, ss)[0]
    x = bf16_to_f64(x_bits)
    return sigmoid(x @ w)


# --------------------------------------------------------------------------
# expert FFN with unmerged LoRA
# --------------------------------------------------------------------------
def _proj(ex, p, v, lam):
    """One projection with its unmerged LoRA delta: deq(Q) v + lam B (A v).

    [P1] Recover-LoRA paragraph / [P3] "三件套" bullets: the int4 base stays
    frozen and a LoRA adapter is kept unmerged and added at inference.
    v: [..., in] float64.
    """
    W = dequant_int4_affine(ex[f"q_{p}"], ex[f"s_{p}"], ex[f"b_{p}"])
    A = bf16_to_f64(ex[f"A_{p}"])  # [r, in]
    B = bf16_to_f64(ex[f"B_{p}"])  # [out, r]
    base = v @ W.T
    lora = (v @ A.T) @ B.T
    return base + lam * lora


def expert_forward(ex, x, lam: float, return_hidden=False):
    """SwiGLU expert with LoRA on gate, up and down.

    a_g = gate(x), a_u = up(x), h = silu(a_g) * a_u, y = down(h);
    x: [..., H] float64 (already widened).  Returns y [..., H].
    """
    a_g = _proj(ex, "gate", x, lam)
    a_u = _proj(ex, "up", x, lam)
    h = silu(a_g) * a_u
    y = _proj(ex, "down", h, lam)
    if return_hidden:
        return y, h
    return y


def moe_block(w, router, expert_of, x_bits, bias=None, shared=None,
              return_parts=False, exec_idx=None):
    """Full MoE block for T tokens, one token at a time by definition.

    w: workload dict (H, E, K, lora_scale, n_shared, norm_topk optional);
    router: dict with router_q/router_s (and sgate_q/sgate_s if shared);
    expert_of(e) -> logical tensors of routed expert e;
    shared: logical tensors of the shared expert or None.
    Returns o [T, H] float64 (before the bf16 output rounding) and, with
    return_parts, a dict of logits, idx, weights, gate and per-slot y.

    Prefill evaluates the same per-token result: the pages' prefill/decode
    paragraph ([P2]) changes how experts are loaded and batched, not what each
    token computes.

    exec_idx [T, K] (prediction-as-routing): execute these experts instead of
    the router's top-K; weights as topk_weights over the given experts.
    """
    K = w["K"]
    lam = float(w["lora_scale"])
    norm = bool(w.get("norm_topk", 1))
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    logits = router_logits(router["router_q"], router["router_s"], x_bits, bias)
    idx = np.zeros((T, K), dtype=np.int64)
    wts = np.zeros((T, K))
    for t in range(T):
        idx[t] = select_topk(logits[t], K) if exec_idx is None else np.asarray(exec_idx)[t]
        wts[t] = topk_weights(logits[t], idx[t], norm)
    n_slots = K + (1 if shared is not None else 0)
    y = np.zeros((T, n_slots, x.shape[1]))
    # evaluate each distinct expert once over the tokens routed to it
    for e in np.unique(idx):
        rows, ks = np.nonzero(idx == e)
        y[rows, ks] = expert_forward(expert_of(int(e)), x[rows], lam)
    g = None
    o = np.einsum("tk,tkh->th", wts, y[:, :K])
    if shared is not None:
        g = shared_gate(router["sgate_q"], router["sgate_s"], x_bits)
        y[:, K] = expert_forward(shared, x, lam)
        o = o + g[:, None] * y[:, K]
    if return_parts:
        return o, dict(logits=logits, idx=idx, w=wts, g=g, y=y)
    return o


# --------------------------------------------------------------------------
# prefill grouping
# --------------------------------------------------------------------------
def group_pairs(idx, E: int):
    """Group (token, k) pairs by expert for batched prefill.

    [P2] prefill/decode paragraph: prefill loads whole layers and computes in
    batches.  Returns counts [E], offsets [E+1] (exclusive prefix, offsets[E] =
    T*K) and perm [T*K]: pair ids p = t*K + k listed expert by expert, each
    expert's pairs in ascending p.
    """
    idx = np.asarray(idx, dtype=np.int64)
    flat = idx.reshape(-1)
    counts = np.array([(flat == e).sum() for e in range(E)], dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.concatenate([np.nonzero(flat == e)[0] for e in range(E)]
                          + [np.zeros(0, dtype=np.int64)]).astype(np.int64)
    return counts, offsets, perm


# --------------------------------------------------------------------------
# stack wiring and Prerouter
# --------------------------------------------------------------------------
def rmsnorm(h, eps: float) -> np.ndarray:
    """RMSNorm with unit gain: h / sqrt(mean(h^2) + eps), per token."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def stack_layer(w, router, expert_of, h_bits, shared=None, eps=1e-6,
                return_parts=False, exec_idx=None):
    """One decoder-free stack layer: h' = bf16(h + MoE(bf16(RMSNorm(h)))).

    Attention is replaced by the identity in the stacked workloads, so layers
    are joined by the residual add and RMSNorm alone.  Returns the bf16 bits
    of h' (and the parts of the MoE call with return_parts).
    """
    h = bf16_to_f64(h_bits)
    xn_bits = round_bf16(rmsnorm(h, eps))
    res = moe_block(w, router, expert_of, xn_bits, shared=shared,
                    return_parts=return_parts, exec_idx=exec_idx)
    o, parts = (res if return_parts else (res, None))
    out = round_bf16(h + o)
    if return_parts:
        parts["xn_bits"] = xn_bits
        parts["o"] = o
        return out, parts
    return out


def prerouter(W1_bits, W2_bits, h_bits, K: int):
    """Prerouter head: z = W2 silu(W1 h); prediction = top-K of z.

    [P1] Prerouter paragraph / [P2] double-shift paragraph: a light MLP head
    after layer N predicts the experts of layer N+1 (for the next token).
    Two bias-free bf16 linear layers with SiLU between; the prediction is
    ordered by (-z, index).  Returns (pred [T, K], z [T, E]).
    """
    W1 = bf16_to_f64(W1_bits)
    W2 = bf16_to_f64(W2_bits)
    h = bf16_to_f64(h_bits)
    z = silu(h @ W1.T) @ W2.T
    pred = np.stack([select_topk(z[t], K) for t in range(z.shape[0])])
    return pred, z


def prerouter_feat(W1_bits, W2_bits, h_bits, prev_idx, K: int):
    """Prerouter head with routing features: the input is h with the one-hot
    of the experts the layer executed appended, z = W2 silu(W1 [h; onehot]).

    [P1] Prerouter paragraph (the head also sees the experts already
    executed) and [P2] Prerouter paragraph (routing features as input).
    W1 is [D, H + E]; prev_idx [T, Kp] holds expert ids, entries outside
    [0, E) are padding.  Returns (pred [T, K], z [T, E]).
    """
    W1 = bf16_to_f64(W1_bits)
    W2 = bf16_to_f64(W2_bits)
    h = bf16_to_f64(h_bits)
    E = W2.shape[0]
    T = h.shape[0]
    onehot = np.zeros((T, E))
    for t in range(T):
        for e in prev_idx[t]:
            if 0 <= e < E:
                onehot[t, e] = 1.0
    z = silu(np.concatenate([h, onehot], axis=1) @ W1.T) @ W2.T
    pred = np.stack([select_topk(z[t], K) for t in range(T)])
    return pred, z


# --------------------------------------------------------------------------
# quantisers (only for the round-trip invariant; inputs are drawn as codes)
# --------------------------------------------------------------------------
def _bf16_down(x):
    """Largest bf16 value <= x."""
    v = bf16_value(x)
    bits = round_bf16(x).astype(np.int64)
    over = v > x
    # step one bf16 ulp toward -inf where rounding went up
    step = np.where(np.asarray(x) >= 0, -1, 1)
    bits = np.where(over, bits + step, bits)
    return bf16_to_f64(bits.astype(np.uint16)), bits.astype(np.uint16)


def _bf16_up(x):
    """Smallest bf16 value >= x."""
    v = bf16_value(x)
    bits = round_bf16(x).astype(np.int64)
    under = v < x
    step = np.where(np.asarray(x) >= 0, 1, -1)
    bits = np.where(under, bits + step, bits)
    return bf16_to_f64(bits.astype(np.uint16)), bits.astype(np.uint16)


def quantize_int4_affine(w):
    """Quantise fp64 weights [out, in] to 4-bit affine group-64 codes.

    b = largest bf16 <= group min, s = smallest bf16 >= (max - b) / 15,
    q = clamp(round_half_even((w - b) / s), 0, 15) (q = 0 when s = 0).
    Returns (q uint8, s bits, b bits).
    """
    w = np.asarray(w, dtype=np.float64)
    out, n_in = w.shape
    g = w.reshape(out, n_in // GROUP, GROUP)
    bmin = g.min(axis=2)
    b, b_bits = _bf16_down(bmin)
    s, s_bits = _bf16_up((g.max(axis=2) - b) / 15.0)
    safe = np.where(s > 0, s, 1.0)
    q = np.rint((g - b[..., None]) / safe[..., None])
    q = np.where(s[..., None] > 0, q, 0.0)
    q = np.clip(q, 0, 15).astype(np.uint8).reshape(out, n_in)
    return q, s_bits, b_bits


def quantize_int8_sym(w):
    """Quantise fp64 weights [rows, in] to symmetric int8 group-64 codes.

    s = max|w| / 127 in fp32, q = round_half_even(w / s) clamped to [-127,
    127] (q = 0 when s = 0).  Returns (q int8, s float32).
    """
    w = np.asarray(w, dtype=np.float64)
    rows, n_in = w.shape
    g = w.reshape(rows, n_in // GROUP, GROUP)
    s = (np.abs(g).max(axis=2) / 127.0).astype(np.float32)
    s64 = s.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    q = np.where(s64[..., None] > 0, np.rint(g / safe[..., None]), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8).reshape(rows, n_in)
    return q, s
