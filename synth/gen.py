"""Seeded generators for every synthetic tensor the MoE workloads use.

Recipe (the pages print no weights, so every value is drawn here):

* routed and shared expert projections gate/up/down: uint4 codes uniform in
  {0..15} (one code per element, uint8 array; each random byte supplies two
  independent codes, low nibble first), per-64-column-group scale
  |N(0, 0.02)| and bias N(0, 0.01), both rounded to bf16;
* LoRA factors A [r, in] and B [out, r]: N(0, 0.02) rounded to bf16;
* router gate and shared-expert gate: fp32 weights N(0, 0.02), stored as
  symmetric int8 codes with one fp32 scale per 64 columns, the group's largest
  magnitude / 127 (codes = weights / scale rounded to nearest, ties to even).
  At H = 2048 and x ~ N(0, 1) this gives router logits of standard deviation
  about 0.02 * sqrt(2048) = 0.9.  This is how the inputs are made; the method
  itself only ever reads the stored codes and scales;
* token activations x: N(0, 1) rounded to bf16;
* Zipf rank bias for the skewed prefill: a seeded permutation of ranks 1..E,
  bias[e] = -s * ln(rank[e]);
* Prerouter head weights W1 [D, H], W2 [E, D]: N(0, 0.02) rounded to bf16.

Every tensor has its own stream: numpy PCG64 seeded with
SeedSequence([seed, workload, layer, tensor_id, index]).  bf16 tensors are
returned as uint16 bit patterns (round-to-nearest-even from float32).
"""
from __future__ import annotations

import numpy as np

# Workload shapes.  Names say what each workload is.
WORKLOADS = {
    0: dict(name="tiny_block_decode_h256_e16_k2", H=256, E=16, K=2, I=128,
            n_shared=1, r=4, lora_scale=1.0, T=1, layers=1),
    1: dict(name="block_decode_h2048_e256_k4_i512", H=2048, E=256, K=4, I=512,
            n_shared=1, r=16, lora_scale=1.0, T=1, layers=1, steps=1000),
    2: dict(name="stack24_decode_h2048_e128_k8_i512", H=2048, E=128, K=8, I=512,
            n_shared=0, r=16, lora_scale=1.0, T=1, layers=24, warmup=10,
            timed=200, rms_eps=1e-6),
    3: dict(name="stack40_prerouter_pool64_decode_h2048_e256_k4_i512", H=2048,
            E=256, K=4, I=512, n_shared=1, r=16, lora_scale=1.0, T=1,
            layers=40, prerouter_D=256, pool_slots=64, warmup=10, timed=200,
            rms_eps=1e-6),
    4: dict(name="block_prefill_t3300_h2048_e256_k4_i512_zipf1.1", H=2048,
            E=256, K=4, I=512, n_shared=1, r=16, lora_scale=1.0, T=3300,
            layers=1, zipf_s=1.1),
    # the 8B-shaped layer (as in the 24-layer stack) as a second prefill
    # workload: 128 experts, top-8, no shared expert, same token count and bias
    5: dict(name="block_prefill_t3300_h2048_e128_k8_i512_zipf1.1", H=2048,
            E=128, K=8, I=512, n_shared=0, r=16, lora_scale=1.0, T=3300,
            layers=1, zipf_s=1.1),
}

_TID = {
    "router_q": 1, "router_s": 2, "sgate_q": 3, "sgate_s": 4, "x": 5,
    "zipf": 6, "pr_w1": 7, "pr_w2": 8, "pr_w1f": 9,
}
_PROJ = ("gate", "up", "down")
for _i, _p in enumerate(_PROJ):
    _TID[f"q_{_p}"] = 10 + 5 * _i
    _TID[f"s_{_p}"] = 11 + 5 * _i
    _TID[f"b_{_p}"] = 12 + 5 * _i
    _TID[f"A_{_p}"] = 13 + 5 * _i
    _TID[f"B_{_p}"] = 14 + 5 * _i


def workload(wid: int, **overrides) -> dict:
    w = dict(WORKLOADS[wid])
    w.update(overrides)
    w["id"] = wid
    return w


def _rng(seed: int, wid: int, layer: int, tensor: str, index: int = 0):
    ss = np.random.SeedSequence([seed, wid, layer, _TID[tensor], index])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite floats have bit patterns below 0xFF800000, so u + 0x8000 cannot
    # wrap in 32 bits (values are drawn finite)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _bf16_normal(rng, std, shape, absval=False):
    v = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    if absval:
        v = np.abs(v)
    return f32_to_bf16_bits(v)


def _codes(rng, shape) -> np.ndarray:
    n = int(np.prod(shape))
    b = np.frombuffer(rng.bytes((n + 1) // 2), dtype=np.uint8)
    c = np.empty(2 * b.size, dtype=np.uint8)
    c[0::2] = b & 15
    c[1::2] = b >> 4
    return c[:n].reshape(shape)


def expert_tensors(w: dict, layer: int, expert: int, seed: int = 0) -> dict:
    """Logical tensors of one expert (expert == E is the shared expert).

    Returns a dict with, for p in gate/up/down:
      q_p uint8 [out, in] codes, s_p / b_p uint16 bf16 [out, in/64],
      A_p uint16 bf16 [r, in], B_p uint16 bf16 [out, r];
    gate/up have (out, in) = (I, H), down has (H, I).
    """
    H, I, r, wid = w["H"], w["I"], w["r"], w["id"]
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    out = {}
    for p in _PROJ:
        o, i = shapes[p]
        out[f"q_{p}"] = _codes(_rng(seed, wid, layer, f"q_{p}", expert), (o, i))
        out[f"s_{p}"] = _bf16_normal(_rng(seed, wid, layer, f"s_{p}", expert),
                                     0.02, (o, i // 64), absval=True)
        out[f"b_{p}"] = _bf16_normal(_rng(seed, wid, layer, f"b_{p}", expert),
                                     0.01, (o, i // 64))
        out[f"A_{p}"] = _bf16_normal(_rng(seed, wid, layer, f"A_{p}", expert),
                                     0.02, (r, i))
        out[f"B_{p}"] = _bf16_normal(_rng(seed, wid, layer, f"B_{p}", expert),
                                     0.02, (o, r))
    return out


def _int8_gate_codes(rng, rows: int, H: int):
    """Draw fp32 N(0, 0.02) gate weights [rows, H] and store them as int8
    codes with a per-64-column fp32 scale (group max magnitude / 127)."""
    v = rng.standard_normal(size=(rows, H), dtype=np.float32) * np.float32(0.02)
    g = v.reshape(rows, H // 64, 64).astype(np.float64)
    s = (np.abs(g).max(axis=2) / 127.0).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float64)
    q = np.clip(np.rint(g / safe[..., None]), -127, 127).astype(np.int8)
    return q.reshape(rows, H), s


def router_tensors(w: dict, layer: int, seed: int = 0) -> dict:
    """int8 router gate [E, H] + fp32 scales [E, H/64]; shared gate [1, H]."""
    H, E, wid = w["H"], w["E"], w["id"]
    out = {}
    out["router_q"], out["router_s"] = _int8_gate_codes(_rng(seed, wid, layer, "router_q"), E, H)
    if w.get("n_shared", 0):
        out["sgate_q"], out["sgate_s"] = _int8_gate_codes(_rng(seed, wid, layer, "sgate_q"), 1, H)
    return out


def tokens(w: dict, step: int, T: int | None = None, seed: int = 0) -> np.ndarray:
    """Token activations x ~ N(0, 1) as bf16 bits [T, H] for one step."""
    T = w["T"] if T is None else T
    return _bf16_normal(_rng(seed, w["id"], 0, "x", step), 1.0, (T, w["H"]))


def zipf_bias(w: dict, seed: int = 0) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank), rank a seeded permutation of 1..E."""
    E = w["E"]
    rank = _rng(seed, w["id"], 0, "zipf").permutation(E).astype(np.float64) + 1.0
    return (-w["zipf_s"] * np.log(rank)).astype(np.float32)


def prerouter_tensors(w: dict, layer: int, seed: int = 0) -> dict:
    """Prerouter head after `layer`: W1 [D, H], W2 [E, D], bf16 bits."""
    D, H, E, wid = w["prerouter_D"], w["H"], w["E"], w["id"]
    return {
        "W1": _bf16_normal(_rng(seed, wid, layer, "pr_w1"), 0.02, (D, H)),
        "W2": _bf16_normal(_rng(seed, wid, layer, "pr_w2"), 0.02, (E, D)),
    }


def prerouter_feat_tensors(w: dict, layer: int, seed: int = 0) -> dict:
    """Prerouter head with routing features after `layer`: W1 [D, H + E] (the
    plain head's W1, then one N(0, 0.02) column per expert for the one-hot of
    the executed experts), W2 [E, D]; bf16 bits."""
    base = prerouter_tensors(w, layer, seed)
    D, E, wid = w["prerouter_D"], w["E"], w["id"]
    extra = _bf16_normal(_rng(seed, wid, layer, "pr_w1f"), 0.02, (D, E))
    return {"W1": np.concatenate([base["W1"], extra], axis=1), "W2": base["W2"]}
