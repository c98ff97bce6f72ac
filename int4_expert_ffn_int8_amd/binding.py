"""ctypes binding of libmoe (argument marshalling only).

Each function has the name of the C entry point it calls and takes torch
tensors (device memory) or None; it passes raw pointers and sizes through
and raises MoeError on a non-OK status.  Every step of the computation runs
in the HIP kernels of libmoe.so; there is no fallback path: if the library
is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that libmoe shares (same soname)

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (the CPU tests use
# it for the host-sanitized build).
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(HERE, "libmoe.so")

c_i32, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EHIP", 4: "MOE_EWORKSPACE"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class MoeDims(ctypes.Structure):
    _fields_ = [("H", c_i32), ("I", c_i32), ("E", c_i32), ("K", c_i32), ("r", c_i32),
                ("n_shared", c_i32), ("norm_topk", c_i32), ("lora_scale", c_f32)]


class MoePoolFill(ctypes.Structure):
    _fields_ = [("layer", c_i32), ("expert", c_i32), ("slot", c_i32), ("evicted", c_i32)]


class MoeExperts(ctypes.Structure):
    _fields_ = [("slots", c_vp), ("n_slots", c_i32), ("expert_to_slot", c_vp),
                ("host_blobs", c_vp), ("counters", c_vp), ("read_delay_ns", ctypes.c_uint32)]


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_expert_blob_bytes": (c_sz, [c_i32, c_i32, c_i32]),
    "moe_pack_expert": (c_i32, [c_i32, c_i32, c_i32] + [c_vp] * 15 + [c_vp, c_sz]),
    "moe_workspace_bytes": (c_sz, [ctypes.POINTER(MoeDims), c_i32, c_i32]),
    "moe_route": (c_i32, [ctypes.POINTER(MoeDims), c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp,
                          c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "moe_expert_forward": (c_i32, [ctypes.POINTER(MoeDims), ctypes.POINTER(MoeExperts), c_vp,
                                   c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "moe_combine": (c_i32, [ctypes.POINTER(MoeDims), c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp,
                            c_f32, c_vp]),
    "moe_rmsnorm": (c_i32, [c_vp, c_i32, c_i32, c_f32, c_vp, c_vp]),
    "moe_block_prefill_workspace_bytes": (c_sz, [ctypes.POINTER(MoeDims), c_i32]),
    "moe_block_prefill": (c_i32, [ctypes.POINTER(MoeDims), c_vp, c_vp, c_vp, c_vp, c_vp,
                                  ctypes.POINTER(MoeExperts), c_vp, c_vp, c_i32, c_vp, c_vp, c_vp,
                                  c_vp, c_vp, c_f32, c_vp, c_sz, c_vp]),
    "moe_block_decode_workspace_bytes": (c_sz, [ctypes.POINTER(MoeDims), c_i32]),
    "moe_workspace_init": (c_i32, [c_vp, c_sz, c_vp]),
    "moe_block_decode": (c_i32, [ctypes.POINTER(MoeDims), c_vp, c_vp, c_vp, c_vp,
                                 ctypes.POINTER(MoeExperts), c_vp, c_vp, c_i32, c_i32, c_f32,
                                 c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "moe_block_decode_exec": (c_i32, [ctypes.POINTER(MoeDims), c_vp, c_vp, c_vp, c_vp,
                                      ctypes.POINTER(MoeExperts), c_vp, c_vp, c_i32, c_i32, c_f32,
                                      c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "moe_block_decode_noalloc": (c_i32, [ctypes.POINTER(MoeDims), c_vp, c_vp, c_vp, c_vp,
                                         ctypes.POINTER(MoeExperts), c_vp, c_vp, c_i32, c_i32,
                                         c_f32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "prerouter_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32]),
    "moe_lru_create": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)]),
    "moe_lru_destroy": (None, [c_vp]),
    "moe_lru_plan": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp, c_i32,
                             ctypes.POINTER(c_i32)]),
    "moe_lru_table": (c_i32, [c_vp, c_i32, c_vp]),
    "moe_lru_stats": (c_i32, [c_vp, ctypes.POINTER(ctypes.c_ulonglong),
                              ctypes.POINTER(ctypes.c_ulonglong)]),
    "moe_pool_create": (c_i32, [c_i32, c_i32, c_i32, c_sz, c_vp, c_vp, c_vp, c_vp,
                                ctypes.POINTER(c_vp)]),
    "moe_pool_destroy": (None, [c_vp]),
    "moe_pool_layer": (c_i32, [c_vp, c_i32, c_vp, ctypes.POINTER(MoeExperts)]),
    "moe_pool_update": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp,
                                ctypes.POINTER(c_i32)]),
    "moe_pool_wait_layer": (c_i32, [c_vp, c_i32, c_vp]),
    "moe_pool_wait_layer_filled": (c_i32, [c_vp, c_i32, c_vp]),
    "moe_pool_set_read_delay": (c_i32, [c_vp, ctypes.c_uint32]),
    "moe_pool_sync": (c_i32, [c_vp, c_vp]),
    "moe_pool_lru": (c_vp, [c_vp]),
    "prerouter_predict": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp,
                                  c_vp, c_vp, c_sz, c_vp]),
    "prerouter_predict_feat": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_i32,
                                       c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
}

# symbols the public header declares (checked by the CPU test suite)
HEADER_SYMBOLS = [
    "moe_last_error", "moe_expert_blob_bytes", "moe_pack_expert", "moe_workspace_bytes",
    "moe_route", "moe_expert_forward", "moe_combine", "moe_rmsnorm",
    "moe_block_prefill_workspace_bytes", "moe_block_prefill",
    "moe_block_decode_workspace_bytes", "moe_workspace_init", "moe_block_decode",
    "moe_block_decode_exec", "moe_block_decode_noalloc",
    "prerouter_workspace_bytes", "prerouter_predict", "prerouter_predict_feat",
    "moe_lru_create", "moe_lru_destroy", "moe_lru_plan", "moe_lru_table", "moe_lru_stats",
    "moe_pool_create", "moe_pool_destroy", "moe_pool_layer", "moe_pool_update",
    "moe_pool_wait_layer", "moe_pool_wait_layer_filled", "moe_pool_set_read_delay",
    "moe_pool_sync", "moe_pool_lru",
]

DECODE_NORM_INPUT = 1
DECODE_RESIDUAL = 2
DECODE_ERR_OFFSET = 512  # MOE_DECODE_ERR_OFFSET


def load(path: str = LIB_PATH):
    """Load libmoe.so.  When the in-tree library has not been built yet it is
    built first (hipcc, gfx950); a build or load failure raises: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path) and path == os.path.join(HERE, "libmoe.so"):
        from . import build as _build
        print(f"{path} is not built: building it now", flush=True)
        _build.build()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python -m int4_expert_ffn_int8_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        if not hasattr(lib, name):
            continue
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load().moe_last_error().decode(errors="replace")
        raise MoeError(status, msg)


def ptr(t) -> int | None:
    """Raw address of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_ptr(stream=None) -> int:
    """hipStream_t of a torch stream (None -> torch's current stream; an int is
    taken as a raw handle, 0 = the default stream)."""
    if isinstance(stream, int):
        return stream
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def dims(H, I, E, K, r, n_shared, lora_scale=1.0, norm_topk=1) -> MoeDims:
    return MoeDims(H, I, E, K, r, n_shared, norm_topk, lora_scale)


def moe_expert_blob_bytes(H: int, I: int, r: int) -> int:
    return int(load().moe_expert_blob_bytes(H, I, r))


def moe_workspace_bytes(d: MoeDims, T: int, prefill: bool) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(d), T, int(bool(prefill))))


def moe_pack_expert(H, I, r, ex: dict, out) -> None:
    """Pack numpy logical tensors of one expert into `out` (host numpy uint8)."""
    import numpy as np
    args = []
    keep = []
    for p in ("gate", "up", "down"):
        for k in ("q", "s", "b", "A", "B"):
            a = np.ascontiguousarray(ex[f"{k}_{p}"])
            keep.append(a)
            args.append(a.ctypes.data if a.size else None)
    assert out.flags["C_CONTIGUOUS"]
    _check(load().moe_pack_expert(H, I, r, *args, out.ctypes.data, out.nbytes))


def moe_route(d, gate_q, gate_s, sgate_q, sgate_s, x, T, logit_bias, topk_idx, topk_w,
              shared_w, logits, counts, offsets, perm, ws, stream=None) -> None:
    _check(load().moe_route(ctypes.byref(d), ptr(gate_q), ptr(gate_s), ptr(sgate_q),
                            ptr(sgate_s), ptr(x), T, ptr(logit_bias), ptr(topk_idx),
                            ptr(topk_w), ptr(shared_w), ptr(logits), ptr(counts),
                            ptr(offsets), ptr(perm), ptr(ws),
                            ws.numel() * ws.element_size() if ws is not None else 0,
                            stream_ptr(stream)))


def experts_struct(slots, n_slots, expert_to_slot=None, host_blobs=None,
                   counters=None, read_delay_ns: int = 0) -> MoeExperts:
    return MoeExperts(ptr(slots), n_slots, ptr(expert_to_slot), ptr(host_blobs), ptr(counters),
                      read_delay_ns)


def moe_expert_forward(d, routed: MoeExperts, shared_blob, x, T, topk_idx, counts, offsets,
                       perm, y, ws, stream=None) -> None:
    _check(load().moe_expert_forward(ctypes.byref(d), ctypes.byref(routed), ptr(shared_blob),
                                     ptr(x), T, ptr(topk_idx), ptr(counts), ptr(offsets),
                                     ptr(perm), ptr(y), ptr(ws),
                                     ws.numel() * ws.element_size() if ws is not None else 0,
                                     stream_ptr(stream)))


def moe_combine(d, y, topk_w, shared_w, T, residual, out, norm_out=None, eps=1e-6,
                stream=None) -> None:
    _check(load().moe_combine(ctypes.byref(d), ptr(y), ptr(topk_w), ptr(shared_w), T,
                              ptr(residual), ptr(out), ptr(norm_out), eps, stream_ptr(stream)))


def moe_rmsnorm(h, T, H, eps, out, stream=None) -> None:
    _check(load().moe_rmsnorm(ptr(h), T, H, eps, ptr(out), stream_ptr(stream)))


def moe_block_prefill_workspace_bytes(d: MoeDims, T: int) -> int:
    return int(load().moe_block_prefill_workspace_bytes(ctypes.byref(d), T))


def moe_block_prefill(d, gate_q, gate_s, sgate_q, sgate_s, logit_bias, routed: MoeExperts,
                      shared_blob, x, T, residual, topk_idx, topk_w, out, norm_out, eps, ws,
                      stream=None) -> None:
    """route + experts + combine for T prefill tokens in one call; the expert
    outputs stay in the workspace (fp16 with a power-of-two exponent per row)."""
    _check(load().moe_block_prefill(ctypes.byref(d), ptr(gate_q), ptr(gate_s), ptr(sgate_q),
                                    ptr(sgate_s), ptr(logit_bias), ctypes.byref(routed),
                                    ptr(shared_blob), ptr(x), T, ptr(residual), ptr(topk_idx),
                                    ptr(topk_w), ptr(out), ptr(norm_out), eps, ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0,
                                    stream_ptr(stream)))


def prerouter_workspace_bytes(D: int, E: int, T: int) -> int:
    """Bytes of the Prerouter's workspace for T tokens. The caller zeroes it
    once, before the first call, and reuses it: the calls leave its hand-off
    counter and words in the state the next call expects."""
    return int(load().prerouter_workspace_bytes(D, E, T))


def prerouter_predict(W1, W2, H, D, E, K, h, T, pred_idx, pred_logits, ws, stream=None) -> None:
    """One launch: the head's two layers and its top-K for T tokens. Calls
    that share a workspace must not overlap (same stream or serialised)."""
    _check(load().prerouter_predict(ptr(W1), ptr(W2), H, D, E, K, ptr(h), T, ptr(pred_idx),
                                    ptr(pred_logits), ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0,
                                    stream_ptr(stream)))


def prerouter_predict_feat(W1, W2, H, D, E, K, h, prev_idx, Kp, T, pred_idx, pred_logits, ws,
                           stream=None) -> None:
    _check(load().prerouter_predict_feat(ptr(W1), ptr(W2), H, D, E, K, ptr(h), ptr(prev_idx), Kp,
                                         T, ptr(pred_idx), ptr(pred_logits), ptr(ws),
                                         ws.numel() * ws.element_size() if ws is not None else 0,
                                         stream_ptr(stream)))


def moe_block_decode_workspace_bytes(d: MoeDims, T: int) -> int:
    return int(load().moe_block_decode_workspace_bytes(ctypes.byref(d), T))


def moe_workspace_init(ws, stream=None) -> None:
    _check(load().moe_workspace_init(ptr(ws), ws.numel() * ws.element_size(),
                                     stream_ptr(stream)))


def moe_block_decode(d, gate_q, gate_s, sgate_q, sgate_s, routed: MoeExperts, shared_blob, h_in,
                     T, flags, eps, topk_idx, topk_w, out, ws, stream=None) -> None:
    _check(load().moe_block_decode(ctypes.byref(d), ptr(gate_q), ptr(gate_s), ptr(sgate_q),
                                   ptr(sgate_s), ctypes.byref(routed), ptr(shared_blob),
                                   ptr(h_in), T, flags, eps, ptr(topk_idx), ptr(topk_w),
                                   ptr(out), ptr(ws),
                                   ws.numel() * ws.element_size() if ws is not None else 0,
                                   stream_ptr(stream)))


def moe_block_decode_exec(d, gate_q, gate_s, sgate_q, sgate_s, routed: MoeExperts, shared_blob,
                          h_in, T, flags, eps, exec_idx, topk_idx, topk_w, out, ws,
                          stream=None) -> None:
    _check(load().moe_block_decode_exec(ctypes.byref(d), ptr(gate_q), ptr(gate_s), ptr(sgate_q),
                                        ptr(sgate_s), ctypes.byref(routed), ptr(shared_blob),
                                        ptr(h_in), T, flags, eps, ptr(exec_idx), ptr(topk_idx),
                                        ptr(topk_w), ptr(out), ptr(ws),
                                        ws.numel() * ws.element_size() if ws is not None else 0,
                                        stream_ptr(stream)))


def moe_block_decode_noalloc(d, gate_q, gate_s, sgate_q, sgate_s, routed: MoeExperts,
                             shared_blob, h_in, T, flags, eps, topk_idx, topk_w, out,
                             error_out=None, stream=None) -> None:
    _check(load().moe_block_decode_noalloc(ctypes.byref(d), ptr(gate_q), ptr(gate_s),
                                           ptr(sgate_q), ptr(sgate_s), ctypes.byref(routed),
                                           ptr(shared_blob), ptr(h_in), T, flags, eps,
                                           ptr(topk_idx), ptr(topk_w), ptr(out), ptr(error_out),
                                           stream_ptr(stream)))


# ---- expert pool ------------------------------------------------------------
def _i32_array(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data


class MoeLru:
    """Host LRU planner (moe_lru_*); usable without a GPU."""

    def __init__(self, n_layers: int, E: int, n_slots: int):
        self.h = None
        h = c_vp()
        _check(load().moe_lru_create(n_layers, E, n_slots, ctypes.byref(h)))
        self.h, self.n_layers, self.E, self.n_slots = h, n_layers, E, n_slots

    def plan(self, executed, predicted=None, max_fills: int = -1):
        """executed int [n_layers, K], predicted int [n_layers, Kp] or None;
        returns a list of (layer, expert, slot, evicted)."""
        import numpy as np
        ex, exp = _i32_array(executed)
        K = ex.shape[1] if ex.ndim == 2 else 0
        if predicted is None:
            pr, prp, Kp = None, None, 0
        else:
            pr, prp = _i32_array(predicted)
            Kp = pr.shape[1]
        cap = self.n_layers * (K + Kp) + 1
        fills = (MoePoolFill * cap)()
        n = c_i32(0)
        _check(load().moe_lru_plan(self.h, exp, K, prp, Kp, max_fills, fills, cap, ctypes.byref(n)))
        return [(f.layer, f.expert, f.slot, f.evicted) for f in fills[:n.value]]

    def table(self, layer: int):
        import numpy as np
        out = np.empty(self.E, np.int32)
        _check(load().moe_lru_table(self.h, layer, out.ctypes.data))
        return out

    def stats(self):
        f, e = ctypes.c_ulonglong(0), ctypes.c_ulonglong(0)
        _check(load().moe_lru_stats(self.h, ctypes.byref(f), ctypes.byref(e)))
        return int(f.value), int(e.value)

    def close(self):
        if getattr(self, "h", None):
            load().moe_lru_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()


class MoePool:
    """Device expert pool (moe_pool_*).  The caller keeps slots, table and
    host_blobs alive for the pool's lifetime."""

    def __init__(self, n_layers, E, n_slots, blob_bytes, slots, table, host_blobs, stream=None):
        self.h = None
        h = c_vp()
        _check(load().moe_pool_create(n_layers, E, n_slots, blob_bytes, ptr(slots), ptr(table),
                                      ptr(host_blobs), stream_ptr(stream), ctypes.byref(h)))
        self.h, self.n_layers, self.E, self.n_slots = h, n_layers, E, n_slots
        self._keep = (slots, table, host_blobs)

    def layer(self, layer: int, counters=None) -> MoeExperts:
        out = MoeExperts()
        _check(load().moe_pool_layer(self.h, layer, ptr(counters), ctypes.byref(out)))
        return out

    def update(self, executed, predicted=None, max_fills: int = -1, side_stream=None) -> int:
        ex, exp = _i32_array(executed)
        K = ex.shape[1]
        if predicted is None:
            pr, prp, Kp = None, None, 0
        else:
            pr, prp = _i32_array(predicted)
            Kp = pr.shape[1]
        n = c_i32(0)
        _check(load().moe_pool_update(self.h, exp, K, prp, Kp, max_fills, stream_ptr(side_stream),
                                      ctypes.byref(n)))
        return n.value

    def wait_layer(self, layer: int, stream=None) -> None:
        _check(load().moe_pool_wait_layer(self.h, layer, stream_ptr(stream)))

    def wait_layer_filled(self, layer: int, stream=None) -> None:
        _check(load().moe_pool_wait_layer_filled(self.h, layer, stream_ptr(stream)))

    def set_read_delay(self, ns: int) -> None:
        _check(load().moe_pool_set_read_delay(self.h, int(ns)))

    def sync(self, side_stream=None) -> None:
        _check(load().moe_pool_sync(self.h, stream_ptr(side_stream)))

    def table(self, layer: int):
        import numpy as np
        out = np.empty(self.E, np.int32)
        _check(load().moe_lru_table(load().moe_pool_lru(self.h), layer, out.ctypes.data))
        return out

    def stats(self):
        f, e = ctypes.c_ulonglong(0), ctypes.c_ulonglong(0)
        _check(load().moe_lru_stats(load().moe_pool_lru(self.h), ctypes.byref(f), ctypes.byref(e)))
        return int(f.value), int(e.value)

    def close(self):
        if getattr(self, "h", None):
            load().moe_pool_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()
