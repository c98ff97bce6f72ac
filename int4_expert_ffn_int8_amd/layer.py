"""Device-resident MoE layer: packs logical tensors into expert blobs, uploads
them, and runs one block through the C ABI (route -> expert_forward ->
combine).  Marshalling only: all arithmetic happens in libmoe's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def pack_experts(H: int, I: int, r: int, experts, n: int | None = None, threads: int = 1,
                 out: np.ndarray | None = None) -> np.ndarray:
    """Pack logical expert tensors into blobs [n, bytes].

    `experts` is a list of dicts of numpy arrays, or a callable e -> dict
    (then `n` experts are produced and packed on `threads` threads; the
    packer releases the GIL).  `out` may be a preallocated (e.g. pinned)
    uint8 array of shape [n, blob_bytes]."""
    nb = B.moe_expert_blob_bytes(H, I, r)
    if callable(experts):
        make = experts
    else:
        lst = list(experts)
        n = len(lst)
        make = lst.__getitem__
    if out is None:
        out = np.zeros((n, nb), np.uint8)

    def one(i):
        B.moe_pack_expert(H, I, r, make(i), out[i])

    if threads <= 1:
        for i in range(n):
            one(i)
    else:
        import concurrent.futures
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n)))
    return out


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 (bf16 bits) travels as int16."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class MoeLayer:
    """One MoE block whose routed experts all live in HBM (or in a pool)."""

    def __init__(self, H, I, E, K, r, n_shared, lora_scale, router: dict, experts,
                 shared: dict | None, norm_topk: int = 1, device="cuda", blobs=None,
                 shared_blob=None):
        self.H, self.I, self.E, self.K, self.r = H, I, E, K, r
        self.S = n_shared
        self.d = B.dims(H, I, E, K, r, n_shared, lora_scale, norm_topk)
        self.device = device
        self.gate_q = dev(router["router_q"], device)
        self.gate_s = dev(router["router_s"], device)
        self.sgate_q = dev(router["sgate_q"].reshape(-1), device) if n_shared else None
        self.sgate_s = dev(router["sgate_s"].reshape(-1), device) if n_shared else None
        self.blob_bytes = B.moe_expert_blob_bytes(H, I, r)
        if blobs is None:
            blobs = pack_experts(H, I, r, experts)
        self.slots = dev(blobs, device) if blobs is not None else None
        if not n_shared:
            self.shared_blob = None
        elif shared_blob is not None:  # already packed
            self.shared_blob = dev(np.ascontiguousarray(shared_blob), device)
        else:
            self.shared_blob = dev(pack_experts(H, I, r, [shared])[0], device)
        self.experts = B.experts_struct(self.slots, E)

    def buffers(self, T: int, prefill: bool = False) -> dict:
        dv = self.device
        KS = self.K + self.S
        b = {
            "T": T,
            "prefill": prefill,
            "idx": torch.empty((T, self.K), dtype=torch.int32, device=dv),
            "w": torch.empty((T, self.K), dtype=torch.float32, device=dv),
            "sw": torch.empty((max(T, 1),), dtype=torch.float32, device=dv) if self.S else None,
            "logits": torch.empty((T, self.E), dtype=torch.float32, device=dv),
            "y": torch.empty((T, KS, self.H), dtype=torch.float32, device=dv),
            "out": torch.empty((T, self.H), dtype=torch.int16, device=dv),
            "ws": torch.empty((max(B.moe_workspace_bytes(self.d, T, prefill), 1),),
                              dtype=torch.uint8, device=dv),
        }
        if prefill:
            b["counts"] = torch.empty((self.E,), dtype=torch.int32, device=dv)
            b["offsets"] = torch.empty((self.E + 1,), dtype=torch.int32, device=dv)
            b["perm"] = torch.empty((max(T * self.K, 1),), dtype=torch.int32, device=dv)
        else:
            b["counts"] = b["offsets"] = b["perm"] = None
        return b

    def route(self, x, b, bias=None, stream=None):
        B.moe_route(self.d, self.gate_q, self.gate_s, self.sgate_q, self.sgate_s, x, b["T"], bias,
                    b["idx"], b["w"], b["sw"], b["logits"], b["counts"], b["offsets"], b["perm"],
                    b["ws"], stream)

    def experts_forward(self, x, b, routed=None, stream=None):
        B.moe_expert_forward(self.d, routed or self.experts, self.shared_blob, x, b["T"],
                             b["idx"], b["counts"], b["offsets"], b["perm"], b["y"], b["ws"],
                             stream)

    def combine(self, b, residual=None, norm_out=None, eps=1e-6, stream=None):
        B.moe_combine(self.d, b["y"], b["w"], b["sw"], b["T"], residual, b["out"], norm_out, eps,
                      stream)

    def forward(self, x, b, bias=None, residual=None, norm_out=None, eps=1e-6, routed=None,
                stream=None):
        self.route(x, b, bias, stream)
        self.experts_forward(x, b, routed, stream)
        self.combine(b, residual, norm_out, eps, stream)
        return b["out"]

    # ---- one-call prefill block ----------------------------------------
    def block_prefill_buffers(self, T: int) -> dict:
        dv = self.device
        return {
            "T": T,
            "ws": torch.empty((max(B.moe_block_prefill_workspace_bytes(self.d, T), 1),),
                              dtype=torch.uint8, device=dv),
            "idx": torch.empty((T, self.K), dtype=torch.int32, device=dv),
            "w": torch.empty((T, self.K), dtype=torch.float32, device=dv),
            "out": torch.empty((T, self.H), dtype=torch.int16, device=dv),
        }

    def block_prefill(self, x, pb, bias=None, residual=None, norm_out=None, eps=1e-6,
                      routed=None, stream=None):
        """moe_block_prefill: route + experts + combine in one call, the
        expert outputs kept compact in the workspace."""
        B.moe_block_prefill(self.d, self.gate_q, self.gate_s, self.sgate_q, self.sgate_s, bias,
                            routed or self.experts, self.shared_blob, x, pb["T"], residual,
                            pb["idx"], pb["w"], pb["out"], norm_out, eps, pb["ws"], stream)
        return pb["out"]

    # ---- fused single-launch decode -----------------------------------
    def fused_buffers(self, T: int) -> dict:
        dv = self.device
        ws = torch.empty((B.moe_block_decode_workspace_bytes(self.d, T),),
                         dtype=torch.uint8, device=dv)
        B.moe_workspace_init(ws)
        return {
            "T": T,
            "ws": ws,
            "idx": torch.empty((T, self.K), dtype=torch.int32, device=dv),
            "w": torch.empty((T, self.K), dtype=torch.float32, device=dv),
            "out": torch.empty((T, self.H), dtype=torch.int16, device=dv),
        }

    def decode_fused(self, h_in, fb, flags=0, eps=1e-6, out=None, routed=None, stream=None,
                     exec_idx=None):
        """One kernel launch: route + experts + combine (+ norm / residual).
        exec_idx: device int32 [T, K] experts to execute instead of the top-K."""
        out = fb["out"] if out is None else out
        args = (self.d, self.gate_q, self.gate_s, self.sgate_q, self.sgate_s,
                routed or self.experts, self.shared_blob, h_in, fb["T"], flags, eps)
        if exec_idx is None:
            B.moe_block_decode(*args, fb["idx"], fb["w"], out, fb["ws"], stream)
        else:
            B.moe_block_decode_exec(*args, exec_idx, fb["idx"], fb["w"], out, fb["ws"], stream)
        return out

    @staticmethod
    def fused_error_word(fb) -> int:
        """Sticky timeout flag of the fused kernel (0 = every wait completed)."""
        o = B.DECODE_ERR_OFFSET
        return int(fb["ws"][o:o + 4].view(torch.int32).item())


class MoeStack:
    """A decode stack of MoE layers, one token step at a time.

    Layer l computes h <- h + MoE_l(RMSNorm(h)) in one fused launch.  With
    Prerouter heads, head l reads layer l's output and predicts the experts
    of layer l + 1 for the next step ([P2] Prerouter paragraph: predictions
    cross one layer and one token and are committed at the step boundary).
    With a pool, routed experts live in per-layer HBM slots fed from a pinned
    host master copy; `end_step` commits the step (executed + predicted
    experts) to the pool, whose fills then overlap the next step.

    exec_mode "router": every layer executes its router's top-K (the
    predictions only steer the pool).  "predict" (prediction-as-routing,
    [P3] "三件套" Prerouter bullet): layers 1 .. L-1 execute the experts that
    the previous step's heads predicted for them, weighted by their router's
    logits; with a pool, such a layer waits for its fills, so those experts
    are read from HBM.  Layer 0, and every layer of the first step, route.

    routers: per layer dict(router_q, router_s, sgate_q, sgate_s);
    shared_blobs: device uint8 [L, blob] or None; routed: device uint8
    [L, E, blob] (all resident) or None with `host_blobs` (pinned uint8
    [L, E, blob]) and `pool_slots`; prerouter: per-layer (W1, W2) device bf16
    for layers 0 .. L-2, or None.  With prerouter_feat, W1 is [D, H + E] and
    each head also sees the experts its layer executed (routing features,
    [P2] Prerouter paragraph).
    """

    def __init__(self, H, I, E, K, r, n_shared, lora_scale, routers, shared_blobs, routed=None,
                 host_blobs=None, pool_slots=0, prerouter=None, pred_k=0, eps=1e-6,
                 max_fills=-1, exec_mode="router", prerouter_feat=False, overlap_heads=False,
                 device="cuda"):
        self.H, self.I, self.E, self.K, self.r, self.S = H, I, E, K, r, n_shared
        self.L = len(routers)
        self.d = B.dims(H, I, E, K, r, n_shared, lora_scale, 1)
        self.eps, self.device, self.max_fills = eps, device, max_fills
        self.blob_bytes = B.moe_expert_blob_bytes(H, I, r)
        dv = device
        self.routers = [{k: dev(v.reshape(-1) if k.startswith("sgate") else v, dv)
                         for k, v in R.items()} for R in routers]
        self.shared = shared_blobs
        self.pool = None
        self.counters = torch.zeros((self.L, 2), dtype=torch.int64, device=dv)
        if routed is not None:
            self.routed = routed
            self.experts = [B.experts_struct(routed[l], E) for l in range(self.L)]
        else:
            assert host_blobs is not None and pool_slots > 0
            self.routed = None
            self.host_blobs = host_blobs
            self.slots = torch.empty((self.L, pool_slots, self.blob_bytes), dtype=torch.uint8, device=dv)
            self.table = torch.empty((self.L, E), dtype=torch.int32, device=dv)
            self.side = torch.cuda.Stream(device=dv)
            self.pool = B.MoePool(self.L, E, pool_slots, self.blob_bytes, self.slots, self.table,
                                  host_blobs)
            self.experts = [self.pool.layer(l, self.counters[l]) for l in range(self.L)]
        self.prerouter = prerouter
        self.prerouter_feat = prerouter_feat
        self.pred_k = pred_k
        # overlap_heads: each Prerouter head runs on a stream of its own after
        # its layer's kernel, overlapping the next layer (default priority, like
        # every stream here).  It costs four event calls per layer on the host,
        # more than the head's GPU time in an eagerly issued step, so it is for
        # steps captured in a graph; by default heads run between the layers.
        self.overlap_heads = overlap_heads and prerouter is not None
        if self.overlap_heads:
            self.head_stream = torch.cuda.Stream(device=dv)
            self.ev_out = [torch.cuda.Event() for _ in range(self.L)]
            self.ev_head = [torch.cuda.Event() for _ in range(self.L)]
        self.exec_mode = "router"
        self.have_pred = False
        T = 1
        self.ws = torch.empty((B.moe_block_decode_workspace_bytes(self.d, T),), dtype=torch.uint8,
                              device=dv)
        B.moe_workspace_init(self.ws)
        self.idx = torch.empty((self.L, T, K), dtype=torch.int32, device=dv)
        self.w = torch.empty((self.L, T, K), dtype=torch.float32, device=dv)
        self.h = [torch.empty((T, H), dtype=torch.int16, device=dv) for _ in range(2)]
        if prerouter is not None:
            D = prerouter[0][0].shape[0]
            # zeroed once: the head's launch counter lives there
            self.pr_ws = torch.zeros((B.prerouter_workspace_bytes(D, E, T),), dtype=torch.uint8,
                                     device=dv)
            self.pred = torch.full((self.L, T, pred_k), -1, dtype=torch.int32, device=dv)
            self.pred_exec = torch.full((self.L, T, pred_k), -1, dtype=torch.int32, device=dv)
        # step-boundary copies for the pool planner
        self.idx_host = torch.empty((self.L, K), dtype=torch.int32, pin_memory=True)
        self.pred_host = torch.full((self.L, max(pred_k, 1)), -1, dtype=torch.int32,
                                    pin_memory=True)
        self.done = torch.cuda.Event()
        self.set_exec_mode(exec_mode)

    def set_exec_mode(self, mode: str):
        """Switch between router-executed and prediction-as-routing steps."""
        if mode not in ("router", "predict"):
            raise ValueError(f"exec_mode must be 'router' or 'predict', not {mode!r}")
        if mode == "predict" and (self.prerouter is None or self.pred_k != self.K):
            raise ValueError("prediction-as-routing needs Prerouter heads with pred_k == K")
        self.exec_mode = mode
        self.have_pred = False

    def set_read_delay(self, ns: int):
        """Modeled storage latency of the pool's master copy (see moe.h)."""
        self.pool.set_read_delay(ns)
        self.experts = [self.pool.layer(l, self.counters[l]) for l in range(self.L)]

    def layer_forward(self, l, h_in, out, stream=None):
        R = self.routers[l]
        given = self.exec_mode == "predict" and self.have_pred and l > 0
        if self.pool is not None:
            if given:
                self.pool.wait_layer_filled(l, stream)
            else:
                self.pool.wait_layer(l, stream)
        args = (self.d, R["router_q"], R["router_s"], R.get("sgate_q"), R.get("sgate_s"),
                self.experts[l], self.shared[l] if self.S else None, h_in, 1,
                B.DECODE_NORM_INPUT | B.DECODE_RESIDUAL, self.eps)
        if given:
            B.moe_block_decode_exec(*args, self.pred_exec[l], self.idx[l], self.w[l], out,
                                    self.ws, stream)
        else:
            B.moe_block_decode(*args, self.idx[l], self.w[l], out, self.ws, stream)

    @staticmethod
    def _torch_stream(stream):
        if stream is None:
            return torch.cuda.current_stream()
        if isinstance(stream, int):
            return torch.cuda.ExternalStream(stream) if stream else torch.cuda.default_stream()
        return stream

    def step(self, x, stream=None, outs=None):
        """One token through every layer; returns the output hidden state.
        outs: optional per-layer output buffers (default: two alternating).
        Every kernel of the step, heads included, is ordered before work issued
        later on `stream`."""
        s = self._torch_stream(stream)
        hs = self.head_stream if self.overlap_heads else s
        cur = x
        for l in range(self.L):
            out = self.h[l % 2] if outs is None else outs[l]
            if self.overlap_heads and outs is None and l >= 2:
                s.wait_event(self.ev_head[l - 2])  # head l-2 has read this buffer
            self.layer_forward(l, cur, out, s)
            if self.prerouter is not None and l + 1 < self.L:
                if self.overlap_heads:
                    self.ev_out[l].record(s)
                    hs.wait_event(self.ev_out[l])
                W1, W2 = self.prerouter[l]
                if self.prerouter_feat:  # h plus the one-hot of this layer's executed experts
                    B.prerouter_predict_feat(W1, W2, self.H, W1.shape[0], self.E, self.pred_k, out,
                                             self.idx[l], self.K, 1, self.pred[l + 1], None,
                                             self.pr_ws, hs)
                else:
                    B.prerouter_predict(W1, W2, self.H, W1.shape[0], self.E, self.pred_k, out, 1,
                                        self.pred[l + 1], None, self.pr_ws, hs)
                if self.overlap_heads:
                    self.ev_head[l].record(hs)
            cur = out
        if self.overlap_heads:
            s.wait_stream(hs)
        if self.exec_mode == "predict":
            # this step's predictions are the next step's routes
            with torch.cuda.stream(s):
                self.pred_exec.copy_(self.pred)
            self.have_pred = True
        return cur

    def end_step(self, stream=None):
        """Commit the step to the pool (no-op without a pool): waits for the
        step's kernels, then plans and enqueues the fills on the side stream."""
        if self.pool is None:
            return 0
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            self.idx_host.copy_(self.idx.view(self.L, self.K), non_blocking=True)
            if self.prerouter is not None:
                self.pred_host.copy_(self.pred.view(self.L, self.pred_k), non_blocking=True)
        self.done.record(s)
        self.done.synchronize()
        pred = self.pred_host.numpy() if self.prerouter is not None else None
        return self.pool.update(self.idx_host.numpy(), pred, self.max_fills, self.side)

    def error_word(self) -> int:
        """Sticky timeout flag shared by every layer's fused launch (0 = every
        wait of every step completed).  Reading it synchronises."""
        o = B.DECODE_ERR_OFFSET
        return int(self.ws[o:o + 4].view(torch.int32).item())

    def hit_counts(self):
        """(lookups served from a slot, all lookups) summed over layers."""
        c = self.counters.sum(0).tolist()
        return int(c[0]), int(c[1])
