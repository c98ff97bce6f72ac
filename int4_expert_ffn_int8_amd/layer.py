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
                 shared: dict | None, norm_topk: int = 1, device="cuda", blobs=None):
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
        self.shared_blob = dev(pack_experts(H, I, r, [shared])[0], device) if n_shared else None
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

    def decode_fused(self, h_in, fb, flags=0, eps=1e-6, out=None, routed=None, stream=None):
        """One kernel launch: route + experts + combine (+ norm / residual)."""
        out = fb["out"] if out is None else out
        B.moe_block_decode(self.d, self.gate_q, self.gate_s, self.sgate_q, self.sgate_s,
                           routed or self.experts, self.shared_blob, h_in, fb["T"], flags, eps,
                           fb["idx"], fb["w"], out, fb["ws"], stream)
        return out

    @staticmethod
    def fused_error_word(fb) -> int:
        """Sticky timeout flag of the fused kernel (0 = every wait completed)."""
        o = B.DECODE_ERR_OFFSET
        return int(fb["ws"][o:o + 4].view(torch.int32).item())
