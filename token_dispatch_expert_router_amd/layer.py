"""One MoE layer, forward then backward, as a sequence of C-ABI calls.

MoELayer owns the device buffers of one layer shape (torch allocations: torch is
the allocator and the stream provider, nothing more) and runs

    moe_route -> moe_permute -> moe_expert_ffn_fwd (+ shared expert) -> moe_unpermute
    -> moe_unpermute_bwd -> moe_expert_ffn_bwd (+ shared) -> moe_route_bwd -> moe_permute_bwd

on one stream with no host synchronisation ("MoE Parallel Folding", arXiv
2504.14960, knowledge-base notes page, method paragraph: route, permute, expert FFN,
un-permute, and the duals in the backward pass; the cross-GPU exchanges are not part
of a one-GPU layer).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, T: int, d: int, E: int, K: int, f: int, sub_seq: int, capacity: int,
                 dtype: torch.dtype, fs: int = 0, device="cuda", flags: int = 0):
        if dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("dtype must be float32 or bfloat16")
        self.T, self.d, self.E, self.K, self.f, self.fs = T, d, E, K, f, fs
        self.dtype = dtype
        self.device = torch.device(device)
        code = L.MOE_F32 if dtype == torch.float32 else L.MOE_BF16
        self.desc = L.make_desc(T, d, E, K, f, sub_seq, capacity, code, flags)
        self.R = L.moe_max_rows(self.desc)
        self.sdesc = L.make_desc(T, d, 1, 1, fs, max(T, 1), -1, code, flags) if fs else None
        dev, dt = self.device, dtype
        i32, f32 = torch.int32, torch.float32
        R1 = max(self.R, 1)
        n_sub = T // sub_seq if sub_seq else 0

        def z(shape, t):
            return torch.zeros(shape, dtype=t, device=dev)

        self.rt = {
            "topk_idx": z((T, K), i32), "topk_prob": z((T, K), f32), "topk_gate": z((T, K), f32),
            "keep": z((T, K), torch.uint8), "row_of": z((T, K), i32), "src_of": z((R1,), i32),
            "routed_counts": z((max(n_sub, 1), E), i32), "kept_counts": z((E,), i32),
            "offsets": z((E + 1,), i32), "n_kept": z((1,), i32),
        }
        self.routing = L.make_routing(self.rt)
        b = {}
        b["logits"] = z((T, E), f32)
        b["sg_logit"] = z((T,), f32) if fs else None
        b["xp"] = z((R1, d), dt)
        for n in ("a", "b", "h"):
            b[n] = z((R1, f), dt)
        b["o"] = z((R1, d), dt)
        b["y"] = z((T, d), dt)
        b["d_o"] = z((R1, d), dt)
        b["dgate"] = z((T, K), f32)
        b["dxp"] = z((R1, d), dt)
        b["dw_gate"] = z((E, d, f), dt)
        b["dw_up"] = z((E, d, f), dt)
        b["dw_down"] = z((E, f, d), dt)
        b["dlogits"] = z((T, E), f32)
        b["dw_router"] = z((d, E), dt)
        b["dx"] = z((T, d), dt)
        if fs:
            for n in ("sa", "sb", "sh"):
                b[n] = z((T, fs), dt)
            b["shared"] = z((T, d), dt)
            b["dshared"] = z((T, d), dt)
            b["dz"] = z((T,), f32)
            b["dx_shared"] = z((T, d), dt)
            b["dws_gate"] = z((1, d, fs), dt)
            b["dws_up"] = z((1, d, fs), dt)
            b["dws_down"] = z((1, fs, d), dt)
            b["dw_sg"] = z((d,), dt)
            b["shared_offsets"] = torch.tensor([0, T], dtype=i32, device=dev)
        self.buf = b

        def ws(desc, which):
            n = L.moe_workspace_size(desc, which)
            return torch.empty((max(n, 1),), dtype=torch.uint8, device=dev) if n else None

        self.ws_route = ws(self.desc, L.MOE_WS_ROUTE)
        n_ffn = L.moe_workspace_size(self.desc, L.MOE_WS_FFN_BWD)
        if fs:
            n_ffn = max(n_ffn, L.moe_workspace_size(self.sdesc, L.MOE_WS_FFN_BWD))
        self.ws_ffn = torch.empty((max(n_ffn, 1),), dtype=torch.uint8, device=dev)
        self.ws_route_bwd = ws(self.desc, L.MOE_WS_ROUTE_BWD)
        self.ws_permute_bwd = ws(self.desc, L.MOE_WS_PERMUTE_BWD)

    # ------------------------------------------------------------------------------
    def route(self, inp: dict, stream=None, logits: Optional[torch.Tensor] = None):
        if logits is not None:
            L.moe_route_from_logits(self.desc, logits, self.routing, self.ws_route, stream)
            return
        b = self.buf
        L.moe_route(self.desc, inp["x"], inp["w_router"], inp.get("bias"), inp.get("w_sg"),
                    b["logits"], b["sg_logit"], self.routing, self.ws_route, stream)

    def forward(self, inp: dict, stream=None, logits: Optional[torch.Tensor] = None):
        b, rt = self.buf, self.rt
        if logits is not None and self.fs:
            # the shared gate logit still comes from moe_route's extra column
            raise ValueError("external logits are not supported with a shared expert")
        self.route(inp, stream, logits)
        L.moe_permute(self.desc, inp["x"], self.routing, b["xp"], stream)
        L.moe_expert_ffn_fwd(self.desc, b["xp"], inp["w_gate"], inp["w_up"], inp["w_down"],
                             rt["offsets"], b["a"], b["b"], b["h"], b["o"], None, stream)
        if self.fs:
            L.moe_expert_ffn_fwd(self.sdesc, inp["x"], inp["ws_gate"], inp["ws_up"],
                                 inp["ws_down"], b["shared_offsets"], b["sa"], b["sb"], b["sh"],
                                 b["shared"], None, stream)
        L.moe_unpermute(self.desc, b["o"], self.routing, b.get("shared"), b["sg_logit"], b["y"],
                        stream)

    def backward(self, inp: dict, stream=None):
        b, rt = self.buf, self.rt
        fs = self.fs
        L.moe_unpermute_bwd(self.desc, inp["dy"], b["o"], self.routing, b.get("shared"),
                            b["sg_logit"], b["d_o"], b["dgate"], b.get("dshared"), b.get("dz"),
                            stream)
        L.moe_expert_ffn_bwd(self.desc, b["xp"], b["a"], b["b"], b["h"], inp["w_gate"],
                             inp["w_up"], inp["w_down"], rt["offsets"], b["d_o"], b["dxp"],
                             b["dw_gate"], b["dw_up"], b["dw_down"], self.ws_ffn, stream)
        if fs:
            L.moe_expert_ffn_bwd(self.sdesc, inp["x"], b["sa"], b["sb"], b["sh"], inp["ws_gate"],
                                 inp["ws_up"], inp["ws_down"], b["shared_offsets"], b["dshared"],
                                 b["dx_shared"], b["dws_gate"], b["dws_up"], b["dws_down"],
                                 self.ws_ffn, stream)
        L.moe_route_bwd(self.desc, inp["x"], self.routing, b["dgate"], b.get("dz"), b["dlogits"],
                        b["dw_router"], b.get("dw_sg"), self.ws_route_bwd, stream)
        L.moe_permute_bwd(self.desc, b["dxp"], self.routing, b["dlogits"], inp["w_router"],
                          b.get("dz"), inp.get("w_sg"), b.get("dx_shared"), b["dx"],
                          self.ws_permute_bwd, stream)

    def forward_backward(self, inp: dict, stream=None, logits: Optional[torch.Tensor] = None):
        self.forward(inp, stream, logits)
        self.backward(inp, stream)


class Dispatch:
    """Routing and permutation alone (moe_route -> moe_permute): the rows one GPU sends
    into the expert-parallel exchange, expert-major."""

    def __init__(self, T: int, d: int, E: int, K: int, sub_seq: int, capacity: int,
                 dtype: torch.dtype, device="cuda"):
        code = L.MOE_F32 if dtype == torch.float32 else L.MOE_BF16
        self.desc = L.make_desc(T, d, E, K, 8, sub_seq, capacity, code, 0)
        self.R = L.moe_max_rows(self.desc)
        dev, i32, f32 = torch.device(device), torch.int32, torch.float32
        R1 = max(self.R, 1)

        def z(shape, t):
            return torch.zeros(shape, dtype=t, device=dev)

        self.rt = {
            "topk_idx": z((T, K), i32), "topk_prob": z((T, K), f32), "topk_gate": z((T, K), f32),
            "keep": z((T, K), torch.uint8), "row_of": z((T, K), i32), "src_of": z((R1,), i32),
            "routed_counts": z((max(T // sub_seq, 1), E), i32), "kept_counts": z((E,), i32),
            "offsets": z((E + 1,), i32), "n_kept": z((1,), i32),
        }
        self.routing = L.make_routing(self.rt)
        self.logits = z((T, E), f32)
        self.xp = z((R1, d), dtype)
        n = L.moe_workspace_size(self.desc, L.MOE_WS_ROUTE)
        self.ws = torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)

    def run(self, x, w_router, bias=None, stream=None):
        L.moe_route(self.desc, x, w_router, bias, None, self.logits, None, self.routing, self.ws,
                    stream)
        L.moe_permute(self.desc, x, self.routing, self.xp, stream)


class ExpertShard:
    """The expert FFN, forward and backward, on the rows one GPU's experts receive.

    Under expert parallelism the GPU holds E experts (a contiguous range) and gets their
    rows from every source GPU; under expert-tensor parallelism it holds an f-slice of
    each expert and its o and dxp are partial sums that the ReduceScatter-V of the
    exchange adds up ("MoE Parallel Folding", knowledge-base notes page, method
    paragraph).  `partial` keeps those two outputs in float32 (MOE_FLAG_F32_PARTIAL).
    """

    def __init__(self, rows: int, d: int, E: int, f: int, dtype: torch.dtype,
                 partial: bool = False, device="cuda", flags: int = 0):
        code = L.MOE_F32 if dtype == torch.float32 else L.MOE_BF16
        if partial:
            flags |= L.MOE_FLAG_F32_PARTIAL
        self.desc = L.make_desc(rows, d, E, 1, f, max(rows, 1), -1, code, flags)
        self.rows, self.d, self.E, self.f = rows, d, E, f
        dev = torch.device(device)
        R1 = max(rows, 1)
        out_t = torch.float32 if partial else dtype

        def z(shape, t):
            return torch.zeros(shape, dtype=t, device=dev)

        self.buf = {"a": z((R1, f), dtype), "b": z((R1, f), dtype), "h": z((R1, f), dtype),
                    "o": z((R1, d), out_t), "dxp": z((R1, d), out_t),
                    "dw_gate": z((E, d, f), dtype), "dw_up": z((E, d, f), dtype),
                    "dw_down": z((E, f, d), dtype)}
        n = L.moe_workspace_size(self.desc, L.MOE_WS_FFN_BWD)
        self.ws = torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)

    def forward(self, xp, w: dict, offsets, stream=None):
        b = self.buf
        L.moe_expert_ffn_fwd(self.desc, xp, w["w_gate"], w["w_up"], w["w_down"], offsets,
                             b["a"], b["b"], b["h"], b["o"], None, stream)

    def backward(self, xp, w: dict, offsets, d_o, stream=None):
        b = self.buf
        L.moe_expert_ffn_bwd(self.desc, xp, b["a"], b["b"], b["h"], w["w_gate"], w["w_up"],
                             w["w_down"], offsets, d_o, b["dxp"], b["dw_gate"], b["dw_up"],
                             b["dw_down"], self.ws, stream)


def expert_rows(dp: Dispatch, e0: int, e1: int):
    """The permuted rows of experts [e0, e1) (a view of dp.xp, they are contiguous) and
    their offsets from 0.  Reads the offsets on the host: a set-up step, it synchronises."""
    offs = dp.rt["offsets"].to("cpu", torch.int64)
    lo, hi = int(offs[e0]), int(offs[e1])
    loc = (offs[e0:e1 + 1] - lo).to(device=dp.xp.device, dtype=torch.int32)
    return dp.xp[lo:hi], loc
