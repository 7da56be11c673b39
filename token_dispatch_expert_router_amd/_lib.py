"""ctypes binding of libmoe.so: the C ABI of include/moe.h, one Python function per
entry point, with the same names.  Arguments are torch tensors (device memory) and
an optional torch stream; this module only marshals pointers and sizes and raises
MoeError on a non-zero status.  Nothing here computes: every step runs in the HIP
kernels of libmoe.so, and importing the functions fails loudly when it is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1
MOE_FLAG_VALU_GEMM = 1
MOE_FLAG_F32_PARTIAL = 2
MOE_WS_ROUTE, MOE_WS_FFN_FWD, MOE_WS_FFN_BWD, MOE_WS_ROUTE_BWD, MOE_WS_PERMUTE_BWD = range(5)

EXPORTS = [
    "moe_abi_version", "moe_last_error", "moe_capacity", "moe_max_rows", "moe_workspace_size",
    "moe_route", "moe_route_noalloc", "moe_route_from_logits", "moe_permute", "moe_expert_ffn_fwd", "moe_unpermute",
    "moe_unpermute_bwd", "moe_expert_ffn_bwd", "moe_route_bwd", "moe_permute_bwd",
]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("f", ctypes.c_int32), ("sub_seq", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_prob", "topk_gate", "keep", "row_of", "src_of",
                 "routed_counts", "kept_counts", "offsets", "n_kept")]


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m token_dispatch_expert_router_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    D = ctypes.POINTER(Desc)
    R = ctypes.POINTER(Routing)
    lib.moe_abi_version.restype = i32
    lib.moe_abi_version.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_capacity.restype = i32
    lib.moe_capacity.argtypes = [i32, i32, i32, ctypes.c_double]
    lib.moe_max_rows.restype = ctypes.c_int64
    lib.moe_max_rows.argtypes = [D]
    lib.moe_workspace_size.restype = sz
    lib.moe_workspace_size.argtypes = [D, i32]
    sigs = {
        "moe_route": [D, vp, vp, vp, vp, vp, vp, R, vp, sz, vp],
        "moe_route_noalloc": [D, vp, vp, vp, vp, vp, vp, R, vp],
        "moe_route_from_logits": [D, vp, R, vp, sz, vp],
        "moe_permute": [D, vp, R, vp, vp],
        "moe_expert_ffn_fwd": [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_unpermute": [D, vp, R, vp, vp, vp, vp],
        "moe_unpermute_bwd": [D, vp, vp, R, vp, vp, vp, vp, vp, vp, vp],
        "moe_expert_ffn_bwd": [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_route_bwd": [D, vp, R, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute_bwd": [D, vp, R, vp, vp, vp, vp, vp, vp, vp, sz, vp],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.restype = i32
        fn.argtypes = args
    _lib = lib
    return lib


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int):
    if status != 0:
        raise MoeError(status, load().moe_last_error().decode())


def make_desc(T, d, E, K, f, sub_seq, capacity, dtype, flags=0) -> Desc:
    return Desc(T, d, E, K, f, sub_seq, capacity, dtype, flags)


def make_routing(bufs: dict) -> Routing:
    return Routing(*[_p(bufs[n]) for n, _ in Routing._fields_])


def ws_bytes(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


# ---- host helpers -------------------------------------------------------------------

def moe_abi_version() -> int:
    return load().moe_abi_version()


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def moe_capacity(S: int, K: int, E: int, cf: float) -> int:
    return load().moe_capacity(S, K, E, float(cf))


def moe_max_rows(desc: Desc) -> int:
    v = load().moe_max_rows(ctypes.byref(desc))
    if v < 0:
        raise MoeError(-1, moe_last_error())
    return v


def moe_workspace_size(desc: Desc, which: int) -> int:
    v = load().moe_workspace_size(ctypes.byref(desc), which)
    if v == ctypes.c_size_t(-1).value:
        raise MoeError(-1, moe_last_error())
    return v


# ---- device calls ---------------------------------------------------------------------

def moe_route(desc, x, w_router, bias, w_sg, logits, sg_logit, routing: Routing, ws, stream=None):
    _check(load().moe_route(ctypes.byref(desc), _p(x), _p(w_router), _p(bias), _p(w_sg),
                            _p(logits), _p(sg_logit), ctypes.byref(routing), _p(ws),
                            ws_bytes(ws), _stream(stream)))


def moe_route_noalloc(desc, x, w_router, bias, w_sg, logits, sg_logit, routing: Routing,
                      stream=None):
    _check(load().moe_route_noalloc(ctypes.byref(desc), _p(x), _p(w_router), _p(bias), _p(w_sg),
                                    _p(logits), _p(sg_logit), ctypes.byref(routing),
                                    _stream(stream)))


MOE_ROUTE_SCRATCH_BYTES = 16 << 20


def moe_route_from_logits(desc, logits, routing: Routing, ws, stream=None):
    _check(load().moe_route_from_logits(ctypes.byref(desc), _p(logits), ctypes.byref(routing),
                                        _p(ws), ws_bytes(ws), _stream(stream)))


def moe_permute(desc, x, routing: Routing, xp, stream=None):
    _check(load().moe_permute(ctypes.byref(desc), _p(x), ctypes.byref(routing), _p(xp),
                              _stream(stream)))


def moe_expert_ffn_fwd(desc, xp, w_gate, w_up, w_down, offsets, a, b, h, o, ws=None,
                       stream=None):
    _check(load().moe_expert_ffn_fwd(ctypes.byref(desc), _p(xp), _p(w_gate), _p(w_up),
                                     _p(w_down), _p(offsets), _p(a), _p(b), _p(h), _p(o),
                                     _p(ws), ws_bytes(ws), _stream(stream)))


def moe_unpermute(desc, o, routing: Routing, shared, sg_logit, y, stream=None):
    _check(load().moe_unpermute(ctypes.byref(desc), _p(o), ctypes.byref(routing), _p(shared),
                                _p(sg_logit), _p(y), _stream(stream)))


def moe_unpermute_bwd(desc, dy, o, routing: Routing, shared, sg_logit, d_o, dgate, dshared,
                      dsg_logit, stream=None):
    _check(load().moe_unpermute_bwd(ctypes.byref(desc), _p(dy), _p(o), ctypes.byref(routing),
                                    _p(shared), _p(sg_logit), _p(d_o), _p(dgate), _p(dshared),
                                    _p(dsg_logit), _stream(stream)))


def moe_expert_ffn_bwd(desc, xp, a, b, h, w_gate, w_up, w_down, offsets, d_o, dxp, dw_gate,
                       dw_up, dw_down, ws, stream=None):
    _check(load().moe_expert_ffn_bwd(ctypes.byref(desc), _p(xp), _p(a), _p(b), _p(h),
                                     _p(w_gate), _p(w_up), _p(w_down), _p(offsets), _p(d_o),
                                     _p(dxp), _p(dw_gate), _p(dw_up), _p(dw_down), _p(ws),
                                     ws_bytes(ws), _stream(stream)))


def moe_route_bwd(desc, x, routing: Routing, dgate, dsg_logit, dlogits, dw_router, dw_sg, ws,
                  stream=None):
    _check(load().moe_route_bwd(ctypes.byref(desc), _p(x), ctypes.byref(routing), _p(dgate),
                                _p(dsg_logit), _p(dlogits), _p(dw_router), _p(dw_sg), _p(ws),
                                ws_bytes(ws), _stream(stream)))


def moe_permute_bwd(desc, dxp, routing: Routing, dlogits, w_router, dsg_logit, w_sg, dx_add,
                    dx, ws, stream=None):
    _check(load().moe_permute_bwd(ctypes.byref(desc), _p(dxp), ctypes.byref(routing),
                                  _p(dlogits), _p(w_router), _p(dsg_logit), _p(w_sg),
                                  _p(dx_add), _p(dx), _p(ws), ws_bytes(ws), _stream(stream)))
