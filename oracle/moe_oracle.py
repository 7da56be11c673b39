"""CPU oracle for one GPU's MoE layer, forward and backward.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module; the product path never does.  It shares no
code with the HIP library: routing runs in the plain C file next to this one, the
rest is numpy in float64.

What it computes ("MoE Parallel Folding", arXiv 2504.14960, knowledge-base notes
page, method paragraph: router Top-K -> permutation so one expert's tokens are
contiguous -> expert FFN -> un-permutation back to token order; Section 3.3 Token
Dispatcher quote: sub-sequence dropping is the default token-drop strategy).
Without the cross-GPU exchanges this is exactly the sparsely-gated MoE layer

    y_t = sum_{k kept} g_tk * FFN_{e_tk}(x_t)   (+ sigmoid(x_t . w_sg) * F_sh(x_t))
    FFN_e(x) = (silu(x W_g,e) * (x W_u,e)) W_d,e

and the backward pass is its vector-Jacobian product with the routing decisions
held fixed.  The steps are written out (route, permute, grouped FFN, un-permute)
because the discrete routing must match the device bit for bit, and because the
device stores some intermediates in bf16: `storage` rounds the values the device
stores ("bf16", "f32") at the same points, "f64" stores nothing rounded.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "route_oracle.c")
_lib = None


def build_oracle(force: bool = False) -> str:
    """Compile the C part of the oracle (gcc, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build_oracle()
        lib = ctypes.CDLL(_SO)
        lib.oracle_exp.restype = ctypes.c_float
        lib.oracle_exp.argtypes = [ctypes.c_float]
        lib.oracle_pairwise_sum.restype = ctypes.c_float
        lib.oracle_pairwise_sum.argtypes = [ctypes.c_void_p, ctypes.c_int]
        lib.oracle_softmax_row.restype = None
        lib.oracle_softmax_row.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.oracle_capacity.restype = ctypes.c_int
        lib.oracle_capacity.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_route.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 11
        lib.oracle_exp_scan.restype = ctypes.c_double
        lib.oracle_exp_scan.argtypes = [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------------
# Routing (fp32, bit-exact decisions): thin wrappers over the C file.
# ----------------------------------------------------------------------------------

def exp32(r: float) -> float:
    return float(_load().oracle_exp(ctypes.c_float(r)))


def pairwise_sum32(v) -> float:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return float(_load().oracle_pairwise_sum(_ptr(v), v.size))


def softmax32(logits) -> np.ndarray:
    """Row softmax in fp32 with the oracle's exp and pairwise sum (one row or [T,E])."""
    l = np.ascontiguousarray(np.atleast_2d(logits), dtype=np.float32)
    out = np.empty_like(l)
    lib = _load()
    for t in range(l.shape[0]):
        lib.oracle_softmax_row(_ptr(l[t]), l.shape[1], _ptr(out[t]))
    return out


def capacity(S: int, K: int, E: int, cf) -> int:
    """ceil(cf*S*K/E) in double; None (or a negative cf) means dropless (-1)."""
    if cf is None:
        return -1
    return int(_load().oracle_capacity(S, K, E, float(cf)))


def exp_scan(lo: float = -88.0):
    n = np.zeros(1, np.int64)
    bf = np.zeros(1, np.int64)
    nm = np.zeros(1, np.int64)
    worst = _load().oracle_exp_scan(ctypes.c_float(lo), _ptr(n), _ptr(bf), _ptr(nm))
    return worst, int(n[0]), int(bf[0]), int(nm[0])


def route(logits, K: int, S: int, capacity: int) -> dict:
    """Softmax top-K routing, capacity drop per (sub-sequence, expert), and the maps.

    logits: [T, E] float32.  capacity < 0 means dropless.
    Returns numpy arrays: topk_idx, topk_prob, topk_gate, keep, row_of [T,K];
    src_of [n_kept]; routed_counts [T/S, E]; kept_counts [E]; offsets [E+1]; n_kept.
    """
    l = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = l.shape
    if T % S != 0:
        raise ValueError("T must be a multiple of the sub-sequence length")
    out = {
        "topk_idx": np.zeros((T, K), np.int32),
        "topk_prob": np.zeros((T, K), np.float32),
        "topk_gate": np.zeros((T, K), np.float32),
        "keep": np.zeros((T, K), np.uint8),
        "row_of": np.zeros((T, K), np.int32),
        "src_of": np.zeros(max(T * K, 1), np.int32),
        "routed_counts": np.zeros((max(T // S, 1), E), np.int32),
        "kept_counts": np.zeros(E, np.int32),
        "offsets": np.zeros(E + 1, np.int32),
        "n_kept": np.zeros(1, np.int32),
    }
    rc = _load().oracle_route(T, E, K, S, capacity, _ptr(l), _ptr(out["topk_idx"]),
                              _ptr(out["topk_prob"]), _ptr(out["topk_gate"]),
                              _ptr(out["keep"]), _ptr(out["row_of"]), _ptr(out["src_of"]),
                              _ptr(out["routed_counts"]), _ptr(out["kept_counts"]),
                              _ptr(out["offsets"]), _ptr(out["n_kept"]))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    n = int(out["n_kept"][0])
    out["n_kept"] = n
    out["src_of"] = out["src_of"][:n].copy()
    if T // S == 0:
        out["routed_counts"] = out["routed_counts"][:0]
    return out


# ----------------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------------

def round_bf16(a) -> np.ndarray:
    """Round to bfloat16 (through fp32, round-to-nearest-even) and return float64."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def store(a, storage: str) -> np.ndarray:
    if storage == "bf16":
        return round_bf16(a)
    if storage == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if storage == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(storage)


def store_fp32(a, storage: str) -> np.ndarray:
    """Values the device always keeps in fp32 (gates' gradients, logits' gradients)."""
    if storage == "f64":
        return np.asarray(a, dtype=np.float64)
    return np.asarray(a, dtype=np.float32)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(a):
    return a / (1.0 + np.exp(-a))


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


# ----------------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------------

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """logits = x W_r (+ b), accumulated in float64, stored as fp32."""
    l = _f64(x) @ _f64(w_router)
    if bias is not None:
        l = l + _f64(bias)[None, :]
    return l.astype(np.float32)


def shared_gate_logit(x, w_sg, storage: str = "bf16") -> np.ndarray:
    """z = x . w_sg, kept in fp32 on the device (the shared expert's gate is sigmoid(z))."""
    return store_fp32(_f64(x) @ _f64(w_sg), storage)


def permute(x, src_of, K: int) -> np.ndarray:
    """Row r of the permuted buffer is token src_of[r] // K (an exact copy)."""
    src = np.asarray(src_of, dtype=np.int64)
    return _f64(x)[src // K]


def ffn_rows_fwd(xp_rows, wg, wu, wd, storage: str, o_storage: str | None = None):
    """SwiGLU expert on some rows of one expert: returns a, b, h, o as stored.

    `o_storage` (default `storage`) rounds o alone: on one rank of an expert-tensor-
    parallel group (knowledge-base notes page, method paragraph: AllGather-V shares the
    rows inside the ETP group, ReduceScatter-V sums the expert outputs) wg, wu are
    column slices and wd the matching row slice, so o is a partial sum kept in fp32."""
    xr = _f64(xp_rows)
    a = xr @ _f64(wg)
    b = xr @ _f64(wu)
    h = silu(a) * b                      # from the unrounded accumulators
    a_s, b_s, h_s = store(a, storage), store(b, storage), store(h, storage)
    o = store(h_s @ _f64(wd), o_storage or storage)
    return a_s, b_s, h_s, o


def expert_ffn_fwd(xp, w_gate, w_up, w_down, offsets, storage: str,
                   o_storage: str | None = None):
    """Grouped SwiGLU FFN over the expert segments [offsets[e], offsets[e+1])."""
    n = int(offsets[-1])
    f = w_gate.shape[2]
    d = w_down.shape[2]
    a = np.zeros((n, f)); b = np.zeros((n, f)); h = np.zeros((n, f)); o = np.zeros((n, d))
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            a[lo:hi], b[lo:hi], h[lo:hi], o[lo:hi] = ffn_rows_fwd(
                xp[lo:hi], w_gate[e], w_up[e], w_down[e], storage, o_storage)
    return a, b, h, o


def unpermute(o, row_of, gate, keep, storage: str, shared=None, z=None) -> np.ndarray:
    """y_t = sum over kept slots k (ascending) of g_tk * o[row_of[t,k]]
    (+ sigmoid(z_t) * shared_t)."""
    T, K = np.shape(row_of)
    o = _f64(o)
    y = np.zeros((T, o.shape[1]))
    for k in range(K):
        kept = np.asarray(keep)[:, k].astype(bool)
        rows = np.asarray(row_of)[kept, k]
        y[kept] += _f64(gate)[kept, k][:, None] * o[rows]
    if shared is not None:
        y += sigmoid(_f64(z))[:, None] * _f64(shared)
    return store(y, storage)


# ----------------------------------------------------------------------------------
# Backward (loss = sum_t <dy_t, y_t>)
# ----------------------------------------------------------------------------------

def unpermute_bwd(dy, o, row_of, gate, keep, n_rows: int, storage: str, shared=None, z=None):
    """d_o[row_of[t,k]] = g_tk * dy_t; dgate_tk = <dy_t, o[row_of[t,k]]> (0 if dropped).
    With a shared expert also: dshared_t = sigmoid(z_t) dy_t and
    dz_t = <dy_t, shared_t> * s_t (1 - s_t)."""
    dy = _f64(dy)
    o = _f64(o)
    T, K = np.shape(row_of)
    d_o = np.zeros((n_rows, dy.shape[1]))
    dgate = np.zeros((T, K))
    for k in range(K):
        kept = np.asarray(keep)[:, k].astype(bool)
        rows = np.asarray(row_of)[kept, k]
        d_o[rows] = _f64(gate)[kept, k][:, None] * dy[kept]
        dgate[kept, k] = np.sum(dy[kept] * o[rows], axis=1)
    res = {"d_o": store(d_o, storage), "dgate": store_fp32(dgate, storage)}
    if shared is not None:
        s = sigmoid(_f64(z))
        res["dshared"] = store(s[:, None] * dy, storage)
        ds = np.sum(dy * _f64(shared), axis=1)
        res["dz"] = store_fp32(ds * s * (1.0 - s), storage)
    return res


def ffn_rows_bwd_data(a_s, b_s, d_o_rows, wg, wu, wd, storage: str,
                      dxp_storage: str | None = None):
    """dgrad for some rows of one expert: returns da, db, dxp as stored (`dxp_storage`,
    default `storage`: on an expert-tensor-parallel rank dxp is a partial sum over the
    rank's ffn slice, kept in fp32 like o)."""
    dh = _f64(d_o_rows) @ _f64(wd).T
    a = _f64(a_s); b = _f64(b_s)
    sg = sigmoid(a)
    da = store(dh * b * sg * (1.0 + a * (1.0 - sg)), storage)
    db = store(dh * a * sg, storage)
    dxp = store(da @ _f64(wg).T + db @ _f64(wu).T, dxp_storage or storage)
    return da, db, dxp


def ffn_cols_fwd(xp_rows, wg, wu, cols, storage: str):
    """Columns `cols` of a, b, h for the rows of one expert (the stored values)."""
    xr = _f64(xp_rows)
    a = xr @ _f64(np.asarray(wg)[:, cols])
    b = xr @ _f64(np.asarray(wu)[:, cols])
    h = silu(a) * b
    return store(a, storage), store(b, storage), store(h, storage)


def ffn_cols_bwd(a_cols, b_cols, d_o_rows, wd, cols, storage: str):
    """Columns `cols` of da, db for the rows of one expert, from the stored a, b."""
    dh = _f64(d_o_rows) @ _f64(np.asarray(wd)[cols, :]).T
    a = _f64(a_cols); b = _f64(b_cols)
    sg = sigmoid(a)
    return store(dh * b * sg * (1.0 + a * (1.0 - sg)), storage), store(dh * a * sg, storage)


def expert_ffn_bwd(xp, a, b, h, w_gate, w_up, w_down, offsets, d_o, storage: str,
                   dxp_storage: str | None = None):
    """B2..B5: dgrad through down, SwiGLU backward, wgrads, dgrad through gate/up."""
    n = int(offsets[-1])
    E, d, f = w_gate.shape
    dxp = np.zeros((n, d))
    dwg = np.zeros((E, d, f)); dwu = np.zeros((E, d, f)); dwd = np.zeros((E, f, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue          # no rows: the weight gradients of this expert are zero
        da, db, dxp[lo:hi] = ffn_rows_bwd_data(a[lo:hi], b[lo:hi], d_o[lo:hi],
                                               w_gate[e], w_up[e], w_down[e], storage,
                                               dxp_storage)
        xr = _f64(xp[lo:hi])
        dwd[e] = _f64(h[lo:hi]).T @ _f64(d_o[lo:hi])
        dwg[e] = xr.T @ da
        dwu[e] = xr.T @ db
    return {"dxp": dxp, "dw_gate": store(dwg, storage), "dw_up": store(dwu, storage),
            "dw_down": store(dwd, storage)}


def router_dlogits(topk_idx, gate, dgate, E: int, storage: str = "bf16") -> np.ndarray:
    """Gradient of the renormalised top-K softmax: for the K chosen experts
    dl_{e_j} = g_j (dgate_j - sum_k g_k dgate_k); the other logits get 0."""
    g = _f64(gate)
    dg = _f64(dgate)
    T, K = g.shape
    inner = np.sum(g * dg, axis=1, keepdims=True)
    dsel = g * (dg - inner)
    dl = np.zeros((T, E))
    for k in range(K):
        dl[np.arange(T), np.asarray(topk_idx)[:, k]] += dsel[:, k]
    return store_fp32(dl, storage)


def permute_bwd(dxp, row_of, keep, T: int, storage: str, dlogits=None, w_router=None,
                dz=None, w_sg=None, dx_extra=None) -> np.ndarray:
    """dx_t = sum over kept k of dxp[row_of[t,k]] + dl_t W_r^T (+ dz_t w_sg + extra_t)."""
    dxp = _f64(dxp)
    K = np.shape(row_of)[1]
    dx = np.zeros((T, dxp.shape[1]))
    for k in range(K):
        kept = np.asarray(keep)[:, k].astype(bool)
        dx[kept] += dxp[np.asarray(row_of)[kept, k]]
    if dlogits is not None:
        dx += _f64(dlogits) @ _f64(w_router).T
    if dz is not None:
        dx += _f64(dz)[:, None] * _f64(w_sg)[None, :]
    if dx_extra is not None:
        dx += _f64(dx_extra)
    return store(dx, storage)


def router_wgrad(x, dlogits, storage: str) -> np.ndarray:
    """dW_r = x^T dl."""
    return store(_f64(x).T @ _f64(dlogits), storage)


# ----------------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------------

def layer_fwd_bwd(inp: dict, K: int, S: int, cap: int, storage: str, logits=None) -> dict:
    """Forward and backward of the layer on numpy inputs.

    inp: x [T,d], w_router [d,E], bias [E] or None, w_gate/w_up [E,d,f], w_down [E,f,d],
         dy [T,d]; optional shared expert w_sg [d], ws_gate/ws_up [1,d,fs], ws_down [1,fs,d].
    logits: route on these fp32 logits instead of the oracle's own (used to compare
         with a device whose logits differ by rounding).
    """
    x = inp["x"]
    T = x.shape[0]
    E = inp["w_router"].shape[1]
    own_logits = router_logits(x, inp["w_router"], inp.get("bias"))
    lg = own_logits if logits is None else np.asarray(logits, np.float32)
    r = route(lg, K, S, cap)
    xp = permute(x, r["src_of"], K)
    a, b, h, o = expert_ffn_fwd(xp, inp["w_gate"], inp["w_up"], inp["w_down"], r["offsets"],
                                storage)
    shared = z = None
    if inp.get("w_sg") is not None:
        z = shared_gate_logit(x, inp["w_sg"], storage)
        sa, sb, sh, shared = expert_ffn_fwd(_f64(x), inp["ws_gate"], inp["ws_up"],
                                            inp["ws_down"], np.array([0, T]), storage)
    y = unpermute(o, r["row_of"], r["topk_gate"], r["keep"], storage, shared, z)

    ub = unpermute_bwd(inp["dy"], o, r["row_of"], r["topk_gate"], r["keep"], r["n_kept"],
                       storage, shared, z)
    fb = expert_ffn_bwd(xp, a, b, h, inp["w_gate"], inp["w_up"], inp["w_down"], r["offsets"],
                        ub["d_o"], storage)
    dxp_s = fb["dxp"]
    dl = router_dlogits(r["topk_idx"], r["topk_gate"], ub["dgate"], E, storage)
    res = {"logits": own_logits, "routing": r, "xp": xp, "a": a, "b": b, "h": h, "o": o,
           "y": y, "d_o": ub["d_o"], "dgate": ub["dgate"], "dxp": dxp_s, "dlogits": dl,
           "dw_gate": fb["dw_gate"], "dw_up": fb["dw_up"], "dw_down": fb["dw_down"],
           "dw_router": router_wgrad(x, dl, storage)}
    dx_extra = None
    dz = None
    if shared is not None:
        sfb = expert_ffn_bwd(_f64(x), sa, sb, sh, inp["ws_gate"], inp["ws_up"], inp["ws_down"],
                             np.array([0, T]), ub["dshared"], storage)
        dz = ub["dz"]
        dx_extra = sfb["dxp"]
        res.update({"z": z, "shared": shared, "dshared": ub["dshared"], "dz": dz,
                    "dws_gate": sfb["dw_gate"], "dws_up": sfb["dw_up"],
                    "dws_down": sfb["dw_down"], "dw_sg": store(_f64(x).T @ _f64(dz), storage),
                    "dx_shared": dx_extra})
    res["dx"] = permute_bwd(dxp_s, r["row_of"], r["keep"], T, storage, dl, inp["w_router"],
                            dz, inp.get("w_sg"), dx_extra)
    return res
