"""Helpers of the GPU parity tests: run the HIP layer through the C ABI, bring its
results to the host and compare them with the CPU oracle on the same inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# Normwise max-abs-rel bounds: fp32 values (logits, the shared-gate logit, every output of
# an fp32 layer) and values stored in bf16 with fp32 accumulation.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2

ROUTING_KEYS = ("topk_idx", "topk_prob", "topk_gate", "keep", "row_of", "routed_counts",
                "kept_counts", "offsets")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t) -> np.ndarray:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.detach().cpu().numpy()
    return np.asarray(t)


def host_inputs(inp: dict) -> dict:
    return {k: host(v) for k, v in inp.items()}


def max_abs_rel(got, exp) -> float:
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    if exp.size == 0:
        return 0.0
    return float(np.max(np.abs(got - exp)) / max(float(np.max(np.abs(exp))), 1e-30))


def assert_close(name, got, exp, tol):
    err = max_abs_rel(got, exp)
    log(f"    {name:12s} max-abs-rel {err:.3e} (tol {tol:.0e})")
    assert err <= tol, f"{name}: max-abs-rel {err:.3e} > {tol:.0e}"


def assert_routing_equal(lay, ref_routing):
    """Bit-exact comparison of every routing output (src_of on its first n_kept)."""
    n = int(host(lay.rt["n_kept"])[0])
    assert n == ref_routing["n_kept"], ("n_kept", n, ref_routing["n_kept"])
    for k in ROUTING_KEYS:
        got = host(lay.rt[k])
        exp = np.asarray(ref_routing[k])
        if k == "routed_counts":
            got = got[: exp.shape[0]]
        assert got.shape == exp.shape, (k, got.shape, exp.shape)
        if got.dtype.kind == "f":
            assert np.array_equal(got.view(np.uint32), exp.astype(np.float32).view(np.uint32)), k
        else:
            assert np.array_equal(got, exp), k
    assert np.array_equal(host(lay.rt["src_of"])[:n], ref_routing["src_of"]), "src_of"


def check_layer(lay, inp: dict, K: int, S: int, cap: int, tol: float):
    """Full element-by-element comparison of one fwd+bwd run with the oracle."""
    storage = "f32" if lay.dtype == torch.float32 else "bf16"
    h = host_inputs(inp)
    gpu_logits = host(lay.buf["logits"])
    own = oracle.router_logits(h["x"], h["w_router"], h.get("bias"))
    assert_close("logits", gpu_logits, own, TOL_F32)
    ref = oracle.layer_fwd_bwd(h, K, S, cap, storage, logits=gpu_logits)
    assert_routing_equal(lay, ref["routing"])
    n = ref["routing"]["n_kept"]
    b = lay.buf
    assert np.array_equal(host(b["xp"])[:n], ref["xp"]), "xp must be an exact copy"
    for k in ("a", "b", "h", "o", "d_o", "dxp"):
        assert_close(k, host(b[k])[:n], ref[k][:n], tol)
    for k in ("y", "dgate", "dlogits", "dx", "dw_gate", "dw_up", "dw_down", "dw_router"):
        assert_close(k, host(b[k]), ref[k], tol)
    if lay.fs:
        assert_close("sg_logit", host(b["sg_logit"]), oracle.shared_gate_logit(h["x"], h["w_sg"],
                                                                                 "f32"), TOL_F32)
        for k in ("shared", "dshared", "dz", "dws_gate", "dws_up", "dws_down", "dw_sg",
                  "dx_shared"):
            assert_close(k, host(b[k]), ref[k], tol)
    return ref
