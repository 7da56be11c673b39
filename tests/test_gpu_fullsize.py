"""GPU parity at the full layer sizes, in the launch configuration bench.py times.

Complete comparison (every element of every output and gradient) for three shapes:
Mixtral-8x22B, Mixtral-8x22B-G8T8 with the Zipf bias, and Qwen2-57B-A14B with its
sigmoid-gated shared expert.  The oracle runs expert by expert (forward on each
expert's rows, the un-permutation over all tokens, then each expert's backward) so host
memory stays bounded:
  - routing over all tokens: the oracle routes the GPU's logits and must match bit for bit;
  - logits and the shared-gate logit of every token (fp32, bound 1e-5);
  - xp: every row an exact copy of its token;
  - a, b, h, o, d_o, dxp: every row; dW_gate, dW_up, dW_down: every entry of every expert;
  - y, dgate, dlogits, dx, dW_router; the shared expert's a, b, h, output, dshared, dz,
    dx contribution and weight gradients, dw_sg: every element.
The three larger shapes (Llama3-8x70B one GPU's 8192-token share, Mixtral dimensions over
16384 tokens dropped per 4096-token sub-sequence or over the whole sequence) get the
routing, logits and xp checks over all tokens, one expert compared completely (every
row and every weight-gradient entry), and for sampled tokens drawn from every expert
(plus a token with a dropped slot) all their rows and y, dgate, dlogits, dx; sampled
weight-gradient entries of four experts.
Every shape's segment offsets also go through the host check of the grouped GEMM's tile
maps (each output tile produced exactly once, inside its segment).
Bounds: normwise max-abs-rel over each whole tensor, 2e-2 for bf16 storage with fp32
accumulation, 1e-5 for fp32 values.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import TOL_BF16, TOL_F32, assert_close, assert_routing_equal, host, log

pytestmark = pytest.mark.gpu

TOL = TOL_BF16
HERE = os.path.dirname(os.path.abspath(__file__))
COMPLETE = ["mixtral_8x22b", "mixtral_g8t8", "qwen2_57b_a14b"]
SAMPLED = ["llama3_8x70b", "mixtral_t16k_s4k", "mixtral_t16k_full"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_dispatch_expert_router_amd import _lib as L
    L.load()


def _f32(t):
    return t.float().cpu().numpy()


class Normwise:
    """max|got - exp| / max|exp| over a tensor compared in pieces."""

    def __init__(self):
        self.diff = {}
        self.ref = {}

    def add(self, key, got, exp):
        got = np.asarray(got, np.float64)
        exp = np.asarray(exp, np.float64)
        if exp.size == 0:
            return
        self.diff[key] = max(self.diff.get(key, 0.0), float(np.max(np.abs(got - exp))))
        self.ref[key] = max(self.ref.get(key, 0.0), float(np.max(np.abs(exp))))

    def check(self, tol):
        for key in self.diff:
            err = self.diff[key] / max(self.ref[key], 1e-30)
            log(f"    {key:12s} max-abs-rel {err:.3e} (tol {tol:.0e})")
            assert err <= tol, f"{key}: max-abs-rel {err:.3e} > {tol:.0e}"


def tile_map_checker():
    """The host program that walks the grouped GEMM's launch grids (tests/native); built
    with hipcc for the host only when it is not there yet."""
    exe = os.path.join(HERE, "native", "tile_map_check")
    if not os.path.exists(exe):
        from token_dispatch_expert_router_amd import build
        build.build_tile_map_check(exe)
    return exe


def check_tile_maps(offsets, R, d, f):
    offs = [int(v) for v in offsets]
    E = len(offs) - 1
    r = subprocess.run([tile_map_checker(), str(E), str(R), str(d), str(f)] + [str(v) for v in offs],
                       capture_output=True, text=True, timeout=120)
    log("    tile maps: " + "; ".join(r.stdout.strip().splitlines()))
    assert r.returncode == 0, r.stdout + r.stderr


def _run_layer(s):
    from token_dispatch_expert_router_amd.layer import MoELayer
    cap = oracle.capacity(s.sub_seq, s.K, s.E, s.cf)
    log(f"  full-size {s.name}: T={s.T} d={s.d} E={s.E} K={s.K} f={s.f} fs={s.fs} cap={cap}")
    inp = moe_synth.make_inputs(s, device="cuda")
    lay = MoELayer(s.T, s.d, s.E, s.K, s.f, s.sub_seq, cap, torch.bfloat16, fs=s.fs,
                   device="cuda")
    lay.forward_backward(inp)
    torch.cuda.synchronize()
    return lay, inp, cap


def _common_checks(s, lay, inp, cap):
    """Routing (bit-exact, all tokens), logits (all tokens), xp (every row), tile maps."""
    b = lay.buf
    gl = host(b["logits"])
    ref_r = oracle.route(gl, s.K, s.sub_seq, cap)
    assert_routing_equal(lay, ref_r)
    n_kept = ref_r["n_kept"]
    kc = ref_r["kept_counts"]
    log(f"    n_kept {n_kept} of {s.T * s.K}; kept per expert {kc.min()}..{kc.max()}")
    x = _f32(inp["x"])
    bias = None if inp["bias"] is None else host(inp["bias"])
    assert_close("logits", gl, oracle.router_logits(x, _f32(inp["w_router"]), bias), TOL_F32)
    src = ref_r["src_of"]
    for lo in range(0, n_kept, 8192):
        hi = min(n_kept, lo + 8192)
        got = _f32(b["xp"][lo:hi])
        assert np.array_equal(got, x[src[lo:hi] // s.K]), f"xp rows {lo}..{hi} are not exact copies"
    check_tile_maps(ref_r["offsets"], lay.R, s.d, s.f)
    return ref_r, x


def _weights(inp, e):
    return (_f32(inp["w_gate"][e])[None], _f32(inp["w_up"][e])[None],
            _f32(inp["w_down"][e])[None])


def _expert_fwd(s, inp, x, ref_r, e, acc, b):
    """Oracle forward of expert e's rows; compares a, b, h, o of those rows."""
    lo, hi = int(ref_r["offsets"][e]), int(ref_r["offsets"][e + 1])
    xs = x[ref_r["src_of"][lo:hi] // s.K]
    wg, wu, wd = _weights(inp, e)
    a, bb, h, o = oracle.expert_ffn_fwd(xs, wg, wu, wd, np.array([0, hi - lo]), "bf16")
    for key, ref_v in (("a", a), ("b", bb), ("h", h), ("o", o)):
        acc.add(key, _f32(b[key][lo:hi]), ref_v)
    return xs, a.astype(np.float32), bb.astype(np.float32), h.astype(np.float32), o


def _expert_bwd(s, inp, xs, a, bb, h, d_o, e, lo, hi, acc, b):
    """Oracle backward of expert e's rows; compares dxp rows and every dW entry."""
    wg, wu, wd = _weights(inp, e)
    fb = oracle.expert_ffn_bwd(xs, a, bb, h, wg, wu, wd, np.array([0, hi - lo]), d_o, "bf16")
    acc.add("dxp", _f32(b["dxp"][lo:hi]), fb["dxp"])
    if hi == lo:
        for k in ("dw_gate", "dw_up", "dw_down"):
            assert not torch.any(b[k][e] != 0), f"{k}[{e}] of an empty expert is not zero"
    else:
        acc.add("dW_gate", _f32(b["dw_gate"][e]), fb["dw_gate"][0])
        acc.add("dW_up", _f32(b["dw_up"][e]), fb["dw_up"][0])
        acc.add("dW_down", _f32(b["dw_down"][e]), fb["dw_down"][0])
    return fb["dxp"]


@pytest.mark.parametrize("name", COMPLETE)
def test_fullsize_complete(name):
    s = moe_synth.shape_by_name(name)
    lay, inp, cap = _run_layer(s)
    b = lay.buf
    ref_r, x = _common_checks(s, lay, inp, cap)
    n_kept, offs = ref_r["n_kept"], ref_r["offsets"]
    dy = _f32(inp["dy"])
    acc = Normwise()

    # forward, expert by expert
    o_all = np.zeros((n_kept, s.d))
    saved = {}
    for e in range(s.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        xs, a, bb, h, o = _expert_fwd(s, inp, x, ref_r, e, acc, b)
        o_all[lo:hi] = o
        saved[e] = (xs, a, bb, h)
        if e % 8 == 7 or e == s.E - 1:
            log(f"    forward: experts 0..{e} done")

    shared = z = None
    if s.fs:
        z = oracle.shared_gate_logit(x, _f32(inp["w_sg"]), "f32")
        assert_close("sg_logit", host(b["sg_logit"]), z, TOL_F32)
        sw = (_f32(inp["ws_gate"]), _f32(inp["ws_up"]), _f32(inp["ws_down"]))
        sa, sb, sh, shared = oracle.expert_ffn_fwd(x, *sw, np.array([0, s.T]), "bf16")
        for key, ref_v in (("sa", sa), ("sb", sb), ("sh", sh), ("shared", shared)):
            acc.add(key, _f32(b[key]), ref_v)
        log("    shared expert forward done")

    gate, keep, row_of = ref_r["topk_gate"], ref_r["keep"], ref_r["row_of"]
    y = oracle.unpermute(o_all, row_of, gate, keep, "bf16", shared, z)
    acc.add("y", _f32(b["y"]), y)
    del y
    ub = oracle.unpermute_bwd(dy, o_all, row_of, gate, keep, n_kept, "bf16", shared, z)
    del o_all
    acc.add("d_o", _f32(b["d_o"][:n_kept]), ub["d_o"])
    acc.add("dgate", host(b["dgate"]), ub["dgate"])

    # backward, expert by expert
    dxp_all = np.zeros((n_kept, s.d))
    for e in range(s.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        xs, a, bb, h = saved.pop(e)
        dxp_all[lo:hi] = _expert_bwd(s, inp, xs, a, bb, h, ub["d_o"][lo:hi], e, lo, hi, acc, b)
        if e % 8 == 7 or e == s.E - 1:
            log(f"    backward: experts 0..{e} done")

    dz = dx_shared = None
    w_sg = None
    if s.fs:
        w_sg = _f32(inp["w_sg"])
        dz = ub["dz"]
        acc.add("dshared", _f32(b["dshared"]), ub["dshared"])
        acc.add("dz", host(b["dz"]), dz)
        sfb = oracle.expert_ffn_bwd(x, sa, sb, sh, *sw, np.array([0, s.T]), ub["dshared"], "bf16")
        dx_shared = sfb["dxp"]
        acc.add("dx_shared", _f32(b["dx_shared"]), dx_shared)
        acc.add("dws_gate", _f32(b["dws_gate"]), sfb["dw_gate"])
        acc.add("dws_up", _f32(b["dws_up"]), sfb["dw_up"])
        acc.add("dws_down", _f32(b["dws_down"]), sfb["dw_down"])
        acc.add("dw_sg", _f32(b["dw_sg"]), oracle.router_wgrad(x, dz[:, None], "bf16")[:, 0])
        log("    shared expert backward done")

    dl = oracle.router_dlogits(ref_r["topk_idx"], gate, ub["dgate"], s.E, "bf16")
    acc.add("dlogits", host(b["dlogits"]), dl)
    dx = oracle.permute_bwd(dxp_all, row_of, keep, s.T, "bf16", dl, _f32(inp["w_router"]), dz,
                            w_sg, dx_shared)
    acc.add("dx", _f32(b["dx"]), dx)
    acc.add("dW_router", _f32(b["dw_router"]), oracle.router_wgrad(x, dl, "bf16"))
    acc.check(TOL)
    del lay, inp
    torch.cuda.empty_cache()


def _pick_tokens(topk, keep, E, rng):
    """Two tokens with a kept slot on each expert (where it has any), and one token that
    lost a slot to the capacity drop (where there is one)."""
    T, K = topk.shape
    picked = set()
    for e in range(E):
        cand = np.nonzero(((topk == e) & keep).any(axis=1))[0]
        if len(cand):
            picked.update(int(t) for t in rng.choice(cand, size=min(2, len(cand)), replace=False))
    dropped = np.nonzero((~keep).any(axis=1))[0]
    if len(dropped):
        picked.add(int(rng.choice(dropped)))
    return sorted(picked)


@pytest.mark.parametrize("name", SAMPLED)
def test_fullsize_sampled(name):
    s = moe_synth.shape_by_name(name)
    lay, inp, cap = _run_layer(s)
    b = lay.buf
    ref_r, x = _common_checks(s, lay, inp, cap)
    n_kept, offs = ref_r["n_kept"], ref_r["offsets"]
    dy = _f32(inp["dy"])
    wr = _f32(inp["w_router"])
    rng = np.random.default_rng(s.seed)
    gate, keep, row_of, topk = (ref_r["topk_gate"], ref_r["keep"].astype(bool), ref_r["row_of"],
                                ref_r["topk_idx"])
    counts = ref_r["kept_counts"]

    # one expert compared completely: every row and every weight-gradient entry
    e_full = int(np.argsort(counts)[len(counts) // 2])
    lo, hi = int(offs[e_full]), int(offs[e_full + 1])
    acc = Normwise()
    xs, a, bb, h, _ = _expert_fwd(s, inp, x, ref_r, e_full, acc, b)
    # d_o of the expert's rows from the oracle's un-permute backward (its dgate, which needs
    # every expert's o, is not used here)
    ub = oracle.unpermute_bwd(dy, np.zeros((n_kept, s.d), np.float32), row_of, gate, keep,
                              n_kept, "bf16")
    d_o = ub["d_o"][lo:hi]
    acc.add("d_o", _f32(b["d_o"][lo:hi]), d_o)
    _expert_bwd(s, inp, xs, a, bb, h, d_o, e_full, lo, hi, acc, b)
    log(f"    expert {e_full} ({hi - lo} rows) compared completely")
    acc.check(TOL)
    del xs, a, bb, h, ub

    # sampled tokens from every expert: all their rows, then y, dgate, dlogits, dx
    toks = _pick_tokens(topk, keep, s.E, rng)
    n_t = len(toks)
    sub_row = -np.ones((n_t, s.K), np.int64)
    pairs = [(i, t, k) for i, t in enumerate(toks) for k in range(s.K) if keep[t, k]]
    experts = sorted({int(topk[t, k]) for _, t, k in pairs})
    log(f"    sampled {n_t} tokens -> {len(pairs)} rows over {len(experts)} experts")
    o_sub = np.zeros((len(pairs), s.d))
    dxp_sub = np.zeros((len(pairs), s.d))
    acc = Normwise()
    for e in experts:
        pe = [(n, i, t, k) for n, (i, t, k) in enumerate(pairs) if topk[t, k] == e]
        xr = x[[t for _, _, t, _ in pe]]
        wg, wu, wd = (w[0] for w in _weights(inp, e))
        a, bb, h, o = oracle.ffn_rows_fwd(xr, wg, wu, wd, "bf16")
        d_o = oracle.round_bf16(np.array([gate[t, k] for _, _, t, k in pe])[:, None] *
                                dy[[t for _, _, t, _ in pe]])
        _, _, dxp = oracle.ffn_rows_bwd_data(a, bb, d_o, wg, wu, wd, "bf16")
        ridx = torch.as_tensor([int(row_of[t, k]) for _, _, t, k in pe], device="cuda")
        for key, ref_v in (("a", a), ("b", bb), ("h", h), ("o", o), ("d_o", d_o), ("dxp", dxp)):
            acc.add(key + "_rows", _f32(b[key][ridx]), ref_v)
        for j, (n, i, t, k) in enumerate(pe):
            o_sub[n] = o[j]
            dxp_sub[n] = dxp[j]
            sub_row[i, k] = n
        del wg, wu, wd
    sub_gate = gate[toks]
    sub_keep = keep[toks]
    y = oracle.unpermute(o_sub, sub_row, sub_gate, sub_keep, "bf16")
    ub = oracle.unpermute_bwd(dy[toks], o_sub, sub_row, sub_gate, sub_keep, len(pairs), "bf16")
    dl = oracle.router_dlogits(topk[toks], sub_gate, ub["dgate"], s.E, "bf16")
    dx = oracle.permute_bwd(dxp_sub, sub_row, sub_keep, n_t, "bf16", dl, wr)
    acc.add("y_tokens", _f32(b["y"])[toks], y)
    acc.add("dgate_tokens", host(b["dgate"])[toks], ub["dgate"])
    acc.add("dlogits_tokens", host(b["dlogits"])[toks], dl)
    acc.add("dx_tokens", _f32(b["dx"])[toks], dx)
    acc.check(TOL)

    # sampled weight-gradient entries (whole-segment sums) of four experts
    order = np.argsort(counts)
    others = [int(e) for e in order[1:-1] if e != e_full]
    chosen = sorted({int(order[0]), int(order[-1])} |
                    set(int(e) for e in rng.choice(others, size=min(2, len(others)), replace=False)))
    acc = Normwise()
    for e in chosen:
        lo, hi = int(offs[e]), int(offs[e + 1])
        src = ref_r["src_of"][lo:hi]
        tt, kk = src // s.K, src % s.K
        xs = x[tt]
        d_o = oracle.round_bf16(gate[tt, kk][:, None] * dy[tt])
        wg, wu, wd = (w[0] for w in _weights(inp, e))
        ci = rng.choice(s.d, size=16, replace=False)     # rows of dW_gate/dW_up, cols of dW_down
        cj = rng.choice(s.f, size=16, replace=False)     # cols of dW_gate/dW_up, rows of dW_down
        a, bb, h = oracle.ffn_cols_fwd(xs, wg, wu, cj, "bf16")
        da, db = oracle.ffn_cols_bwd(a, bb, d_o, wd, cj, "bf16")
        ii, jj = np.meshgrid(ci, cj, indexing="ij")
        acc.add("dW_gate_smp", _f32(b["dw_gate"][e])[ii, jj],
                oracle.round_bf16(xs[:, ci].T.astype(np.float64) @ da))
        acc.add("dW_up_smp", _f32(b["dw_up"][e])[ii, jj],
                oracle.round_bf16(xs[:, ci].T.astype(np.float64) @ db))
        acc.add("dW_down_smp", _f32(b["dw_down"][e])[jj.T, ii.T],
                oracle.round_bf16(h.T @ d_o[:, ci]))
        log(f"    expert {e}: {hi - lo} rows, 16 x 16 weight-gradient entries")
    acc.check(TOL)

    # router weight gradient from the GPU's dlogits (the router wgrad given its input)
    assert_close("dW_router", _f32(b["dw_router"]), oracle.router_wgrad(x, host(b["dlogits"]), "bf16"),
                 TOL)
    del lay, inp
    torch.cuda.empty_cache()


def test_fullsize_repeat_is_bit_identical():
    """Two forward + backward steps of the Mixtral-shaped layer on the same inputs give the
    same bits in every output, gradient and routing array (fixed-order reductions, no
    atomics on floating-point values)."""
    s = moe_synth.shape_by_name("mixtral_8x22b")
    lay, inp, cap = _run_layer(s)
    first = {k: v.clone() for k, v in lay.buf.items() if isinstance(v, torch.Tensor)}
    first_rt = {k: v.clone() for k, v in lay.rt.items()}
    lay.forward_backward(inp)
    torch.cuda.synchronize()
    n = int(lay.rt["n_kept"].item())
    for k, v in first.items():
        cur = lay.buf[k]
        if k in ("xp", "a", "b", "h", "o", "d_o", "dxp"):
            v, cur = v[:n], cur[:n]     # rows past n_kept are not written
        assert torch.equal(v, cur), f"{k} differs between two identical steps"
    for k, v in first_rt.items():
        cur = lay.rt[k]
        if k == "src_of":
            v, cur = v[:n], cur[:n]
        assert torch.equal(v, cur), f"routing {k} differs between two identical steps"
    log(f"    two steps bit-identical over {len(first)} buffers and {len(first_rt)} routing arrays")
    del lay, inp, first
    torch.cuda.empty_cache()
