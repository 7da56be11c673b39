"""Pins for the CPU oracle: each test checks it against something other than itself
(hand-worked fixtures, closed forms, brute force, libm, a dense formulation written
here, complex-step derivatives) so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------------
# exp, pairwise sum, softmax
# --------------------------------------------------------------------------------

def test_exp_exhaustive_against_libm():
    """Every fp32 r in [-88, 0]: within 2 ulp of double exp, +0 only where exp < 2^-125,
    and never a result below 2^-125."""
    worst, n, bad_flush, bad_tiny = oracle.exp_scan(-88.0)
    assert n > 1_100_000_000
    assert worst <= 2.0, worst
    assert bad_flush == 0 and bad_tiny == 0


def test_exp_special_values():
    assert oracle.exp32(0.0) == 1.0
    assert oracle.exp32(-0.0) == 1.0
    assert oracle.exp32(-100.0) == 0.0          # below the flush point
    assert abs(oracle.exp32(-1.0) - math.exp(-1.0)) < 1e-7


def test_pairwise_sum_order_and_bound():
    # exact cases
    assert oracle.pairwise_sum32([1, 2, 3, 4, 5, 6, 7, 8]) == 36.0
    assert oracle.pairwise_sum32([0.5]) == 0.5
    # the tree adds neighbours first: (1 + 2^-24) + (2^-24 + 2^-24) rounds differently
    # from a left-to-right sum; both sides of the pairing are pinned by hand here
    e = 2.0 ** -24
    # pairs: (1 + e) -> 1 (tie to even), (e + e) = 2e; 1 + 2e = 1 + 2^-23 exactly
    assert oracle.pairwise_sum32([1.0, e, e, e]) == np.float32(1.0 + 2.0 ** -23)
    # left to right would give ((1 + e) + e) + e = 1.0
    rng = np.random.default_rng(5)
    for n in (3, 7, 8, 13, 64):
        v = rng.random(n).astype(np.float32)
        exact = math.fsum(float(t) for t in v)
        bound = math.ceil(math.log2(n)) * 2.0 ** -24 * exact * 1.01 + 1e-30
        assert abs(oracle.pairwise_sum32(v) - exact) <= bound


def test_softmax_against_float64():
    rng = np.random.default_rng(1)
    for E in (2, 4, 8, 64):
        l = (rng.standard_normal((50, E)) * 3).astype(np.float32)
        p = oracle.softmax32(l).astype(np.float64)
        # given the fp32-rounded reduced arguments r = l - max, the result is within a
        # few ulp (exp <= 2 ulp, the sum log2(E) roundings, one division)
        r32 = (l - l.max(1, keepdims=True)).astype(np.float64)
        ref = np.exp(r32)
        ref /= ref.sum(1, keepdims=True)
        assert np.max(np.abs(p - ref) / ref) < (4 + math.log2(E)) * 2.0 ** -24
        # against exact float64 the rounding of r adds |r| * 2^-24 relative
        l64 = l.astype(np.float64)
        r64 = l64 - l64.max(1, keepdims=True)
        ref64 = np.exp(r64)
        ref64 /= ref64.sum(1, keepdims=True)
        bound = (np.abs(r64) + E / math.e + 4 + math.log2(E)) * 2.0 ** -24
        assert np.all(np.abs(p - ref64) / ref64 < bound)
        assert np.max(np.abs(p.sum(1) - 1.0)) <= E * 2.0 ** -24


# --------------------------------------------------------------------------------
# top-K and gates
# --------------------------------------------------------------------------------

def _brute_topk(p, K):
    """The unique K-subset where every member beats every non-member under
    (p desc, index asc), found by enumeration; slots ordered the same way."""
    E = len(p)
    found = []
    for sub in itertools.combinations(range(E), K):
        out = [j for j in range(E) if j not in sub]
        if all((p[i] > p[j]) or (p[i] == p[j] and i < j) for i in sub for j in out):
            found.append(sub)
    assert len(found) == 1
    return sorted(found[0], key=lambda i: (-p[i], i))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(300):
        E = int(rng.integers(2, 9))
        K = int(rng.integers(1, E + 1))
        # coarse logits so that exact ties are common
        l = rng.integers(-3, 4, size=(1, E)).astype(np.float32)
        r = oracle.route(l, K, 1, -1)
        p = oracle.softmax32(l)[0]
        assert list(r["topk_idx"][0]) == _brute_topk(p, K)
        assert np.array_equal(r["topk_prob"][0], p[r["topk_idx"][0]])


def test_gates_sum_to_one_and_equal_softmax_over_chosen():
    rng = np.random.default_rng(3)
    for E, K in ((8, 2), (64, 8), (4, 1), (6, 6), (5, 3)):
        l = (rng.standard_normal((64, E)) * 2).astype(np.float32)
        r = oracle.route(l, K, 64, -1)
        g = r["topk_gate"].astype(np.float64)
        assert np.max(np.abs(g.sum(1) - 1.0)) <= K * 2.0 ** -24 * 2
        sel = np.take_along_axis(l.astype(np.float64), r["topk_idx"].astype(np.int64), 1)
        ref = np.exp(sel - sel.max(1, keepdims=True))
        ref /= ref.sum(1, keepdims=True)
        assert np.max(np.abs(g - ref)) < 1e-6
        if K == 1:
            assert np.all(g == 1.0)
            assert np.array_equal(r["topk_idx"][:, 0], np.argmax(l, 1))   # first max wins
        if K == E:
            assert np.array_equal(np.sort(r["topk_idx"], 1), np.tile(np.arange(E), (64, 1)))


# --------------------------------------------------------------------------------
# capacity, drops and maps
# --------------------------------------------------------------------------------

def test_capacity_values():
    assert oracle.capacity(4096, 2, 8, 1.0) == 1024
    assert oracle.capacity(4096, 8, 64, 1.0) == 512
    assert oracle.capacity(10, 1, 3, 1.0) == 4          # ceil(3.33)
    assert oracle.capacity(6, 2, 3, 1.0) == 4
    assert oracle.capacity(8, 2, 4, 0.0) == 0
    assert oracle.capacity(8, 2, 4, None) == -1
    assert oracle.capacity(8, 2, 4, 1.5) == 6


@pytest.mark.parametrize("name", sorted(os.listdir(GOLDEN)))
def test_golden_route(name):
    if not name.startswith("route_"):
        pytest.skip("not a routing fixture")
    g = json.load(open(os.path.join(GOLDEN, name)))
    assert oracle.capacity(g["S"], g["K"], g["E"], g["cf"]) == g["capacity"]
    r = oracle.route(np.array(g["logits"], np.float32), g["K"], g["S"], g["capacity"])
    for key in ("topk_idx", "keep", "row_of", "src_of", "routed_counts", "kept_counts",
                "offsets"):
        assert np.array_equal(np.asarray(r[key]), np.asarray(g[key])), key
    assert r["n_kept"] == g["n_kept"]
    assert np.max(np.abs(r["topk_gate"] - np.array(g["topk_gate"]))) <= g["gate_tol"]


def _brute_drop(cands, cap):
    """cands: list of (p, t, slot).  The kept set is the unique cap-subset whose members
    all beat all non-members under (p desc, t asc); found by enumeration."""
    if cap < 0 or len(cands) <= cap:
        return {c[2] for c in cands}
    hits = []
    for sub in itertools.combinations(range(len(cands)), cap):
        rest = [j for j in range(len(cands)) if j not in sub]
        ok = all(cands[i][0] > cands[j][0] or (cands[i][0] == cands[j][0] and
                                                  cands[i][1] < cands[j][1])
                 for i in sub for j in rest)
        if ok:
            hits.append({cands[i][2] for i in sub})
    assert len(hits) == 1
    return hits[0]


def test_drop_brute_force_tiny():
    rng = np.random.default_rng(4)
    for trial in range(200):
        E = int(rng.integers(2, 5))
        K = int(rng.integers(1, E + 1))
        S = int(rng.integers(1, 7))
        n_sub = int(rng.integers(1, 3))
        T = S * n_sub
        cap = int(rng.integers(0, 4))
        l = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        r = oracle.route(l, K, S, cap)
        keep = r["keep"]
        for s in range(n_sub):
            for e in range(E):
                cands = [(float(r["topk_prob"][t, k]), t, t * K + k)
                         for t in range(s * S, (s + 1) * S) for k in range(K)
                         if r["topk_idx"][t, k] == e]
                kept = {t * K + k for t in range(s * S, (s + 1) * S) for k in range(K)
                        if r["topk_idx"][t, k] == e and keep[t, k]}
                assert kept == _brute_drop(cands, cap)
                assert r["routed_counts"][s, e] == len(cands)
                assert len(kept) == min(len(cands), cap)


def _check_maps(r, T, K, E):
    keep = r["keep"].astype(bool)
    idx = r["topk_idx"]
    flat = [(idx[t, k], t, t * K + k) for t in range(T) for k in range(K) if keep[t, k]]
    # the kept assignments, stably sorted by expert, are exactly src_of
    order = np.argsort(np.array([a[0] for a in flat], np.int64), kind="stable")
    assert np.array_equal(r["src_of"], np.array([flat[i][2] for i in order], np.int32))
    # row_of is the inverse of src_of on kept slots, -1 elsewhere
    for t in range(T):
        for k in range(K):
            if keep[t, k]:
                assert r["src_of"][r["row_of"][t, k]] == t * K + k
            else:
                assert r["row_of"][t, k] == -1
    counts = np.bincount(np.array([a[0] for a in flat], np.int64), minlength=E)
    assert np.array_equal(r["kept_counts"], counts)
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert r["n_kept"] == len(flat)
    # each kept token appears exactly once per selected expert
    for e in range(E):
        seg = r["src_of"][r["offsets"][e]:r["offsets"][e + 1]] // K
        assert len(set(seg.tolist())) == len(seg)
        assert np.all(np.diff(seg) > 0)            # tokens ascending inside a segment


def test_maps_invariants_random():
    rng = np.random.default_rng(6)
    for (T, E, K, S, cf) in ((64, 4, 2, 64, None), (64, 8, 2, 32, 1.0), (96, 16, 4, 32, 1.0),
                             (48, 6, 3, 16, 0.5), (32, 4, 4, 8, 1.0)):
        l = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
        if cf is not None:
            l[:, 0] += 2.0                          # skew the load so drops happen
        cap = oracle.capacity(S, K, E, cf)
        r = oracle.route(l, K, S, cap)
        _check_maps(r, T, K, E)
        if cap >= 0:
            assert np.all(r["kept_counts"] <= cap * (T // S))


def test_drop_degenerate_capacities():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((40, 5)).astype(np.float32)
    free = oracle.route(l, 2, 8, -1)
    big = oracle.route(l, 2, 8, 8)                 # capacity >= S: nothing can be dropped
    for key in ("keep", "row_of", "src_of", "offsets"):
        assert np.array_equal(free[key], big[key])
    zero = oracle.route(l, 2, 8, 0)                # capacity 0: everything dropped
    assert zero["n_kept"] == 0 and np.all(zero["keep"] == 0) and np.all(zero["row_of"] == -1)
    assert np.array_equal(zero["offsets"], np.zeros(6, np.int32))


# --------------------------------------------------------------------------------
# The continuous path: a dense-masked formulation written here, in float64
# --------------------------------------------------------------------------------

def _silu(a):
    return a / (1.0 + np.exp(-a))


def _dense_layer(x, wr, bias, wg, wu, wd, sel, keepm, shared=None):
    """y_t = sum_e G_te FFN_e(x_t) with every expert evaluated on every token.
    sel [T,E]: 1 where e is one of the token's K chosen experts (held fixed);
    keepm [T,E]: 1 where that assignment survived the drop.  G_te = keepm * (softmax of
    the logits over the chosen experts).  Works for complex inputs (complex step)."""
    l = x @ wr
    if bias is not None:
        l = l + bias[None, :]
    el = np.exp(l) * sel
    G = el / el.sum(1, keepdims=True) * keepm
    y = 0
    for e in range(wr.shape[1]):
        ffn = (_silu(x @ wg[e]) * (x @ wu[e])) @ wd[e]
        y = y + G[:, e:e + 1] * ffn
    if shared is not None:
        w_sg, sg, su, sd = shared
        s = 1.0 / (1.0 + np.exp(-(x @ w_sg)))
        y = y + s[:, None] * ((_silu(x @ sg[0]) * (x @ su[0])) @ sd[0])
    return y


def _tiny_inputs(rng, T, d, E, f, fs=0, bias=False):
    inp = {
        "x": rng.standard_normal((T, d)),
        "w_router": rng.standard_normal((d, E)) * 0.5,
        "bias": rng.standard_normal(E) * 0.3 if bias else None,
        "w_gate": rng.standard_normal((E, d, f)) / math.sqrt(d),
        "w_up": rng.standard_normal((E, d, f)) / math.sqrt(d),
        "w_down": rng.standard_normal((E, f, d)) / math.sqrt(f),
        "dy": rng.standard_normal((T, d)),
    }
    if fs:
        inp["w_sg"] = rng.standard_normal(d) * 0.3
        inp["ws_gate"] = rng.standard_normal((1, d, fs)) / math.sqrt(d)
        inp["ws_up"] = rng.standard_normal((1, d, fs)) / math.sqrt(d)
        inp["ws_down"] = rng.standard_normal((1, fs, d)) / math.sqrt(fs)
    return inp


def _masks(r, T, E, K):
    sel = np.zeros((T, E))
    keepm = np.zeros((T, E))
    for t in range(T):
        for k in range(K):
            sel[t, r["topk_idx"][t, k]] = 1
            keepm[t, r["topk_idx"][t, k]] = r["keep"][t, k]
    return sel, keepm


CASES = [  # T, d, E, K, f, S, cf, fs, bias
    (24, 8, 4, 2, 6, 24, None, 0, False),
    (24, 8, 4, 2, 6, 12, 1.0, 0, True),
    (16, 6, 3, 1, 5, 8, 1.0, 0, False),
    (20, 8, 6, 3, 4, 20, None, 7, False),
    (12, 5, 1, 1, 7, 12, None, 0, False),       # E = K = 1: a dense SwiGLU MLP
]


@pytest.mark.parametrize("case", CASES)
def test_layer_forward_equals_dense_masked(case):
    T, d, E, K, f, S, cf, fs, bias = case
    rng = np.random.default_rng(11)
    inp = _tiny_inputs(rng, T, d, E, f, fs, bias)
    cap = oracle.capacity(S, K, E, cf)
    res = oracle.layer_fwd_bwd(inp, K, S, cap, "f64")
    r = res["routing"]
    sel, keepm = _masks(r, T, E, K)
    shared = (inp["w_sg"], inp["ws_gate"], inp["ws_up"], inp["ws_down"]) if fs else None
    y_ref = _dense_layer(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                         inp["w_down"], sel, keepm, shared)
    # the oracle's gates are fp32 (routing precision); everything else is float64
    scale = np.max(np.abs(y_ref))
    assert np.max(np.abs(res["y"] - y_ref)) / scale < 2e-6
    if E == 1:
        dense = (_silu(inp["x"] @ inp["w_gate"][0]) * (inp["x"] @ inp["w_up"][0])) @ inp["w_down"][0]
        assert np.max(np.abs(res["y"] - dense)) / np.max(np.abs(dense)) < 1e-12


def test_permute_unpermute_identity():
    rng = np.random.default_rng(12)
    T, d, E, K = 30, 5, 6, 3
    x = rng.standard_normal((T, d))
    l = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(l, K, T, -1)
    xp = oracle.permute(x, r["src_of"], K)
    y = oracle.unpermute(xp, r["row_of"], r["topk_gate"], r["keep"], "f64")
    assert np.max(np.abs(y - x)) < 1e-6                       # gates sum to 1
    ones = np.ones_like(r["topk_gate"])
    y1 = oracle.unpermute(xp, r["row_of"], ones, r["keep"], "f64")
    assert np.max(np.abs(y1 - K * x)) < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_backward_adjoint_complex_step(case):
    """<dy, J v> computed by the complex step through the dense formulation equals
    <oracle gradient, v> for a random direction v in every parameter."""
    T, d, E, K, f, S, cf, fs, bias = case
    rng = np.random.default_rng(13)
    inp = _tiny_inputs(rng, T, d, E, f, fs, bias)
    cap = oracle.capacity(S, K, E, cf)
    res = oracle.layer_fwd_bwd(inp, K, S, cap, "f64")
    r = res["routing"]
    sel, keepm = _masks(r, T, E, K)
    names = ["x", "w_router", "w_gate", "w_up", "w_down"]
    grads = {"x": res["dx"], "w_router": res["dw_router"], "w_gate": res["dw_gate"],
             "w_up": res["dw_up"], "w_down": res["dw_down"]}
    if fs:
        names += ["w_sg", "ws_gate", "ws_up", "ws_down"]
        grads.update({"w_sg": res["dw_sg"], "ws_gate": res["dws_gate"],
                      "ws_up": res["dws_up"], "ws_down": res["dws_down"]})
    h = 1e-30
    for name in names:
        v = rng.standard_normal(np.shape(inp[name]))
        args = {k: (np.asarray(inp[k], dtype=complex) if k in inp and inp[k] is not None
                    else None) for k in inp}
        args[name] = args[name] + 1j * h * v
        shared = (args["w_sg"], args["ws_gate"], args["ws_up"], args["ws_down"]) if fs else None
        y = _dense_layer(args["x"], args["w_router"], args["bias"], args["w_gate"],
                         args["w_up"], args["w_down"], sel, keepm, shared)
        jvp = np.sum(inp["dy"] * y).imag / h
        vjp = np.sum(grads[name] * v)
        assert abs(jvp - vjp) <= 2e-6 * (abs(jvp) + 1e-3), (name, jvp, vjp)


def test_backward_central_differences():
    """A few coordinates by central differences (routing held fixed)."""
    T, d, E, K, f, S, cf = 16, 6, 4, 2, 5, 8, 1.0
    rng = np.random.default_rng(14)
    inp = _tiny_inputs(rng, T, d, E, f, 0, True)
    cap = oracle.capacity(S, K, E, cf)
    res = oracle.layer_fwd_bwd(inp, K, S, cap, "f64")
    sel, keepm = _masks(res["routing"], T, E, K)
    grads = {"x": res["dx"], "w_router": res["dw_router"], "w_gate": res["dw_gate"],
             "w_up": res["dw_up"], "w_down": res["dw_down"]}

    def loss(p):
        y = _dense_layer(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"],
                         p["w_down"], sel, keepm)
        return float(np.sum(inp["dy"] * y))

    eps = 1e-6
    for name, g in grads.items():
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in np.shape(inp[name]))
            p1 = {k: (None if v is None else np.array(v, copy=True)) for k, v in inp.items()}
            p2 = {k: (None if v is None else np.array(v, copy=True)) for k, v in inp.items()}
            p1[name][idx] += eps
            p2[name][idx] -= eps
            fd = (loss(p1) - loss(p2)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, g[idx])


def test_bf16_storage_within_bound_of_f64():
    """With the same bf16-rounded inputs, the oracle that rounds its stored values to
    bf16 stays within the 2e-2 normwise bound of the unrounded float64 oracle, so the
    bound is reachable by a correct implementation."""
    rng = np.random.default_rng(15)
    T, d, E, K, f = 64, 32, 4, 2, 48
    inp = _tiny_inputs(rng, T, d, E, f, 40, False)
    for k, v in list(inp.items()):
        if v is not None:
            inp[k] = oracle.round_bf16(v)
    r64 = oracle.layer_fwd_bwd(inp, K, T, -1, "f64")
    rbf = oracle.layer_fwd_bwd(inp, K, T, -1, "bf16")
    for key in ("y", "dx", "dw_gate", "dw_up", "dw_down", "dw_router", "dws_gate", "dw_sg"):
        a, b = np.asarray(rbf[key], np.float64), np.asarray(r64[key], np.float64)
        err = np.max(np.abs(a - b)) / np.max(np.abs(b))
        assert err < 2e-2, (key, err)


def test_round_bf16_ties_to_even():
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20])
    out = oracle.round_bf16(vals)
    assert list(out) == [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7]


def test_column_restricted_ffn_equals_full():
    """The column versions used for sampled weight-gradient checks agree with the full
    (pinned) forward and backward."""
    rng = np.random.default_rng(16)
    T, d, E, K, f = 40, 12, 3, 2, 10
    inp = _tiny_inputs(rng, T, d, E, f)
    for k in list(inp):
        if inp[k] is not None:
            inp[k] = oracle.round_bf16(inp[k])
    res = oracle.layer_fwd_bwd(inp, K, T, -1, "bf16")
    r = res["routing"]
    cols = np.array([0, 3, 7, 9])
    for e in range(E):
        lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
        a, b, h = oracle.ffn_cols_fwd(res["xp"][lo:hi], inp["w_gate"][e], inp["w_up"][e], cols,
                                      "bf16")
        assert np.array_equal(a, res["a"][lo:hi][:, cols])
        assert np.array_equal(b, res["b"][lo:hi][:, cols])
        assert np.array_equal(h, res["h"][lo:hi][:, cols])
        da, db = oracle.ffn_cols_bwd(a, b, res["d_o"][lo:hi], inp["w_down"][e], cols, "bf16")
        dwg = oracle.round_bf16(res["xp"][lo:hi].T @ da)
        assert np.max(np.abs(dwg - res["dw_gate"][e][:, cols])) <= 1e-2 * np.max(np.abs(dwg))
        dwd = oracle.round_bf16(h.T @ res["d_o"][lo:hi])
        assert np.max(np.abs(dwd - res["dw_down"][e][cols, :])) <= 1e-2 * np.max(np.abs(dwd))


def test_expert_shards_reassemble_full_ffn():
    """One GPU's share of the experts under expert parallelism (a contiguous range of
    experts, rows from every source) and under expert-tensor parallelism (every expert,
    an ffn slice of each): in float64 the expert-range results are the full grouped FFN's
    rows and weight gradients, the ffn-slice results are its columns, and the slices'
    partial o and dxp sum to the full ones (the contraction over the ffn index splits
    into the slices)."""
    rng = np.random.default_rng(17)
    d, E, f, etp = 16, 4, 24, 3
    counts = np.array([7, 0, 11, 5])
    offs = np.concatenate([[0], np.cumsum(counts)])
    n = int(offs[-1])
    xp = rng.standard_normal((n, d))
    wg, wu = rng.standard_normal((E, d, f)), rng.standard_normal((E, d, f))
    wd = rng.standard_normal((E, f, d))
    d_o = rng.standard_normal((n, d))
    a, b, h, o = oracle.expert_ffn_fwd(xp, wg, wu, wd, offs, "f64")
    full = oracle.expert_ffn_bwd(xp, a, b, h, wg, wu, wd, offs, d_o, "f64")
    close = lambda u, v: np.allclose(u, v, rtol=1e-12, atol=1e-12 * np.max(np.abs(v)))

    # expert range [1, 3): segments 1 and 2 of the full layer
    lo, hi = int(offs[1]), int(offs[3])
    lo_offs = offs[1:4] - offs[1]
    ea, eb, eh, eo = oracle.expert_ffn_fwd(xp[lo:hi], wg[1:3], wu[1:3], wd[1:3], lo_offs, "f64")
    assert close(eo, o[lo:hi]) and close(eh, h[lo:hi])
    eg = oracle.expert_ffn_bwd(xp[lo:hi], ea, eb, eh, wg[1:3], wu[1:3], wd[1:3], lo_offs,
                               d_o[lo:hi], "f64")
    assert close(eg["dxp"], full["dxp"][lo:hi])
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert close(eg[k], full[k][1:3]), k
    assert np.all(eg["dw_gate"][0] == 0)          # expert 1 has no rows

    # ffn slices: columns of a, b, h and of the gate/up weight gradients, rows of
    # dW_down; o and dxp are partial sums
    o_sum = np.zeros_like(o)
    dxp_sum = np.zeros_like(full["dxp"])
    for r in range(etp):
        cols = slice(r * f // etp, (r + 1) * f // etp)
        sg, su, sd = wg[:, :, cols], wu[:, :, cols], wd[:, cols, :]
        sa, sb, sh, so = oracle.expert_ffn_fwd(xp, sg, su, sd, offs, "f64", o_storage="f64")
        assert close(sa, a[:, cols]) and close(sb, b[:, cols]) and close(sh, h[:, cols])
        sgr = oracle.expert_ffn_bwd(xp, sa, sb, sh, sg, su, sd, offs, d_o, "f64",
                                    dxp_storage="f64")
        assert close(sgr["dw_gate"], full["dw_gate"][:, :, cols])
        assert close(sgr["dw_up"], full["dw_up"][:, :, cols])
        assert close(sgr["dw_down"], full["dw_down"][:, cols, :])
        assert not close(so, o)                   # one slice alone is not the output
        o_sum += so
        dxp_sum += sgr["dxp"]
    assert close(o_sum, o)
    assert close(dxp_sum, full["dxp"])


def test_partial_outputs_keep_fp32():
    """With bf16 storage, o_storage / dxp_storage = "f32" rounds only those outputs to
    fp32: they differ from the bf16-stored ones by at most half a bf16 ulp of the value,
    and equal the fp32 rounding of the float64 product of the stored h (resp. da, db)."""
    rng = np.random.default_rng(18)
    d, f = 16, 32
    xp = oracle.round_bf16(rng.standard_normal((9, d)))
    wg, wu = oracle.round_bf16(rng.standard_normal((1, d, f)) * 0.3), oracle.round_bf16(
        rng.standard_normal((1, d, f)) * 0.3)
    wd = oracle.round_bf16(rng.standard_normal((1, f, d)) * 0.3)
    offs = np.array([0, 9])
    a, b, h, o16 = oracle.expert_ffn_fwd(xp, wg, wu, wd, offs, "bf16")
    _, _, _, o32 = oracle.expert_ffn_fwd(xp, wg, wu, wd, offs, "bf16", o_storage="f32")
    exact = h @ wd[0]
    assert np.array_equal(o32, exact.astype(np.float32).astype(np.float64))
    assert np.array_equal(o16, oracle.round_bf16(exact))
    assert np.all(np.abs(o16 - o32) <= np.abs(o32) * 2.0 ** -8 + 1e-30)
    d_o = oracle.round_bf16(rng.standard_normal((9, d)))
    g16 = oracle.expert_ffn_bwd(xp, a, b, h, wg, wu, wd, offs, d_o, "bf16")
    g32 = oracle.expert_ffn_bwd(xp, a, b, h, wg, wu, wd, offs, d_o, "bf16", dxp_storage="f32")
    assert np.array_equal(oracle.round_bf16(g32["dxp"]), g16["dxp"])
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(g16[k], g32[k]), k
