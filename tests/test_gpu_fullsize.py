"""GPU parity at the full layer sizes, in the launch configuration bench.py times.

For each bf16 layer shape (Mixtral-8x22B, Qwen2-57B-A14B with its shared expert,
Mixtral-8x22B-G8T8 with the Zipf bias, Llama3-8x70B one GPU's share, and Mixtral
dimensions over 16384 tokens dropped per 4096-token sub-sequence or over the full
sequence):
  - routing over all tokens: the oracle routes the GPU's logits and must match bit for bit;
  - logits of sampled tokens against the oracle's float64 GEMM;
  - the permuted buffer is an exact copy of x on sampled rows;
  - for sampled tokens, every kept (token, expert) row: a, b, h, o, dxp against the
    oracle computed row by row, then y, dgate, dlogits and dx of those tokens;
  - sampled entries of dW_gate, dW_up, dW_down of two experts (whole-segment columns);
  - dW_router over all tokens from the GPU's dlogits (the router wgrad given its input).
Tolerance: normwise max-abs-rel 2e-2 over each sampled set (bf16 storage, fp32 accumulate).
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import assert_close, assert_routing_equal, host, log

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_dispatch_expert_router_amd import _lib as L
    L.load()


def _f32(t):
    return t.float().cpu().numpy()


def _pick_tokens(topk, keep, E, rng):
    """Tokens whose kept experts all lie in a small expert set (few weights to convert)."""
    T, K = topk.shape
    if E <= 8:
        want = {0, 1}
        cand = [t for t in range(T) if all((not keep[t, k]) or topk[t, k] in want for k in range(K))
                and keep[t].any()]
        dropped = [t for t in cand if not keep[t].all()]
        picked = list(rng.choice(cand, size=min(6, len(cand)), replace=False))
        if dropped:
            picked.append(dropped[0])
        return sorted(set(int(t) for t in picked))
    return sorted(int(t) for t in rng.choice(T, size=3, replace=False))


@pytest.mark.parametrize("name", ["mixtral_8x22b", "qwen2_57b_a14b", "mixtral_g8t8",
                                  "llama3_8x70b", "mixtral_t16k_s4k", "mixtral_t16k_full"])
def test_fullsize_parity(name):
    from token_dispatch_expert_router_amd.layer import MoELayer
    s = moe_synth.shape_by_name(name)
    cap = oracle.capacity(s.sub_seq, s.K, s.E, s.cf)
    log(f"  full-size {name}: T={s.T} d={s.d} E={s.E} K={s.K} f={s.f} fs={s.fs} cap={cap}")
    inp = moe_synth.make_inputs(s, device="cuda")
    lay = MoELayer(s.T, s.d, s.E, s.K, s.f, s.sub_seq, cap, torch.bfloat16, fs=s.fs,
                   device="cuda")
    lay.forward_backward(inp)
    torch.cuda.synchronize()
    b = lay.buf
    rng = np.random.default_rng(s.seed)

    # routing over all tokens, from the GPU's logits
    gl = host(b["logits"])
    ref_r = oracle.route(gl, s.K, s.sub_seq, cap)
    assert_routing_equal(lay, ref_r)
    n_kept = ref_r["n_kept"]
    log(f"    n_kept {n_kept} of {s.T * s.K}; kept per expert "
        f"{ref_r['kept_counts'].min()}..{ref_r['kept_counts'].max()}")

    x = _f32(inp["x"])
    dy = _f32(inp["dy"])
    wr = _f32(inp["w_router"])
    bias = None if inp["bias"] is None else host(inp["bias"])
    ts = rng.choice(s.T, size=64, replace=False)
    assert_close("logits", gl[ts], oracle.router_logits(x[ts], wr, bias), 2e-5)

    rows = rng.choice(n_kept, size=64, replace=False)
    xp_rows = _f32(b["xp"][torch.as_tensor(rows, device="cuda")])
    assert np.array_equal(xp_rows, x[ref_r["src_of"][rows] // s.K]), "permute is not an exact copy"

    # sampled tokens, row by row
    topk, keep, row_of, gate = ref_r["topk_idx"], ref_r["keep"], ref_r["row_of"], ref_r["topk_gate"]
    toks = _pick_tokens(topk, keep.astype(bool), s.E, rng)
    pairs = [(t, k) for t in toks for k in range(s.K) if keep[t, k]]
    experts = sorted({int(topk[t, k]) for t, k in pairs})
    log(f"    sampled tokens {toks} -> {len(pairs)} rows over experts {experts}")
    o_ref, dxp_ref = {}, {}
    got = {k: [] for k in ("a", "b", "h", "o", "dxp")}
    exp = {k: [] for k in ("a", "b", "h", "o", "dxp")}
    for e in experts:
        wg, wu, wd = _f32(inp["w_gate"][e]), _f32(inp["w_up"][e]), _f32(inp["w_down"][e])
        pe = [(t, k) for t, k in pairs if topk[t, k] == e]
        xr = x[[t for t, _ in pe]]
        a, bb, h, o = oracle.ffn_rows_fwd(xr, wg, wu, wd, "bf16")
        d_o = oracle.round_bf16(np.array([gate[t, k] for t, k in pe])[:, None] * dy[[t for t, _ in pe]])
        da, db, dxp = oracle.ffn_rows_bwd_data(a, bb, d_o, wg, wu, wd, "bf16")
        ridx = torch.as_tensor([int(row_of[t, k]) for t, k in pe], device="cuda")
        for key, ref_v in (("a", a), ("b", bb), ("h", h), ("o", o), ("dxp", dxp)):
            got[key].append(_f32(b[key][ridx]))
            exp[key].append(ref_v)
        for n_, (t, k) in enumerate(pe):
            o_ref[(t, k)] = o[n_]
            dxp_ref[(t, k)] = dxp[n_]
        del wg, wu, wd
    for key in got:
        assert_close(key + "_rows", np.concatenate(got[key]), np.concatenate(exp[key]), TOL)

    shared_ref = z_ref = dxs_ref = None
    if s.fs:
        z_ref = oracle.shared_gate_logit(x[toks], _f32(inp["w_sg"]), "f32")
        assert_close("sg_logit", host(b["sg_logit"])[toks], z_ref, 2e-5)
        sg, su, sd = _f32(inp["ws_gate"][0]), _f32(inp["ws_up"][0]), _f32(inp["ws_down"][0])
        sa, sb, sh, shared_ref = oracle.ffn_rows_fwd(x[toks], sg, su, sd, "bf16")
        assert_close("shared_rows", host(b["shared"])[toks], shared_ref, TOL)
        s_ = oracle.sigmoid(z_ref.astype(np.float64))
        dsh = oracle.round_bf16(s_[:, None] * dy[toks])
        _, _, dxs_ref = oracle.ffn_rows_bwd_data(sa, sb, dsh, sg, su, sd, "bf16")
        assert_close("dx_shared", host(b["dx_shared"])[toks], dxs_ref, TOL)

    # y, dgate, dlogits, dx of the sampled tokens
    y_ref = np.zeros((len(toks), s.d))
    dg_ref = np.zeros((len(toks), s.K))
    dx_ref = np.zeros((len(toks), s.d))
    for n_, t in enumerate(toks):
        for k in range(s.K):
            if keep[t, k]:
                y_ref[n_] += gate[t, k] * o_ref[(t, k)]
                dg_ref[n_, k] = float(np.dot(dy[t], o_ref[(t, k)]))
                dx_ref[n_] += dxp_ref[(t, k)]
    if s.fs:
        s_ = oracle.sigmoid(z_ref.astype(np.float64))
        y_ref += s_[:, None] * shared_ref
        dz = np.sum(dy[toks] * shared_ref, axis=1) * s_ * (1 - s_)
        dx_ref += dz[:, None] * _f32(inp["w_sg"])[None, :] + dxs_ref
    dl_ref = oracle.router_dlogits(topk[toks], gate[toks], dg_ref, s.E, "f64")
    dx_ref += dl_ref @ wr.T.astype(np.float64)
    assert_close("y_tokens", host(b["y"])[toks], y_ref, TOL)
    assert_close("dgate_tok", host(b["dgate"])[toks], dg_ref, TOL)
    assert_close("dlogits_tok", host(b["dlogits"])[toks], dl_ref, TOL)
    assert_close("dx_tokens", host(b["dx"])[toks], dx_ref, TOL)

    # sampled weight-gradient entries of two experts (whole segments)
    counts = ref_r["kept_counts"]
    e_big = int(np.argmax(counts))
    e_small = int(np.argmin(counts))
    for e in sorted({e_big, e_small}):
        lo, hi = int(ref_r["offsets"][e]), int(ref_r["offsets"][e + 1])
        src = ref_r["src_of"][lo:hi]
        tt, kk = src // s.K, src % s.K
        xs = x[tt]
        d_o = oracle.round_bf16(gate[tt, kk][:, None] * dy[tt])
        wg, wu, wd = _f32(inp["w_gate"][e]), _f32(inp["w_up"][e]), _f32(inp["w_down"][e])
        ci = rng.choice(s.d, size=6, replace=False)     # rows of dW_gate/dW_up, cols of dW_down
        cj = rng.choice(s.f, size=6, replace=False)     # cols of dW_gate/dW_up, rows of dW_down
        a, bb, h = oracle.ffn_cols_fwd(xs, wg, wu, cj, "bf16")
        da, db = oracle.ffn_cols_bwd(a, bb, d_o, wd, cj, "bf16")
        dwg_ref = oracle.round_bf16(xs[:, ci].T.astype(np.float64) @ da)
        dwu_ref = oracle.round_bf16(xs[:, ci].T.astype(np.float64) @ db)
        dwd_ref = oracle.round_bf16(h.T @ d_o[:, ci])
        ii, jj = np.meshgrid(ci, cj, indexing="ij")
        got_g = _f32(b["dw_gate"][e])[ii, jj]
        got_u = _f32(b["dw_up"][e])[ii, jj]
        got_d = _f32(b["dw_down"][e])[jj.T, ii.T]
        log(f"    expert {e}: {hi - lo} rows")
        if hi == lo:
            assert np.all(got_g == 0) and np.all(got_u == 0) and np.all(got_d == 0)
            continue
        assert_close(f"dW_gate[{e}]", got_g, dwg_ref, TOL)
        assert_close(f"dW_up[{e}]", got_u, dwu_ref, TOL)
        assert_close(f"dW_down[{e}]", got_d, dwd_ref, TOL)

    # router weight gradient from the GPU's dlogits (and dz)
    dwr_ref = oracle.router_wgrad(x, host(b["dlogits"]), "bf16")
    assert_close("dW_router", host(b["dw_router"]), dwr_ref, TOL)
    if s.fs:
        dwsg_ref = oracle.round_bf16(x.T.astype(np.float64) @ host(b["dz"]).astype(np.float64))
        assert_close("dw_sg", host(b["dw_sg"]), dwsg_ref, TOL)
    del lay, inp
    torch.cuda.empty_cache()
