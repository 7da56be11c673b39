"""GPU parity of the expert FFN on one GPU's share of a layer spread over G GPUs.

Rows of G source GPUs are routed (one sub-sequence per source) and permuted; one GPU
then holds a range of experts (expert parallelism, rows from every source) or an
ffn slice of every expert (expert-tensor parallelism, whose o and dxp are fp32
partial sums that the exchange's ReduceScatter-V adds up).

Small shapes: each shard against the oracle element by element, and against the
unsharded GPU run: an expert range reproduces the full run's rows and weight
gradients bit for bit, an ffn slice reproduces its columns of a, b, h and of the
weight gradients bit for bit (same per-element accumulation order), and the slices'
partial o and dxp sum to the full ones.
Full-size Mixtral-8x22B shards (the launch configuration bench.py --shard times):
routing bit-exact, then sampled rows and weight-gradient entries against the oracle.
Tolerance: normwise max-abs-rel 2e-2 (bf16 storage, fp32 accumulate).
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import assert_close, host, log

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


SRC = moe_synth.LayerShape("shard_src", T=256, d=256, E=4, K=2, f=1024, seed=21, dtype="bf16",
                           cf=1.0, sub_seq=256, w_std=0.05, wr_std=0.3)
G = 4


def _routed_rows(src, G):
    """Oracle routing of G sources' tokens (sub-sequence = one source) and the permuted
    rows, all on the host."""
    tok = moe_synth.make_source_tokens(src, G)
    x = _f32(tok["x"])
    logits = oracle.router_logits(x, _f32(tok["w_router"]))
    cap = oracle.capacity(src.T, src.K, src.E, src.cf)
    r = oracle.route(logits, src.K, src.T, cap)
    xp = x[r["src_of"] // src.K]
    return xp, r["offsets"].astype(np.int64), r


def _run_shard(xp, offs, w, d_o, partial=False, flags=0):
    from token_dispatch_expert_router_amd.layer import ExpertShard
    E, d, f = w["w_gate"].shape
    n = xp.shape[0]
    sh = ExpertShard(n, d, E, f, torch.bfloat16, partial=partial, device="cuda", flags=flags)
    xg = torch.as_tensor(xp, dtype=torch.float32).to(torch.bfloat16).cuda()
    og = torch.as_tensor(np.asarray(offs), dtype=torch.int32).cuda()
    sh.forward(xg, w, og)
    sh.backward(xg, w, og, d_o)
    torch.cuda.synchronize()
    return sh


def _oracle_shard(xp, offs, w, d_o, partial):
    wg, wu, wd = _f32(w["w_gate"]), _f32(w["w_up"]), _f32(w["w_down"])
    ps = "f32" if partial else None
    a, b, h, o = oracle.expert_ffn_fwd(xp, wg, wu, wd, offs, "bf16", o_storage=ps)
    g = oracle.expert_ffn_bwd(xp, a, b, h, wg, wu, wd, offs, _f32(d_o), "bf16", dxp_storage=ps)
    return {"a": a, "b": b, "h": h, "o": o, **g}


def _check_oracle(tag, sh, ref):
    n = ref["o"].shape[0]
    for k in ("a", "b", "h", "o", "dxp"):
        assert_close(f"{tag} {k}", _f32(sh.buf[k][:n]), ref[k], TOL)
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert_close(f"{tag} {k}", _f32(sh.buf[k]), ref[k], TOL)


@pytest.fixture(scope="module")
def full_run():
    xp, offs, r = _routed_rows(SRC, G)
    shard = moe_synth.ShardShape("full", SRC.name, G=G, e0=0, e1=SRC.E)
    w = moe_synth.make_shard_weights(shard, device="cuda", layer=SRC)
    d_o = moe_synth.make_shard_grad(shard, xp.shape[0], device="cuda", layer=SRC)
    log(f"  {G} sources x {SRC.T} tokens: {xp.shape[0]} rows, per expert "
        f"{np.diff(offs).tolist()}")
    sh = _run_shard(xp, offs, w, d_o)
    return xp, offs, w, d_o, sh


def test_full_expert_set_parity(full_run):
    xp, offs, w, d_o, sh = full_run
    _check_oracle("full", sh, _oracle_shard(xp, offs, w, d_o, False))


@pytest.mark.parametrize("e0,e1", [(1, 3), (0, 1), (3, 4)])
def test_expert_range_is_bit_exact_slice(full_run, e0, e1):
    xp, offs, w, d_o, full = full_run
    lo, hi = int(offs[e0]), int(offs[e1])
    sub = {k: v[e0:e1].contiguous() for k, v in w.items()}
    sh = _run_shard(xp[lo:hi], offs[e0:e1 + 1] - offs[e0], sub, d_o[lo:hi].contiguous())
    for k in ("a", "b", "h", "o", "dxp"):
        assert torch.equal(sh.buf[k][:hi - lo], full.buf[k][lo:hi]), k
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert torch.equal(sh.buf[k], full.buf[k][e0:e1]), k


@pytest.mark.parametrize("etp", [2, 4])
def test_ffn_slices_reassemble_full(full_run, etp):
    xp, offs, w, d_o, full = full_run
    n = xp.shape[0]
    f = SRC.f
    fl = f // etp
    o_sum = torch.zeros((n, SRC.d), dtype=torch.float64, device="cuda")
    dxp_sum = torch.zeros_like(o_sum)
    for rank in range(etp):
        c = slice(rank * fl, (rank + 1) * fl)
        sw = {"w_gate": w["w_gate"][:, :, c].contiguous(), "w_up": w["w_up"][:, :, c].contiguous(),
              "w_down": w["w_down"][:, c, :].contiguous()}
        sh = _run_shard(xp, offs, sw, d_o, partial=True)
        assert sh.buf["o"].dtype == torch.float32 and sh.buf["dxp"].dtype == torch.float32
        for k in ("a", "b", "h"):
            assert torch.equal(sh.buf[k][:n], full.buf[k][:n, c]), (rank, k)
        assert torch.equal(sh.buf["dw_gate"], full.buf["dw_gate"][:, :, c]), rank
        assert torch.equal(sh.buf["dw_up"], full.buf["dw_up"][:, :, c]), rank
        assert torch.equal(sh.buf["dw_down"], full.buf["dw_down"][:, c, :]), rank
        if rank == 0:
            _check_oracle(f"etp{etp} rank0", sh, _oracle_shard(xp, offs, sw, d_o, True))
        o_sum += sh.buf["o"][:n].double()
        dxp_sum += sh.buf["dxp"][:n].double()
    ref = _oracle_shard(xp, offs, w, d_o, False)
    assert_close(f"etp{etp} sum o", o_sum.cpu().numpy(), ref["o"], TOL)
    assert_close(f"etp{etp} sum dxp", dxp_sum.cpu().numpy(), ref["dxp"], TOL)
    # the sum of fp32 partials rounds once; the unsharded run rounds o to bf16
    assert_close(f"etp{etp} sum o vs full", o_sum.cpu().numpy(), _f32(full.buf["o"][:n]), 1e-2)


def test_partial_slice_on_vector_alu(full_run):
    """An ffn slice that the matrix-core kernel does not tile (f_local = 136) and a forced
    vector-ALU run: fp32 partial outputs from the vector-ALU GEMMs."""
    from token_dispatch_expert_router_amd import _lib as L
    xp, offs, w, d_o, _ = full_run
    for c, flags in ((slice(0, 136), 0), (slice(256, 512), L.MOE_FLAG_VALU_GEMM)):
        sw = {"w_gate": w["w_gate"][:, :, c].contiguous(), "w_up": w["w_up"][:, :, c].contiguous(),
              "w_down": w["w_down"][:, c, :].contiguous()}
        sh = _run_shard(xp, offs, sw, d_o, partial=True, flags=flags)
        _check_oracle(f"valu {c.start}:{c.stop}", sh, _oracle_shard(xp, offs, sw, d_o, True))


def test_shard_without_rows():
    """A GPU whose experts received no rows: zero weight gradients, nothing else written."""
    from token_dispatch_expert_router_amd.layer import ExpertShard
    shard = moe_synth.ShardShape("empty", SRC.name, G=1, e0=0, e1=2, etp=4)
    w = moe_synth.make_shard_weights(shard, device="cuda", layer=SRC)
    sh = ExpertShard(0, SRC.d, 2, SRC.f // 4, torch.bfloat16, partial=True, device="cuda")
    for k in ("dw_gate", "dw_up", "dw_down"):
        sh.buf[k].fill_(1.0)
    og = torch.zeros(3, dtype=torch.int32, device="cuda")
    sh.forward(None, w, og)
    sh.backward(None, w, og, None)
    torch.cuda.synchronize()
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert torch.count_nonzero(sh.buf[k]) == 0, k


# --------------------------------------------------------------------------------------
# Full-size Mixtral-8x22B shards
# --------------------------------------------------------------------------------------

def shard_setup(s, device="cuda"):
    """Route and permute the G sources' tokens on the GPU and cut out this GPU's rows
    (the steps bench.py --shard takes before timing)."""
    from token_dispatch_expert_router_amd import _lib as L
    from token_dispatch_expert_router_amd.layer import Dispatch, expert_rows
    src = s.layer
    cap = L.moe_capacity(src.T, src.K, src.E, src.cf) if src.cf is not None else -1
    tok = moe_synth.make_source_tokens(src, s.G, device=device)
    dp = Dispatch(s.G * src.T, src.d, src.E, src.K, src.T, cap, src.torch_dtype, device=device)
    dp.run(tok["x"], tok["w_router"], tok["bias"])
    xp, loc = expert_rows(dp, s.e0, s.e1)
    return tok, dp, cap, xp, loc


@pytest.mark.parametrize("name", [s.name for s in moe_synth.SHARDS])
def test_fullsize_shard_parity(name):
    from token_dispatch_expert_router_amd.layer import ExpertShard
    s = moe_synth.shard_by_name(name)
    src = s.layer
    tok, dp, cap, xp, loc = shard_setup(s)
    torch.cuda.synchronize()
    ref_r = oracle.route(host(dp.logits), src.K, src.T, cap)
    for k in ("topk_idx", "keep", "row_of", "offsets", "kept_counts"):
        assert np.array_equal(host(dp.rt[k]), ref_r[k]), k
    x = tok["x"]
    n = xp.shape[0]
    offs = host(loc).astype(np.int64)
    log(f"  {name}: {s.G} x {src.T} tokens, experts [{s.e0}, {s.e1}) slice {s.cols} "
        f"-> {n} rows, per expert {np.diff(offs).tolist()}")
    lo = int(ref_r["offsets"][s.e0])
    src_rows = ref_r["src_of"][lo:lo + n] // src.K
    rng = np.random.default_rng(src.seed + 100)
    samp = rng.choice(n, size=8, replace=False)
    assert np.array_equal(_f32(xp[torch.as_tensor(samp, device="cuda")]),
                          _f32(x[torch.as_tensor(src_rows[samp], device="cuda")]))

    w = moe_synth.make_shard_weights(s, device="cuda")
    d_o = moe_synth.make_shard_grad(s, n, device="cuda")
    partial = s.etp > 1
    sh = ExpertShard(n, src.d, s.E_local, s.f_local, torch.bfloat16, partial=partial,
                     device="cuda")
    sh.forward(xp, w, loc)
    sh.backward(xp, w, loc, d_o)
    torch.cuda.synchronize()
    b = sh.buf
    ps = "f32" if partial else None

    rows = np.sort(rng.choice(n, size=48, replace=False))
    seg = np.searchsorted(offs, rows, side="right") - 1
    got = {k: [] for k in ("a", "b", "h", "o", "dxp")}
    exp = {k: [] for k in got}
    xs_all = _f32(xp[torch.as_tensor(rows, device="cuda")])
    do_all = _f32(d_o[torch.as_tensor(rows, device="cuda")])
    for e in sorted(set(seg.tolist())):
        sel = seg == e
        wg, wu, wd = _f32(w["w_gate"][e]), _f32(w["w_up"][e]), _f32(w["w_down"][e])
        a, bb, h, o = oracle.ffn_rows_fwd(xs_all[sel], wg, wu, wd, "bf16", o_storage=ps)
        _, _, dxp = oracle.ffn_rows_bwd_data(a, bb, do_all[sel], wg, wu, wd, "bf16",
                                             dxp_storage=ps)
        idx = torch.as_tensor(rows[sel], device="cuda")
        for k, v in (("a", a), ("b", bb), ("h", h), ("o", o), ("dxp", dxp)):
            got[k].append(_f32(b[k][idx]))
            exp[k].append(v)
        del wg, wu, wd
    for k in got:
        assert_close(f"{name} {k}_rows", np.concatenate(got[k]), np.concatenate(exp[k]), TOL)

    # weight-gradient entries of the first and the last local expert (whole segments)
    for e in sorted({0, s.E_local - 1}):
        lo_e, hi_e = int(offs[e]), int(offs[e + 1])
        xs = _f32(xp[lo_e:hi_e])
        de = _f32(d_o[lo_e:hi_e])
        wg, wu, wd = _f32(w["w_gate"][e]), _f32(w["w_up"][e]), _f32(w["w_down"][e])
        ci = rng.choice(src.d, size=6, replace=False)
        cj = rng.choice(s.f_local, size=6, replace=False)
        a, bb, h = oracle.ffn_cols_fwd(xs, wg, wu, cj, "bf16")
        da, db = oracle.ffn_cols_bwd(a, bb, de, wd, cj, "bf16")
        ii, jj = np.meshgrid(ci, cj, indexing="ij")
        assert_close(f"{name} dW_gate[{e}]", _f32(b["dw_gate"][e])[ii, jj],
                     oracle.round_bf16(xs[:, ci].T.astype(np.float64) @ da), TOL)
        assert_close(f"{name} dW_up[{e}]", _f32(b["dw_up"][e])[ii, jj],
                     oracle.round_bf16(xs[:, ci].T.astype(np.float64) @ db), TOL)
        assert_close(f"{name} dW_down[{e}]", _f32(b["dw_down"][e])[jj.T, ii.T],
                     oracle.round_bf16(h.T @ de[:, ci]), TOL)
        del xs, wg, wu, wd
    del sh, dp, tok, w
    torch.cuda.empty_cache()
