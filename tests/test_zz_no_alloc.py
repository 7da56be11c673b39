"""moe_route_noalloc (the route call with the library's fixed scratch instead of a
caller workspace) against moe_route on the same inputs, through the C ABI: logits, the
shared-gate logit and every routing output must be bit-identical.  Two calls in a row,
the second on a smaller layer with a different expert count, so a result that leaned on
what the first call left in the scratch would show."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import ROUTING_KEYS, host, log

pytestmark = pytest.mark.gpu


def _shape(name, **kw):
    base = dict(T=256, d=256, E=4, K=2, f=256, seed=40, dtype="bf16", cf=1.0, sub_seq=256,
                w_std=0.05, wr_std=0.3)
    base.update(kw)
    return moe_synth.LayerShape(name, **base)


CALLS = [
    # matrix-core router (d % 256 == 0), two sub-sequences with drops, a shared gate
    _shape("noalloc_big", T=2048, d=512, E=16, K=4, sub_seq=1024, fs=256, seed=41),
    # smaller, fewer experts, one sub-sequence, vector-ALU router (d % 128 != 0)
    _shape("noalloc_small", T=384, d=200, E=6, K=2, sub_seq=384, seed=42),
]


def _routing_bufs(T, E, K, R, n_sub, dev):
    i32, f32 = torch.int32, torch.float32

    def z(shape, t):
        return torch.full(shape, -7, dtype=t, device=dev) if t != torch.uint8 else \
            torch.full(shape, 7, dtype=t, device=dev)

    return {"topk_idx": z((T, K), i32), "topk_prob": z((T, K), f32),
            "topk_gate": z((T, K), f32), "keep": z((T, K), torch.uint8),
            "row_of": z((T, K), i32), "src_of": z((max(R, 1),), i32),
            "routed_counts": z((max(n_sub, 1), E), i32), "kept_counts": z((E,), i32),
            "offsets": z((E + 1,), i32), "n_kept": z((1,), i32)}


def _route(L, s, inp, noalloc):
    cap = oracle.capacity(s.sub_seq, s.K, s.E, s.cf)
    code = L.MOE_BF16 if s.dtype == "bf16" else L.MOE_F32
    desc = L.make_desc(s.T, s.d, s.E, s.K, s.f, s.sub_seq, cap, code)
    R = L.moe_max_rows(desc)
    rt = _routing_bufs(s.T, s.E, s.K, R, s.T // s.sub_seq, "cuda")
    routing = L.make_routing(rt)
    logits = torch.full((s.T, s.E), -3.0, dtype=torch.float32, device="cuda")
    sg = torch.full((s.T,), -3.0, dtype=torch.float32, device="cuda") if s.fs else None
    w_sg = inp.get("w_sg") if s.fs else None
    if noalloc:
        L.moe_route_noalloc(desc, inp["x"], inp["w_router"], inp["bias"], w_sg, logits, sg,
                            routing)
    else:
        n = L.moe_workspace_size(desc, L.MOE_WS_ROUTE)
        ws = torch.empty((max(n, 1),), dtype=torch.uint8, device="cuda")
        L.moe_route(desc, inp["x"], inp["w_router"], inp["bias"], w_sg, logits, sg, routing, ws)
    torch.cuda.synchronize()
    out = {k: host(v) for k, v in rt.items()}
    out["logits"] = host(logits)
    if sg is not None:
        out["sg_logit"] = host(sg)
    out["n"] = int(out["n_kept"][0])
    return out, cap


def _same(a, b):
    if a.dtype.kind == "f":
        return np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return np.array_equal(a, b)


def test_noalloc_route_matches_route_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_dispatch_expert_router_amd import _lib as L
    L.load()
    for s in CALLS:
        inp = moe_synth.make_inputs(s, device="cuda")
        ref, cap = _route(L, s, inp, noalloc=False)
        got, _ = _route(L, s, inp, noalloc=True)
        log(f"  {s.name}: T={s.T} d={s.d} E={s.E} K={s.K} S={s.sub_seq} cap={cap} "
            f"n_kept={got['n']}")
        assert got["n"] == ref["n"]
        assert 0 < ref["n"] < s.T * s.K, "the case should drop some assignments"
        for k in ROUTING_KEYS + ("n_kept", "logits") + (("sg_logit",) if s.fs else ()):
            assert _same(got[k], ref[k]), f"{s.name}: {k} differs from moe_route"
        assert np.array_equal(got["src_of"][:got["n"]], ref["src_of"][:ref["n"]]), "src_of"
        # and the routing is the oracle's on those logits (bit for bit)
        orc = oracle.route(got["logits"], s.K, s.sub_seq, cap)
        for k in ("topk_idx", "keep", "row_of", "offsets"):
            assert np.array_equal(got[k], np.asarray(orc[k])), f"{s.name}: {k} vs oracle"
