"""GPU parity of the HIP MoE layer against the CPU oracle, element by element, on
shapes the oracle finishes in seconds that still span several GEMM tiles and ragged
segment tails.  Routing outputs are bit-exact; continuous outputs are within the
normwise max-abs-rel bound (1e-5 fp32, 2e-2 bf16)."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import assert_close, assert_routing_equal, check_layer, host, log

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_dispatch_expert_router_amd import _lib as L
    L.load()
    return L


def _shape(name, **kw):
    base = dict(T=256, d=64, E=4, K=2, f=128, seed=10, dtype="bf16", cf=None, sub_seq=256,
                w_std=0.05, wr_std=0.3)
    base.update(kw)
    return moe_synth.LayerShape(name, **base)


def _run(shape, flags=0, bias=None):
    from token_dispatch_expert_router_amd.layer import MoELayer
    inp = moe_synth.make_inputs(shape, device="cuda")
    if bias is not None:
        inp["bias"] = torch.tensor(bias, dtype=torch.float32, device="cuda")
    cap = oracle.capacity(shape.sub_seq, shape.K, shape.E, shape.cf)
    lay = MoELayer(shape.T, shape.d, shape.E, shape.K, shape.f, shape.sub_seq, cap,
                   shape.torch_dtype, fs=shape.fs, device="cuda", flags=flags)
    log(f"  case {shape.name}: T={shape.T} d={shape.d} E={shape.E} K={shape.K} f={shape.f} "
        f"S={shape.sub_seq} cap={cap} fs={shape.fs} flags={flags}")
    lay.forward_backward(inp)
    torch.cuda.synchronize()
    return lay, inp, cap


CASES = {
    # fp32 tiny layer of the benchmark list (vector-ALU GEMMs)
    "tiny_fp32": moe_synth.shape_by_name("tiny"),
    # bf16 on the matrix cores: 2 sub-sequences, capacity drops, ragged segments
    "mfma_drop": _shape("mfma_drop", T=1024, d=512, E=4, K=2, f=768, sub_seq=512, cf=1.0,
                        seed=11),
    # bf16 dropless on the matrix cores, more experts, K=4
    "mfma_dropless": _shape("mfma_dropless", T=768, d=256, E=8, K=4, f=512, seed=12),
    # bf16 shape the matrix-core kernel does not tile: vector-ALU fallback
    "valu_odd": _shape("valu_odd", T=96, d=136, E=3, K=2, f=200, sub_seq=32, cf=1.0, seed=13),
    # shared expert with a sigmoid gate
    "shared": _shape("shared", T=512, d=256, E=8, K=2, f=256, fs=512, seed=14, w_std=0.05),
    # 64 experts plus the shared gate: the gate logit is column 64 (past the last lane)
    "shared_e64": _shape("shared_e64", T=256, d=256, E=64, K=8, f=256, fs=256, seed=19,
                         w_std=0.05),
    # the same on the vector-ALU router (d not a multiple of 128)
    "shared_e64_valu": _shape("shared_e64_valu", T=128, d=200, E=64, K=4, f=136, fs=72, sub_seq=128,
                              seed=20, w_std=0.05),
    # fp32 with a shared expert and sharp gates: the shared gate's derivative and every
    # shared-expert output and gradient held to the fp32 bound
    "fp32_shared": _shape("fp32_shared", T=320, d=96, E=8, K=2, f=64, fs=48, sub_seq=160,
                          cf=1.0, seed=39, dtype="f32", w_std=0.05, wr_std=0.5),
    # fp32 with 16 experts (the router weight gradient's many-column kernel, in fp32)
    "fp32_e16": _shape("fp32_e16", T=192, d=72, E=16, K=4, f=40, sub_seq=64, cf=1.0, seed=21,
                       dtype="f32", w_std=None, wr_std=0.5),
    # d % 256 == 128: the router GEMM splits d over 4 waves (the expert GEMMs take the
    # vector-ALU path)
    "d384": _shape("d384", T=320, d=384, E=8, K=2, f=128, sub_seq=160, cf=1.0, seed=23),
    # 32 experts, dropless
    "e32": _shape("e32", T=256, d=256, E=32, K=4, f=256, seed=22, w_std=0.05),
    # one expert, top-1: a dense SwiGLU MLP
    "dense": _shape("dense", T=300, d=256, E=1, K=1, f=512, sub_seq=300, seed=15),
    # segments of about 320 rows: every expert's last row tile holds 40-90 valid rows
    "short_tail": _shape("short_tail", T=1280, d=512, E=8, K=2, f=1024, seed=24, w_std=0.05),
    # segments of 50-80 rows: one mostly empty row tile per expert
    "short_segments": _shape("short_segments", T=512, d=512, E=16, K=2, f=512, seed=25,
                             w_std=0.05),
    # slot counts between the kernels' compile-time bounds (2, 4, 8): K = 3 with drops,
    # K = 5 dropless (8 experts: the permute backward's slice form), K = 6 with 20 experts
    # (its one-wave-per-token form), and K = 2 with 24 experts (that form's smallest bound)
    "k3_drop": _shape("k3_drop", T=256, d=256, E=6, K=3, f=256, sub_seq=128, cf=1.0, seed=31,
                      w_std=0.05),
    "k5_e8": _shape("k5_e8", T=192, d=256, E=8, K=5, f=256, sub_seq=192, seed=32, w_std=0.05),
    "k6_e20_drop": _shape("k6_e20_drop", T=128, d=256, E=20, K=6, f=256, sub_seq=64, cf=1.0,
                          seed=33, w_std=0.05),
    "k2_e24": _shape("k2_e24", T=256, d=256, E=24, K=2, f=256, seed=34, w_std=0.05),
    # router GEMM with three 16-column blocks, the 4-wave split of d (d % 256 != 0, five
    # k-steps per wave: a partial batch) and a last block of 8 tokens
    "e40_t200": _shape("e40_t200", T=200, d=640, E=40, K=4, f=256, sub_seq=200, seed=35,
                       w_std=0.05),
    # every expert chosen by every token (K = E): the gates are the whole softmax
    "k_eq_e": _shape("k_eq_e", T=256, d=256, E=4, K=4, f=256, seed=36, w_std=0.05),
    # fp32, two experts, sharp gates (one gate within a few ulps of 1 for some tokens) and
    # heavy drops: the router gradient g (dgate - sum g dgate) cancels, which fp32
    # arithmetic held only to 1.1e-5 of the largest dlogit here (now formed in fp64)
    "f32_sharp_gates": _shape("f32_sharp_gates", T=492, d=224, E=2, K=2, f=120, seed=342,
                              dtype="f32", cf=0.27, sub_seq=123, w_std=0.05, wr_std=0.5),
    # a single 16-token router block and sub-sequence
    "t16": _shape("t16", T=16, d=256, E=8, K=2, f=256, sub_seq=16, cf=1.0, seed=37, w_std=0.05),
    # two segments of about 1024 rows: four m-tiles each, one full group of the grouped
    # tile order per segment
    "two_long": _shape("two_long", T=1024, d=512, E=2, K=2, f=768, seed=30, w_std=0.05),
    # more than 640 rows per expert: the weight gradients take the one-tile-per-block kernel
    # (every shorter case here takes the persistent one); one expert, and three with a
    # ragged last k-step
    "onetile_e1": _shape("onetile_e1", T=768, d=256, E=1, K=1, f=512, sub_seq=768, seed=38,
                         w_std=0.05),
    "onetile_e3": _shape("onetile_e3", T=1000, d=512, E=3, K=2, f=256, sub_seq=1000, seed=39,
                         w_std=0.05),
    # f = 16384: the dgrads' pairs of k-steps at a 32 KB row pitch and a gate/up dgrad K of
    # 32768 (512 pairs), as in the Mixtral-8x22B shape
    "paired_dgrad": _shape("paired_dgrad", T=384, d=512, E=2, K=1, f=16384, sub_seq=384, seed=27,
                           w_std=0.02),
    # the permute backward's two forms at their boundary: E = 15 with a shared expert fills
    # all 16 LDS columns of the slice kernel (w_sg in the last), E = 16 takes the transposed
    # router weight; d = 640 leaves the last column slice partly empty
    "slice_e15": _shape("slice_e15", T=256, d=640, E=15, K=8, f=256, fs=256, seed=28, w_std=0.05),
    "rows_e16": _shape("rows_e16", T=256, d=640, E=16, K=8, f=256, fs=256, seed=29, w_std=0.05),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    s = CASES[name]
    lay, inp, cap = _run(s)
    tol = 1e-5 if s.dtype == "f32" else 2e-2
    check_layer(lay, inp, s.K, s.sub_seq, cap, tol)


def test_layer_parity_forced_valu():
    s = CASES["mfma_drop"]
    from token_dispatch_expert_router_amd import _lib as L
    lay, inp, cap = _run(s, flags=L.MOE_FLAG_VALU_GEMM)
    check_layer(lay, inp, s.K, s.sub_seq, cap, 2e-2)


def test_mfma_and_valu_agree():
    """The two GEMM paths compute the same function (to bf16 rounding)."""
    from token_dispatch_expert_router_amd import _lib as L
    s = CASES["mfma_drop"]
    a, _, _ = _run(s)
    b, _, _ = _run(s, flags=L.MOE_FLAG_VALU_GEMM)
    for k in ("y", "dx", "dw_gate", "dw_up", "dw_down"):
        assert_close(k, host(a.buf[k]), host(b.buf[k]), 1e-2)


def test_capacity_zero_drops_everything():
    s = _shape("cap0", T=128, d=256, E=4, K=2, f=256, sub_seq=128, cf=0.0, seed=16)
    lay, inp, cap = _run(s)
    assert cap == 0
    assert int(host(lay.rt["n_kept"])[0]) == 0
    assert np.all(host(lay.buf["y"]) == 0)
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert np.all(host(lay.buf[k]) == 0), k
    check_layer(lay, inp, s.K, s.sub_seq, cap, 2e-2)


def test_capacity_at_least_S_equals_dropless():
    s1 = _shape("capS", T=256, d=256, E=4, K=2, f=256, sub_seq=128, cf=2.0, seed=17)
    s2 = dataclasses.replace(s1, name="free", cf=None)
    a, _, cap = _run(s1)
    assert cap >= s1.sub_seq
    b, _, _ = _run(s2)
    for k in ("keep", "row_of", "offsets"):
        assert np.array_equal(host(a.rt[k]), host(b.rt[k])), k
    for k in ("y", "dx", "dw_gate"):
        assert np.array_equal(host(a.buf[k]), host(b.buf[k])), k


def test_expert_without_rows_gets_zero_grads():
    s = _shape("empty", T=256, d=256, E=4, K=2, f=256, seed=18)
    lay, inp, cap = _run(s, bias=[0.0, 0.0, 0.0, -80.0])
    counts = host(lay.rt["kept_counts"])
    assert counts[3] == 0
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert np.all(host(lay.buf[k])[3] == 0), k
    check_layer(lay, inp, s.K, s.sub_seq, cap, 2e-2)


def test_zero_tokens():
    from token_dispatch_expert_router_amd.layer import MoELayer
    lay = MoELayer(0, 256, 4, 2, 256, 1, -1, torch.bfloat16, device="cuda")
    inp = moe_synth.make_inputs(_shape("t0", d=256, f=256), device="cuda", T=0)
    lay.forward_backward(inp)
    torch.cuda.synchronize()
    assert int(host(lay.rt["n_kept"])[0]) == 0
    assert np.all(host(lay.rt["offsets"]) == 0)
    for k in ("dw_gate", "dw_up", "dw_down", "dw_router"):
        assert np.all(host(lay.buf[k]) == 0), k


def test_deterministic_repeat():
    s = CASES["mfma_drop"]
    from token_dispatch_expert_router_amd.layer import MoELayer
    inp = moe_synth.make_inputs(s, device="cuda")
    cap = oracle.capacity(s.sub_seq, s.K, s.E, s.cf)
    lay = MoELayer(s.T, s.d, s.E, s.K, s.f, s.sub_seq, cap, s.torch_dtype, device="cuda")
    lay.forward_backward(inp)
    first = {k: v.clone() for k, v in lay.buf.items() if isinstance(v, torch.Tensor)}
    lay.forward_backward(inp)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(v, lay.buf[k]), k


# --------------------------------------------------------------------------------
# Routing from given logits: bit-exact against the oracle
# --------------------------------------------------------------------------------

ROUTE_CASES = [  # T, E, K, S, cf, integer-valued logits (many exact ties)
    (256, 4, 2, 256, None, False), (4096, 8, 2, 4096, 1.0, False), (4096, 64, 8, 4096, 1.0, False),
    (2048, 64, 8, 512, 1.0, True), (1000, 16, 4, 250, 0.5, True), (512, 8, 1, 64, 1.0, False),
    (333, 5, 5, 111, 1.0, True), (8192, 8, 2, 1024, 1.25, False), (64, 64, 8, 64, 0.0, False),
    (640, 3, 2, 640, None, True), (4096, 64, 8, 4096, None, False),
    # sub-sequences at and past the 16384 / 32768 tokens the register-resident selects
    # handle (longer ones take the list-based kernel)
    (16384, 8, 2, 16384, 1.0, False), (20480, 8, 2, 20480, 1.0, False),
    (32768, 16, 4, 32768, 0.75, True), (40960, 8, 2, 40960, 1.0, False),
]


def _route_layer(T, E, K, S, cap):
    from token_dispatch_expert_router_amd.layer import MoELayer
    return MoELayer(T, 64, E, K, 64, S, cap, torch.float32, device="cuda")


@pytest.mark.parametrize("case", ROUTE_CASES)
def test_route_from_logits_bit_exact(case):
    T, E, K, S, cf, ints = case
    g = torch.Generator().manual_seed(T * 131 + E * 7 + K)
    if ints:
        lg = torch.randint(-3, 4, (T, E), generator=g).float()
    else:
        lg = torch.randn((T, E), generator=g) * 2.0
        lg[:, 0] += 1.0                              # skewed load: drops happen
    cap = oracle.capacity(S, K, E, cf)
    lay = _route_layer(T, E, K, S, cap)
    lay.route({}, logits=lg.cuda())
    torch.cuda.synchronize()
    ref = oracle.route(lg.numpy(), K, S, cap)
    log(f"  route T={T} E={E} K={K} S={S} cap={cap}: n_kept={ref['n_kept']}")
    assert_routing_equal(lay, ref)


@pytest.mark.parametrize("name", sorted(n for n in os.listdir(GOLDEN) if n.startswith("route_")))
def test_route_golden_on_gpu(name):
    gd = json.load(open(os.path.join(GOLDEN, name)))
    lay = _route_layer(gd["T"], gd["E"], gd["K"], gd["S"], gd["capacity"])
    lay.route({}, logits=torch.tensor(gd["logits"], dtype=torch.float32).cuda())
    torch.cuda.synchronize()
    for k in ("topk_idx", "keep", "row_of", "routed_counts", "kept_counts", "offsets"):
        assert np.array_equal(host(lay.rt[k]), np.asarray(gd[k])), k
    n = gd["n_kept"]
    assert np.array_equal(host(lay.rt["src_of"])[:n], np.asarray(gd["src_of"]))
    assert np.max(np.abs(host(lay.rt["topk_gate"]) - np.asarray(gd["topk_gate"]))) <= gd["gate_tol"]


def _random_shapes(n=24, seed=2024):
    """Seeded random small layers: bf16 with d, f multiples of 256 (matrix-core GEMMs; d of
    384 or 640 takes the matrix-core router with four waves per block and the vector-ALU
    GEMMs) or of 8 (vector-ALU router and GEMMs), and some fp32 layers; E up to 64 with K up
    to 8, dropless or cf in (0.25, 2], one to four sub-sequences, an optional shared
    expert (on every kind; the vector-ALU and fp32 layers draw theirs from a second
    generator, so the other draws keep their values) and, from that generator too, an
    optional skewed router bias."""
    rng = np.random.default_rng(seed)
    rng_fs = np.random.default_rng(seed + 1)
    out = []
    for i in range(n):
        kind = int(rng.integers(0, 5))  # 0-1 matrix cores, 2 four-wave router, 3 VALU, 4 fp32
        fs_other = int(8 * rng_fs.integers(4, 40)) if rng_fs.random() < 1 / 3 else 0
        zipf = bool(rng_fs.random() < 0.2)
        mfma = kind <= 1
        if mfma:
            d = int(rng.choice([256, 512]))
        elif kind == 2:
            d = int(rng.choice([384, 640]))
        else:
            d = int(8 * rng.integers(4, 40))
        f = int(rng.choice([256, 512, 768])) if mfma else int(8 * rng.integers(4, 40))
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 64]))
        K = int(rng.integers(1, min(E, 8) + 1))
        n_sub = int(rng.integers(1, 5))
        S = int(rng.integers(16, 160))
        cf = None if rng.random() < 0.3 else float(np.round(rng.uniform(0.25, 2.0), 2))
        fs = int(rng.choice([0, 0, 256])) if mfma else fs_other
        dtype = "f32" if kind == 4 else "bf16"
        out.append(_shape(f"rand{i}", T=n_sub * S, d=d, E=E, K=K, f=f, sub_seq=S, cf=cf, fs=fs,
                          seed=100 + i, w_std=0.05, wr_std=0.5, dtype=dtype, zipf_bias=zipf))
    return out


def _medium_shapes(n=8, seed=4242):
    """Seeded random medium layers: 256-1279-token sub-sequences, one or two of them, d up
    to 1024, f up to 1024, 1 to 16 experts, K up to 4, dropless or cf in [0.5, 1.5], an
    optional shared expert: segments of several row tiles, several n-tiles, and the
    one-tile weight-gradient kernel whenever an expert gets more than 640 rows."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([256, 512, 768, 1024]))
        f = int(rng.choice([256, 512, 1024]))
        E = int(rng.choice([1, 2, 4, 8, 16]))
        K = int(rng.integers(1, min(E, 4) + 1))
        n_sub = int(rng.integers(1, 3))
        S = int(rng.integers(256, 1280))
        cf = None if rng.random() < 0.4 else float(np.round(rng.uniform(0.5, 1.5), 2))
        fs = int(rng.choice([0, 0, 0, 512]))
        out.append(_shape(f"med{i}", T=n_sub * S, d=d, E=E, K=K, f=f, sub_seq=S, cf=cf, fs=fs,
                          seed=5000 + i, w_std=0.03, wr_std=0.5))
    return out


# MOE_PARITY_MEDIUM / MOE_PARITY_SEED widen this sweep (default 8 layers, seed 4242)
@pytest.mark.parametrize("shape", _medium_shapes(int(os.environ.get("MOE_PARITY_MEDIUM", "8")),
                                                 int(os.environ.get("MOE_PARITY_SEED", "4242"))),
                         ids=lambda s: s.name)
def test_medium_layer_parity(shape):
    lay, inp, cap = _run(shape)
    check_layer(lay, inp, shape.K, shape.sub_seq, cap, 2e-2)


# MOE_PARITY_RANDOM / MOE_PARITY_SEED widen the sweep (default 24 layers, seed 2024)
@pytest.mark.parametrize("shape", _random_shapes(int(os.environ.get("MOE_PARITY_RANDOM", "24")),
                                                 int(os.environ.get("MOE_PARITY_SEED", "2024"))),
                         ids=lambda s: s.name)
def test_random_layer_parity(shape):
    lay, inp, cap = _run(shape)
    check_layer(lay, inp, shape.K, shape.sub_seq, cap, 1e-5 if shape.dtype == "f32" else 2e-2)


def test_user_stream_matches_default_stream():
    """The calls take the caller's stream: a layer run on a separate stream gives the same
    bits as on the current stream."""
    from token_dispatch_expert_router_amd.layer import MoELayer
    s = CASES["k3_drop"]
    inp = moe_synth.make_inputs(s, device="cuda")
    cap = oracle.capacity(s.sub_seq, s.K, s.E, s.cf)
    a = MoELayer(s.T, s.d, s.E, s.K, s.f, s.sub_seq, cap, s.torch_dtype, device="cuda")
    b = MoELayer(s.T, s.d, s.E, s.K, s.f, s.sub_seq, cap, s.torch_dtype, device="cuda")
    a.forward_backward(inp)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    b.forward_backward(inp, stream=st)
    st.synchronize()
    for k in ("y", "dx", "dw_gate", "dw_up", "dw_down", "dw_router", "dlogits"):
        assert torch.equal(a.buf[k], b.buf[k]), k
    for k in ("topk_idx", "keep", "row_of", "offsets"):
        assert torch.equal(a.rt[k], b.rt[k]), k
