"""A whole forward + backward step captured in a HIP graph.

The ABI calls allocate nothing, copy nothing between host and device and never
synchronise, and every size they launch with is fixed by the descriptor, so one layer
step can be captured once and replayed.  The kernels are deterministic, so every replay
must reproduce the eager step bit for bit.  Between replays the outputs are overwritten
with a sentinel and other eager GPU work runs, so a replay that skipped or reused
anything would show."""
import dataclasses

import pytest
import torch

import moe_synth
import oracle
from gpu_util import log

pytestmark = pytest.mark.gpu

# rows of these buffers past n_kept are never written by a step
ROW_BUFFERS = ("xp", "a", "b", "h", "o", "d_o", "dxp")

BASE = moe_synth.shape_by_name("tiny")
SHAPES = {
    "tiny_fp32": BASE,
    # matrix-core GEMMs, two sub-sequences with capacity drops
    "bf16_drop": dataclasses.replace(BASE, name="bf16_drop", T=1024, d=512, E=4, K=2, f=768,
                                     seed=31, dtype="bf16", cf=1.0, sub_seq=512, w_std=0.05,
                                     wr_std=0.3),
    # 64 experts and a sigmoid-gated shared expert (its own FFN launches)
    "bf16_shared_e64": dataclasses.replace(BASE, name="bf16_shared_e64", T=256, d=256, E=64,
                                           K=8, f=256, fs=256, seed=32, dtype="bf16", cf=None,
                                           sub_seq=256, w_std=0.05, wr_std=0.3),
}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_dispatch_expert_router_amd import _lib as L
    L.load()
    return L


def _outputs(lay):
    """Every tensor a step writes (row buffers cut at n_kept), by name."""
    n = int(lay.rt["n_kept"].item())
    out = {}
    for k, v in lay.rt.items():
        out["rt." + k] = v[:n] if k == "src_of" else v
    for k, v in lay.buf.items():
        if v is None or k == "shared_offsets":
            continue
        out[k] = v[:n] if k in ROW_BUFFERS else v
    return out


def _clobber(lay):
    for k, v in list(lay.rt.items()) + list(lay.buf.items()):
        if v is None or k == "shared_offsets":
            continue
        v.fill_(0x5A if v.dtype == torch.uint8 else -7)


@pytest.mark.parametrize("name", list(SHAPES))
def test_graph_replay_matches_eager(name):
    from token_dispatch_expert_router_amd.layer import MoELayer
    s = SHAPES[name]
    log(f"  graph case {name}: T={s.T} d={s.d} E={s.E} K={s.K} f={s.f} fs={s.fs} {s.dtype}")
    inp = moe_synth.make_inputs(s, device="cuda")
    cap = oracle.capacity(s.sub_seq, s.K, s.E, s.cf) if s.cf is not None else -1
    lay = MoELayer(s.T, s.d, s.E, s.K, s.f, s.sub_seq, cap, s.torch_dtype, fs=s.fs,
                   device="cuda")

    lay.forward_backward(inp)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in _outputs(lay).items()}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lay.forward_backward(inp)
    torch.cuda.synchronize()

    other = torch.randn((512, 512), device="cuda")
    for i in range(3):
        _clobber(lay)
        other = torch.tanh(other @ other.T * 1e-3)   # unrelated eager work
        if i == 1:                                    # eager library calls in between
            lay.forward_backward(inp)
            _clobber(lay)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(lay)
        assert set(got) == set(eager)
        for k, v in eager.items():
            assert torch.equal(got[k], v), f"replay {i}: {k} differs from the eager step"
    del graph
