"""Host check of the grouped GEMM's tile maps (no GPU).

The functions that pick a block's output tile (csrc/tile_map.h: the three row maps, the
grouped m/n order and the weight-gradient split) are compiled for the CPU into
tests/native/tile_map_check, which walks every block of each of the six launches (the
row passes with and without half-height tiles, under each row map) and asserts that
every output tile is produced exactly once, inside its segment, with each XCD on one
contiguous range of tiles (contiguous row map), on whole chunks dealt round-robin
(chunked row map) or on an equal, contiguous share of every expert (shared row map,
weight gradients); for the weight gradients it also walks the persistent launch (256, 64
or 8 blocks, each stepping through the one-tile launch's blocks of its XCD until the
first without a tile) and asserts the same exact-once coverage.  Offsets: each bf16
layer shape routed by the oracle on router inputs drawn on the CPU (the same recipe and
sizes as on the GPU; the CPU generator's values differ from the GPU's, so the segments
are of the same distribution, not identical; the GPU test runs the same check on the
device's own offsets), plus edge cases: empty experts, one expert holding every row,
segments of exactly 256 rows and of one row, fewer kept rows than the buffer holds.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import moe_synth
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    from token_dispatch_expert_router_amd import build
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not available")
    return build.build_tile_map_check(str(tmp_path_factory.mktemp("tm") / "tile_map_check"))


def _run(exe, offsets, R, d, f):
    offs = [int(v) for v in offsets]
    r = subprocess.run([exe, str(len(offs) - 1), str(R), str(d), str(f)] + [str(v) for v in offs],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 26 and all(ln.endswith(" ok") for ln in lines), r.stdout
    return lines


def _max_rows(T, K, E, S, cap):
    return T * K if cap < 0 else min(T * K, (T // S) * E * cap)


@pytest.mark.parametrize("name", [s.name for s in moe_synth.SHAPES if s.dtype == "bf16"])
def test_tile_maps_on_routed_shapes(checker, name):
    s = moe_synth.shape_by_name(name)
    inp = moe_synth.make_router_inputs(s, device="cpu")
    x = inp["x"].float().numpy()
    bias = None if inp["bias"] is None else inp["bias"].numpy()
    logits = oracle.router_logits(x, inp["w_router"].float().numpy(), bias)
    cap = oracle.capacity(s.sub_seq, s.K, s.E, s.cf)
    r = oracle.route(logits, s.K, s.sub_seq, cap)
    R = _max_rows(s.T, s.K, s.E, s.sub_seq, cap)
    lines = _run(checker, r["offsets"], R, s.d, s.f)
    print(name, r["kept_counts"].min(), r["kept_counts"].max(), lines)


EDGE = [
    # (name, segment sizes, R, d, f)
    ("empty experts", [0, 300, 0, 0, 513, 0, 256, 0], 2048, 512, 768),
    ("one expert holds every row", [0] * 7 + [4096], 4096, 256, 512),
    ("segments of exactly 256", [256] * 8, 2048, 256, 256),
    ("one-row segments", [1] * 64, 64, 256, 256),
    ("kept rows fewer than the buffer", [100, 7, 900, 3], 8192, 1024, 2048),
    ("64 skewed experts", [512] * 17 + [int(512 * 0.9 ** i) for i in range(47)], 32768, 6144, 2048),
    ("no rows at all", [0] * 8, 16, 256, 256),
    ("more than four m-tiles in a segment", [8132, 8120], 16384, 6144, 8192),
]


@pytest.mark.parametrize("name,sizes,R,d,f", EDGE, ids=[c[0] for c in EDGE])
def test_tile_maps_edge_cases(checker, name, sizes, R, d, f):
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    assert offsets[-1] <= R
    _run(checker, offsets, R, d, f)


def test_checker_rejects_bad_offsets(checker):
    """The checker itself fails on offsets that are not a valid segmentation."""
    r = subprocess.run([checker, "2", "100", "256", "256", "0", "60", "40"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "decrease" in r.stdout
    r = subprocess.run([checker, "2", "100", "256", "256", "0", "60", "140"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "offsets[E] > R" in r.stdout
