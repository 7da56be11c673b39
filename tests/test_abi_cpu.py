"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/moe.h declares, and rejects bad arguments before any HIP call (so these run
without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from token_dispatch_expert_router_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    _lib.load()
    return _lib


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 14
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTS) == names


def test_abi_version_and_capacity(L):
    assert L.moe_abi_version() == 1
    assert L.moe_capacity(4096, 2, 8, 1.0) == 1024
    assert L.moe_capacity(4096, 8, 64, 1.0) == 512
    assert L.moe_capacity(10, 1, 3, 1.0) == 4
    assert L.moe_capacity(8, 2, 4, 0.0) == 0
    assert L.moe_capacity(8, 2, 4, -1.0) == -1


def test_capacity_agrees_with_oracle(L):
    import oracle
    for S, K, E, cf in ((4096, 2, 8, 1.0), (4096, 8, 64, 1.0), (100, 3, 7, 1.25),
                        (33, 2, 5, 0.5), (8, 1, 3, 2.0)):
        assert L.moe_capacity(S, K, E, cf) == oracle.capacity(S, K, E, cf)


def test_max_rows_and_workspace(L):
    d = L.make_desc(4096, 6144, 8, 2, 16384, 4096, 1024, L.MOE_BF16)
    assert L.moe_max_rows(d) == 8192
    d = L.make_desc(4096, 6144, 64, 8, 2048, 4096, 512, L.MOE_BF16)
    assert L.moe_max_rows(d) == 32768
    d = L.make_desc(4096, 6144, 64, 8, 2048, 1024, 10, L.MOE_BF16)
    assert L.moe_max_rows(d) == 4 * 64 * 10
    d = L.make_desc(256, 64, 4, 2, 128, 256, -1, L.MOE_F32)
    assert L.moe_max_rows(d) == 512
    for w in range(5):
        assert L.moe_workspace_size(d, w) >= 0
    assert L.moe_workspace_size(d, L.MOE_WS_FFN_BWD) >= 2 * 512 * 128 * 4


@pytest.mark.parametrize("E,dtype,esz", [(1, "MOE_F32", 4), (8, "MOE_BF16", 2), (15, "MOE_BF16", 2),
                                         (16, "MOE_BF16", 2), (64, "MOE_BF16", 2), (64, "MOE_F32", 4)])
def test_permute_bwd_workspace(L, E, dtype, esz):
    # up to 15 experts a block keeps its slice of the router weight in LDS (no workspace);
    # from 16 on the library writes a transposed copy, (E + 1) * d elements
    d = L.make_desc(512, 6144, E, 1, 2048, 512, -1, getattr(L, dtype))
    n = L.moe_workspace_size(d, L.MOE_WS_PERMUTE_BWD)
    if E + 1 <= 16:
        assert n == 0
    else:
        assert n >= (E + 1) * 6144 * esz and n % 256 == 0


@pytest.mark.parametrize("field,value,status", [
    ("K", 9, -1), ("K", 0, -1), ("E", 65, -2), ("E", 0, -2), ("d", 12, -2), ("f", 0, -1),
    ("sub_seq", 100, -1), ("capacity", -2, -1), ("dtype", 7, -2), ("T", -1, -1),
    ("flags", 4, -1),
])
def test_invalid_desc_rejected(L, field, value, status):
    d = L.make_desc(256, 64, 4, 2, 128, 256, -1, L.MOE_F32)
    setattr(d, field, value)
    lib = L.load()
    assert lib.moe_max_rows(ctypes.byref(d)) == -1
    r = L.Routing()
    st = lib.moe_route_from_logits(ctypes.byref(d), None, ctypes.byref(r), None, 0, None)
    assert st == status, (field, st, L.moe_last_error())
    assert L.moe_last_error()


def test_null_pointers_and_workspace(L):
    lib = L.load()
    d = L.make_desc(256, 64, 4, 2, 128, 256, -1, L.MOE_F32)
    r = L.Routing()
    assert lib.moe_permute(ctypes.byref(d), None, ctypes.byref(r), None, None) == -1
    assert "routing" in L.moe_last_error()
    # a routing bundle with fake non-null pointers passes the routing check and then
    # fails on the workspace size, still before any launch
    fake = L.Routing(*[ctypes.c_void_p(4096 * (i + 1)) for i in range(10)])
    st = lib.moe_route_from_logits(ctypes.byref(d), ctypes.c_void_p(4096), ctypes.byref(fake),
                                   ctypes.c_void_p(4096), 1, None)
    assert st == -3 and "workspace" in L.moe_last_error()
    assert lib.moe_expert_ffn_fwd(ctypes.byref(d), *([None] * 10), 0, None) == -1
    assert lib.moe_route_bwd(ctypes.byref(fake and d), None, ctypes.byref(fake), None, None,
                             None, None, None, None, 0, None) == -1
    assert lib.moe_unpermute(ctypes.byref(d), ctypes.c_void_p(4096), ctypes.byref(fake),
                             ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), None) == -1
    assert "sg_logit" in L.moe_last_error()


def test_partial_flag_accepted_by_ffn_rejected_by_row_calls(L):
    """MOE_FLAG_F32_PARTIAL is a valid descriptor flag (the two FFN calls take it), and
    the row-movement calls that read o or dxp refuse it before any launch."""
    lib = L.load()
    d = L.make_desc(256, 64, 4, 1, 128, 256, -1, L.MOE_BF16, L.MOE_FLAG_F32_PARTIAL)
    assert lib.moe_max_rows(ctypes.byref(d)) == 256
    assert L.moe_workspace_size(d, L.MOE_WS_FFN_BWD) > 0
    fake = L.Routing(*[ctypes.c_void_p(4096 * (i + 1)) for i in range(10)])
    p = ctypes.c_void_p(4096)
    assert lib.moe_unpermute(ctypes.byref(d), p, ctypes.byref(fake), None, None, p, None) == -1
    assert "MOE_FLAG_F32_PARTIAL" in L.moe_last_error()
    assert lib.moe_unpermute_bwd(ctypes.byref(d), p, p, ctypes.byref(fake), None, None, p, p,
                                 None, None, None) == -1
    assert "MOE_FLAG_F32_PARTIAL" in L.moe_last_error()
    assert lib.moe_permute_bwd(ctypes.byref(d), p, ctypes.byref(fake), None, None, None, None,
                               None, p, None, 0, None) == -1
    assert "MOE_FLAG_F32_PARTIAL" in L.moe_last_error()


def test_binding_raises_library_error(L):
    """The Python binding turns a failed status into MoeError carrying the library's
    message, before any launch (a null stream handle is never touched)."""
    import types
    s0 = types.SimpleNamespace(cuda_stream=0)
    bad = L.make_desc(256, 64, 4, 9, 128, 256, -1, L.MOE_F32)
    with pytest.raises(L.MoeError) as ei:
        L.moe_permute(bad, None, L.Routing(), None, stream=s0)
    assert ei.value.status == -1 and "K = 9" in str(ei.value)
    uneven = L.make_desc(100, 64, 4, 2, 128, 48, -1, L.MOE_F32)
    with pytest.raises(L.MoeError) as ei:
        L.moe_route_from_logits(uneven, None, L.Routing(), None, stream=s0)
    assert "multiple" in str(ei.value)


def test_noalloc_route_rejects_oversize_before_any_launch(L):
    """moe_route_noalloc works inside a fixed scratch of MOE_ROUTE_SCRATCH_BYTES: a shape
    whose route workspace is larger is refused with MOE_ERR_UNSUPPORTED (no HIP call is
    made, so this runs without a GPU); the Mixtral- and G8T8-shaped layers fit."""
    lib = L.load()
    fake = L.Routing(*[ctypes.c_void_p(4096 * (i + 1)) for i in range(10)])
    p = ctypes.c_void_p(4096)
    big = L.make_desc(65536, 6144, 64, 8, 2048, 65536, 4096, L.MOE_BF16)
    assert L.moe_workspace_size(big, L.MOE_WS_ROUTE) > L.MOE_ROUTE_SCRATCH_BYTES
    st = lib.moe_route_noalloc(ctypes.byref(big), p, p, None, None, p, None, ctypes.byref(fake),
                               None)
    assert st == -2 and "scratch" in L.moe_last_error()
    for shape in ((4096, 6144, 8, 2, 16384, 4096, 1024), (4096, 6144, 64, 8, 2048, 4096, 512),
                  (8192, 8192, 8, 2, 28672, 8192, -1), (16384, 6144, 8, 2, 16384, 16384, 4096)):
        d = L.make_desc(*shape, L.MOE_BF16)
        assert L.moe_workspace_size(d, L.MOE_WS_ROUTE) <= L.MOE_ROUTE_SCRATCH_BYTES
    # argument errors come first, as for moe_route
    assert lib.moe_route_noalloc(ctypes.byref(big), None, p, None, None, p, None,
                                 ctypes.byref(fake), None) == -1
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert "#define MOE_ROUTE_SCRATCH_BYTES (16u << 20)" in src
    assert L.MOE_ROUTE_SCRATCH_BYTES == 16 << 20
