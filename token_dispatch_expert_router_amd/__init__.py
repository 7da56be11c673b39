"""One MI355X's MoE layer (router top-K, capacity drop, permute, grouped SwiGLU
experts, gate-weighted un-permute; forward and backward) as hand-written HIP kernels
for gfx950 behind the C ABI of include/moe.h.  `_lib` binds that ABI; `layer` runs
the whole layer on one stream."""
from . import _lib  # noqa: F401
from ._lib import MoeError, load  # noqa: F401

__all__ = ["_lib", "MoeError", "load"]
