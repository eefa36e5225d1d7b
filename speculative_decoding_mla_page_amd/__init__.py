"""Tree-masked MLA verify attention for MI355X (gfx950).

The compute lives in libmla_verify.so (HIP kernels behind a C ABI, declared in
include/mla_verify.h); `binding` is its ctypes mirror and `device` holds the
torch-side helpers that move inputs to the GPU and call it.
"""
from . import binding  # noqa: F401
