"""Decode-time int4 grouped MoE expert path for AMD Instinct MI355X (gfx950).

The compute lives in libi4moe.so (HIP kernels behind the C ABI of include/i4moe.h);
``binding`` exposes that ABI under the same names and ``runtime.Context`` wraps it.
"""

from . import binding  # noqa: F401
from .runtime import Context, I4moeError, host_rows  # noqa: F401
