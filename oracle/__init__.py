"""Oracle for the contiguous grouped block-scaled MoE GEMM with fused epilogue.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  It is a plain, slow, float64 CPU
evaluation of the equations on the cuDNN frontend pages "Grouped GEMM + Quant
(SM100)", "Grouped GEMM + SwiGLU (SM100)", "Grouped GEMM + sReLU (SM100)" and
"Grouped GEMM + dGLU (SM100)", and it shares no code with the HIP library
(``moe_grouped_block_amd``): no kernels, headers, tables, constants or
pre/post-processing.  Neither side imports the other.

The package holds two independent writings of the same definitions: the
numpy modules here (``formats``, ``grouped``) and a plain C++ implementation
in ``oracle/cpp`` (float64 loops, OpenMP over rows; ``cxx`` is its ctypes
binding, built by ``cxx.build()``).  Neither calls the other; the GPU parity
tests compare against the numpy one, the CPU baseline of the benchmark times
the C++ one, and a CPU test checks that the two agree on every seeded recipe.

Pins (tests that tie this code to something other than itself) live in
``tests/test_oracle_*.py`` and run on both implementations; every function
here is pinned, none is "parity unpinned", except the order of the SwiGLU
blocks relative to the GLU+Hadamard page (a reading, see ``grouped_gemm``'s
docstring).
"""
from . import formats  # noqa: F401
from .grouped import grouped_gemm, dequantize, group_of_rows  # noqa: F401
