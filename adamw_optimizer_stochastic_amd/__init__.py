"""Fused AdamW with stochastic-rounding bf16 write-back for AMD MI355X (gfx950).

The computation lives in libadamw_sr.so (HIP kernels behind the C ABI of
include/adamw_sr.h); this package is its Python binding:
  * ``_abi``  ctypes binding, one function per C entry point (same names);
  * ``ops``   tensor-level wrappers (torch supplies device memory, streams):
    the AdamW step, the SR/RN conversions and ``to()``, the bf16 GEMM with
    an SR epilogue;
  * ``random`` uniform/normal draws and dropout on the same stream;
  * ``AdamWSR`` the optimizer (a torch.optim.AdamW drop-in);
  * ``workloads`` seeded synthetic inputs for tests and the benchmark.
The library is loaded on first use; if it is missing, calls raise.
"""

from .optim import AdamWSR  # noqa: F401
from . import ops  # noqa: F401
from .ops import (  # noqa: F401
    adamw_step, philox_4x32_fill, cvt_f32_bf16_sr, cvt_f32_bf16_rn, gemm_bf16, AsrError,
    RoundingMode, to,
)
from . import random  # noqa: F401,E402

__all__ = ["AdamWSR", "ops", "adamw_step", "philox_4x32_fill", "cvt_f32_bf16_sr",
           "cvt_f32_bf16_rn", "gemm_bf16", "AsrError", "RoundingMode", "to", "random"]
