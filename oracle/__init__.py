"""CPU oracle for the fused AdamW step with stochastic-rounding bf16 write-back.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain reference that the
GPU library is checked against. Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path (the C-ABI
library and its Python binding) never does, and this package imports nothing
from the product path.

Sources (the pages are cited by title and section):
  * "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request),
    Primitives and Tests sections: the add-and-truncate rounding rule and the
    counter-based Philox generator.
  * The same FlyDSL page, Consumer and Tests sections: a bf16 GEMM whose f32
    accumulator is rounded to bf16 by RN or by SR keyed per output element
    (oracle/gemm.py).
  * The same FlyDSL page, discussion section: the generator as a general
    random-number facility (dropout, initialisation) -- oracle/rng.py.
  * "adamw-sr" (kernels hub page), intro, Usage, Method, Correctness sections:
    the decoupled-weight-decay AdamW step, fp32 states, bf16 write-back by
    stochastic rounding, random bits tied to the key (seed, step) and to
    each element's position in the whole parameter set.
  * Published definitions the pages name but do not print: Philox4x32 with 10
    rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
    1, 2, 3", SC 2011) and the AdamW update as documented for
    torch.optim.AdamW (Loshchilov and Hutter, "Decoupled Weight Decay
    Regularization", 2019, in the torch form).

Every function exists in two forms where it matters:
  * ``*_scalar``: pure-Python integers / Python floats rounded to binary32,
    for tiny inputs;
  * vectorized numpy (uint32/uint64 integer ops, float32 ufuncs).
The two are written independently and checked against each other and against
the pins in ``tests/test_oracle_*.py``.

Parity status: every function here is pinned (see the tests); none is
"parity unpinned".
"""

from .philox import (  # noqa: F401
    MUL_A, MUL_B, WEYL_A, WEYL_B, ROUNDS,
    philox4x32_10, philox4x32_10_scalar,
)
from .bf16 import (  # noqa: F401
    sr_bf16, sr_bf16_scalar, rn_bf16, rn_bf16_scalar,
    bf16_to_f32, f32_bits, bits_f32,
)
from .stream import random16, random16_scalar  # noqa: F401
from .adamw import (  # noqa: F401
    HostScalars, host_scalars, adamw_f32, adamw_f32_scalar,
    step_tensor, step_tensor_scalar, step_list,
    ROUND_SR, ROUND_RN, F32, BF16,
)
from .stream import philox_fill  # noqa: F401,E402
from .convert import cvt_f32_bf16_sr, cvt_f32_bf16_rn  # noqa: F401,E402
from .gemm import (  # noqa: F401,E402
    gemm_exact, gemm_exact_scalar, gemm_dot, abs_products, f32_sum_bound,
    gemm_round, gemm_round_at,
)
from . import rng  # noqa: F401,E402
