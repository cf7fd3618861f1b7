"""Random numbers on the library's position-keyed Philox stream.

"Add stochastic rounding and philox RNG helpers" (FlyDSL pull request),
discussion: the counter-based generator belongs in a random-number namespace
of its own, serving dropout and initialisation as well as rounding. Every
function here draws from the stream the optimizer's rounding uses: element
i of a tensor is global position base_index + i under key (seed, step), so
a tensor split into pieces that pass their own base_index reproduces the
whole, and a fixed key reproduces the same values on every run.

All work runs in the library's kernels (C entry points asr_random_uniform,
asr_random_normal, asr_dropout, asr_philox_4x32_fill); torch only supplies
memory and the stream. bf16 outputs are the round-to-nearest-even of the
binary32 value.
"""

import torch

from . import _abi, ops
from .ops import _require_gpu, _stream, _DTYPE_CODE, _u32 as _u32_named, _u64 as _u64_named

__all__ = ["philox_4x32", "uniform", "normal", "uniform_", "normal_", "dropout"]


def _u64(x):
    return _u64_named("base_index", x)


def _u32(name, x):
    return _u32_named(name, x)


def _code(t):
    code = _DTYPE_CODE.get(t.dtype)
    if code is None:
        raise TypeError(f"float32 or bfloat16 tensors only (got {t.dtype})")
    return code


def philox_4x32(n_counters, counter_base=0, *, seed, step=0, counter_upper=0, device="cuda"):
    """Raw words of Philox4x32-10 calls counter_base .. + n_counters - 1
    under key (seed, step): an int32 tensor of 4 * n_counters (reinterpret
    as uint32); call j's words at 4j .. 4j + 3."""
    return ops.philox_4x32_fill(n_counters, counter_base, _u32("seed", seed), _u32("step", step),
                                counter_upper, device=device)


def uniform_(tensor, low=0.0, high=1.0, *, seed, step=0, base_index=0):
    """Fill `tensor` in place with draws in [low, high): element i is
    low + (high - low) * U(base_index + i), U = (W >> 8) * 2**-24."""
    _require_gpu(tensor, "tensor")
    code = _code(tensor)
    with torch.cuda.device(tensor.device):
        _abi.asr_random_uniform(tensor.data_ptr(), code, tensor.numel(), float(low), float(high),
                                _u32("seed", seed), _u32("step", step), _u64(base_index),
                                _stream(tensor.device))
    return tensor


def normal_(tensor, mean=0.0, std=1.0, *, seed, step=0, base_index=0):
    """Fill `tensor` in place with normal draws (Box-Muller on position
    pairs): element i is mean + std * z(base_index + i)."""
    _require_gpu(tensor, "tensor")
    code = _code(tensor)
    with torch.cuda.device(tensor.device):
        _abi.asr_random_normal(tensor.data_ptr(), code, tensor.numel(), float(mean), float(std),
                               _u32("seed", seed), _u32("step", step), _u64(base_index),
                               _stream(tensor.device))
    return tensor


def uniform(shape, low=0.0, high=1.0, *, seed, step=0, base_index=0, dtype=torch.float32,
            device="cuda"):
    return uniform_(torch.empty(shape, dtype=dtype, device=device), low, high, seed=seed,
                    step=step, base_index=base_index)


def normal(shape, mean=0.0, std=1.0, *, seed, step=0, base_index=0, dtype=torch.float32,
           device="cuda"):
    return normal_(torch.empty(shape, dtype=dtype, device=device), mean, std, seed=seed,
                   step=step, base_index=base_index)


def dropout(x, p=0.5, *, seed, step=0, base_index=0, training=True, inplace=False,
            return_mask=False):
    """Inverted dropout: element i is dropped when its stream word is below
    floor(p * 2**32) and kept elements are scaled by 1 / (1 - p) (one binary32
    multiply). Returns y, or (y, mask) with mask a bool tensor of kept
    elements. training=False returns x unchanged (and an all-True mask)."""
    _require_gpu(x, "x")
    code = _code(x)
    if not (0.0 <= p < 1.0):
        raise ValueError("p must be in [0, 1)")
    if not training:
        return (x, torch.ones(x.shape, dtype=torch.bool, device=x.device)) if return_mask else x
    y = x if inplace else torch.empty_like(x)
    mask = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if return_mask else None
    with torch.cuda.device(x.device):
        _abi.asr_dropout(x.data_ptr(), y.data_ptr(), mask.data_ptr() if mask is not None else None,
                         code, x.numel(), float(p), _u32("seed", seed), _u32("step", step),
                         _u64(base_index), _stream(x.device))
    return (y, mask.view(torch.bool)) if return_mask else y
