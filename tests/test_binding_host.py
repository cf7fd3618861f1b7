"""Argument checks of the Python binding that run before any GPU work.

The C entry points take 32-bit seeds and steps and 64-bit stream
positions; ctypes would wrap an out-of-range Python int without a word, so
the binding rejects it instead."""

import numpy as np
import pytest
import torch

from adamw_optimizer_stochastic_amd import _abi, ops, random as arng


def test_integer_ranges():
    assert ops._u32("seed", 0) == 0
    assert ops._u32("seed", (1 << 32) - 1) == (1 << 32) - 1
    assert ops._u32("seed", np.uint32(7)) == 7
    assert ops._u64("base_index", (1 << 64) - 1) == (1 << 64) - 1
    assert ops._u64("base_index", np.int64(1 << 40)) == 1 << 40
    for bad in (-1, 1 << 32):
        with pytest.raises(ValueError, match="seed"):
            ops._u32("seed", bad)
    for bad in (-1, 1 << 64):
        with pytest.raises(ValueError, match="base_index"):
            ops._u64("base_index", bad)
    with pytest.raises(TypeError):
        ops._u32("seed", 1.0)


def test_adamw_step_key_checked_before_launch():
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    ops.adamw_step([], [], [], [], [], step=1, seed=0, **kw)  # nothing to do
    with pytest.raises(ValueError, match="seed"):
        ops.adamw_step([], [], [], [], [], step=1, seed=1 << 32, **kw)
    for step in (0, 1 << 32):
        with pytest.raises(ValueError, match="step"):
            ops.adamw_step([], [], [], [], [], step=step, seed=0, **kw)


def test_stream_arguments_checked_before_launch():
    x = torch.zeros(8)
    with pytest.raises(ValueError, match="seed"):
        ops.cvt_f32_bf16_sr(x, -1, 0)
    with pytest.raises(ValueError, match="step"):
        ops.cvt_f32_bf16_sr(x, 0, 1 << 32)
    with pytest.raises(ValueError, match="base_index"):
        ops.cvt_f32_bf16_sr(x, 0, 0, base_index=-5)
    with pytest.raises(ValueError, match="counter_base"):
        ops.philox_4x32_fill(4, -1, 0, 0)
    ab = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="seed"):
        ops.gemm_bf16(ab, ab, rounding="sr", seed=1 << 32)
    with pytest.raises(ValueError, match="base_index"):
        ops.gemm_bf16(ab, ab, rounding="sr", base_index=-1)
    with pytest.raises(ValueError, match="base_index"):
        arng._u64(1 << 64)   # the random module's position argument


def test_descriptor_dtype_matches_the_c_struct():
    """The numpy form of asr_tensor that the step's binding fills has the C
    struct's size and field offsets."""
    import ctypes
    dt = _abi.ASR_TENSOR_DTYPE
    assert dt.itemsize == ctypes.sizeof(_abi.AsrTensor) == 56
    for name, _ in _abi.AsrTensor._fields_:
        assert dt.fields[name][1] == getattr(_abi.AsrTensor, name).offset


def test_vectorized_overlap_check_agrees_with_the_plain_one():
    """The step's array form of the overlap check refuses exactly the span
    sets that check_disjoint refuses (random spans, some empty, some
    touching, some nested or identical)."""
    import numpy as np
    rng = np.random.default_rng(5)
    for trial in range(400):
        k = int(rng.integers(1, 12))
        starts = rng.integers(0, 200, k).astype(np.uint64) * 8
        sizes = (rng.integers(0, 6, k) * 8).astype(np.uint64)
        spans = [(int(a), int(n), f"s{i}") for i, (a, n) in enumerate(zip(starts, sizes))]
        try:
            ops.check_disjoint(spans)
            plain = None
        except ValueError as e:
            plain = str(e)
        try:
            ops._check_disjoint_arrays(starts, sizes, lambda i: f"s{i}")
            arr = None
        except ValueError as e:
            arr = str(e)
        assert (plain is None) == (arr is None), (spans, plain, arr)


def test_descriptor_address_checks_the_array():
    """Only a C-contiguous array of the descriptor dtype is passed by address."""
    import numpy as np
    assert _abi.array_address(np.zeros(0, dtype=_abi.ASR_TENSOR_DTYPE)) is None
    a = np.zeros(3, dtype=_abi.ASR_TENSOR_DTYPE)
    assert _abi.array_address(a) == a.ctypes.data
    with pytest.raises(TypeError):
        _abi.array_address(np.zeros(3, dtype=np.uint64))
    with pytest.raises(TypeError):
        _abi.array_address(a[::2])
