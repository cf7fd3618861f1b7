"""Tensor-level entry points over the C ABI (torch supplies memory and streams).

Each function checks devices, dtypes, sizes and contiguity, then calls the
C entry point of the same name (without the ``asr_`` prefix) on the current
HIP stream of the tensors' device. All arithmetic runs in the library's
kernels; there is no CPU path.
"""

import operator

import numpy as np
import torch

from . import _abi
from ._abi import ASR_F32, ASR_BF16, ASR_ROUND_SR, ASR_ROUND_RN, AsrError  # noqa: F401

_DTYPE_CODE = {torch.float32: ASR_F32, torch.bfloat16: ASR_BF16}
ROUNDING_CODE = {"sr": ASR_ROUND_SR, "rn": ASR_ROUND_RN}


def _require_gpu(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _uint(name, x, bits):
    """x as a Python int in [0, 2**bits) (the C argument's range), else
    ValueError: ctypes would otherwise wrap it silently."""
    try:
        v = operator.index(x)
    except TypeError:
        raise TypeError(f"{name} must be an integer (got {type(x).__name__})") from None
    if not 0 <= v < (1 << bits):
        raise ValueError(f"{name} must be in [0, 2**{bits})")
    return v


def _u32(name, x):
    return _uint(name, x, 32)


def _u64(name, x):
    return _uint(name, x, 64)


def check_disjoint(spans):
    """Raise ValueError if any two of the byte ranges overlap. spans: an
    iterable of (start, nbytes, name); empty ranges are ignored."""
    live = sorted((int(a), int(a) + int(n), name) for a, n, name in spans if int(n) > 0)
    for (a0, e0, n0), (a1, _, n1) in zip(live, live[1:]):
        if a1 < e0:
            raise ValueError(f"{n0} and {n1} share memory; every buffer of the step "
                             "must be disjoint from the others")


def _extent(t, name):
    """(start, nbytes, name) of the memory a strided tensor spans."""
    if t.numel() == 0:
        return (t.data_ptr(), 0, name)
    last = sum((size - 1) * stride for size, stride in zip(t.shape, t.stride()))
    return (t.data_ptr(), (last + 1) * t.element_size(), name)


def workspace_bytes(numels):
    """Workspace bytes for a list of tensors with these element counts."""
    return _abi.asr_adamw_workspace_bytes([dict(numel=int(n)) for n in numels])


def make_workspace(numels, device):
    """A device buffer big enough for a list of tensors with these numels."""
    return torch.empty(max(workspace_bytes(numels), 1), dtype=torch.uint8, device=device)


_STEP_NAMES = ("param", "grad", "exp_avg", "exp_avg_sq")
_SMALL_LIST = 8   # lists up to this long take the plain overlap check (less fixed cost)
_ELEM_BYTES = {torch.float32: 4, torch.bfloat16: 2}


def _step_descriptors(params, grads, exp_avgs, exp_avg_sqs, base_indices, device):
    """Checks the four lists and returns their asr_tensor array (numpy), its
    address and the workspace bytes the step needs. Raises TypeError /
    ValueError."""
    n = len(params)
    lists = (params, grads, exp_avgs, exp_avg_sqs)
    index = device.index
    for ts, name in zip(lists, _STEP_NAMES):
        for i, t in enumerate(ts):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name}[{i}] must be a torch.Tensor")
            if not t.is_cuda:
                raise ValueError(f"{name}[{i}] must be on a GPU (got {t.device})")
            if t.get_device() != index:
                raise ValueError("all tensors must be on one device")
            if not t.is_contiguous():
                raise ValueError(f"{name}[{i}] must be contiguous")
    pdt, gdt = [p.dtype for p in params], [g.dtype for g in grads]
    for i, (a, b) in enumerate(zip(pdt, gdt)):
        if a not in _DTYPE_CODE or b not in _DTYPE_CODE:
            raise TypeError(f"tensor {i}: params and grads must be float32 or bfloat16")
    for ts in (exp_avgs, exp_avg_sqs):
        for i, t in enumerate(ts):
            if t.dtype != torch.float32:
                raise TypeError(f"tensor {i}: optimizer states must be float32")
    numels = [p.numel() for p in params]
    for ts in lists[1:]:
        for i, (t, k) in enumerate(zip(ts, numels)):
            if t.numel() != k:
                raise ValueError(f"tensor {i}: param, grad and states differ in size")
    arr = np.zeros(n, dtype=_abi.ASR_TENSOR_DTYPE)
    ptrs = [[t.data_ptr() for t in ts] for ts in lists]
    for name, col in zip(_STEP_NAMES, ptrs):
        arr[name] = col
    arr["numel"] = numels
    arr["base_index"] = [_u64(f"base_indices[{i}]", b) for i, b in enumerate(base_indices)]
    arr["param_dtype"] = [_DTYPE_CODE[d] for d in pdt]
    arr["grad_dtype"] = [_DTYPE_CODE[d] for d in gdt]
    # p, m and v are written in place, so no buffer may share memory with another
    if n <= _SMALL_LIST:
        sizes = [[k * _ELEM_BYTES[d] for k, d in zip(numels, pdt)],
                 [k * _ELEM_BYTES[d] for k, d in zip(numels, gdt)],
                 [k * 4 for k in numels], [k * 4 for k in numels]]
        check_disjoint((a, b, f"{name}[{i}]")
                       for name, col, sz in zip(_STEP_NAMES, ptrs, sizes)
                       for i, (a, b) in enumerate(zip(col, sz)))
    else:
        num = np.asarray(numels, dtype=np.int64)
        sizes = [num * np.asarray([_ELEM_BYTES[d] for d in pdt], dtype=np.int64),
                 num * np.asarray([_ELEM_BYTES[d] for d in gdt], dtype=np.int64), num * 4, num * 4]
        starts = np.concatenate([np.asarray(c, dtype=np.uint64) for c in ptrs])
        _check_disjoint_arrays(starts, np.concatenate(sizes).astype(np.uint64),
                               lambda k: f"{_STEP_NAMES[k // n]}[{k % n}]")
    address = _abi.array_address(arr)
    return arr, address, _abi.asr_adamw_workspace_bytes_at(address, n)


def _check_disjoint_arrays(starts, nbytes, name_of):
    """check_disjoint over arrays of starts and sizes (uint64); name_of(k)
    names span k in the error."""
    live = np.nonzero(nbytes > 0)[0]
    if live.size < 2:
        return
    order = live[np.argsort(starts[live], kind="stable")]
    ends = starts[order] + nbytes[order]
    bad = np.nonzero(starts[order[1:]] < ends[:-1])[0]
    if bad.size:
        k0, k1 = int(order[bad[0]]), int(order[bad[0] + 1])
        raise ValueError(f"{name_of(k0)} and {name_of(k1)} share memory; every buffer of the "
                         "step must be disjoint from the others")


def _step_key(params, grads, exp_avgs, exp_avg_sqs, base_indices, device):
    """What the descriptors of a list depend on: addresses, sizes, dtypes,
    base indices and the device."""
    return (device, tuple(p.data_ptr() for p in params), tuple(g.data_ptr() for g in grads),
            tuple(m.data_ptr() for m in exp_avgs), tuple(v.data_ptr() for v in exp_avg_sqs),
            tuple(p.numel() for p in params), tuple(p.dtype for p in params),
            tuple(g.dtype for g in grads), tuple(base_indices))


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, base_indices, *, lr, beta1, beta2,
               eps, weight_decay, step, seed, rounding="sr", workspace=None, _cache=None):
    """One fused AdamW step over lists of tensors on one device (in place).

    params: f32 or bf16; grads: f32 or bf16, same numel as their param;
    exp_avgs / exp_avg_sqs: f32; base_indices: global position of element 0
    of each tensor. ``rounding`` ("sr" | "rn") applies to bf16 params.

    ``_cache`` (internal, for AdamWSR): a dict kept across steps of one
    list. The checked descriptor array is kept in it and reused while every
    tensor keeps its address, size and dtype and the base indices stay the
    same; anything else is checked again. Contiguity and the device are
    checked only then, so the caller must keep its tensors contiguous and on
    one device (AdamWSR checks its parameters and grads at every step).
    """
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == len(base_indices) == n):
        raise ValueError("all lists must have the same length")
    if rounding not in ROUNDING_CODE:
        raise ValueError("rounding must be 'sr' or 'rn'")
    seed = _u32("seed", seed)
    step = operator.index(step)
    if not 1 <= step < (1 << 32):
        raise ValueError("step must be in [1, 2**32 - 1]")
    if n == 0:
        return
    if not isinstance(params[0], torch.Tensor):
        raise TypeError("param[0] must be a torch.Tensor")
    device = params[0].device
    if device.type != "cuda":
        raise ValueError(f"param[0] must be on a GPU (got {device})")
    if _cache is not None:
        try:
            key = _step_key(params, grads, exp_avgs, exp_avg_sqs, base_indices, device)
        except (AttributeError, TypeError):   # not all tensors: the full check says why
            key = None
        if key is None or _cache.get("key") != key:
            _cache.clear()
            arr, address, need = _step_descriptors(params, grads, exp_avgs, exp_avg_sqs,
                                                   base_indices, device)
            if key is not None:   # (the array stays alive in the cache with its address)
                _cache.update(key=key, arr=arr, address=address, need=need)
        else:
            arr, address, need = _cache["arr"], _cache["address"], _cache["need"]
    else:
        arr, address, need = _step_descriptors(params, grads, exp_avgs, exp_avg_sqs,
                                               base_indices, device)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if workspace.device != device or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be on {device} and hold {need} bytes")
    with torch.cuda.device(device):
        _abi.asr_adamw_step_at(address, n, float(lr), float(beta1), float(beta2), float(eps),
                               float(weight_decay), step, seed, ROUNDING_CODE[rounding],
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream(device))


def philox_4x32_fill(n_counters, counter_base, seed, step, counter_upper=0, *, out=None,
                     device="cuda"):
    """Words of n_counters Philox4x32-10 calls as an int32 tensor of 4*n_counters
    (reinterpret as uint32)."""
    args = (_u64("counter_base", counter_base), _u64("counter_upper", counter_upper),
            _u32("seed", seed), _u32("step", step))
    if out is None:
        out = torch.empty(4 * n_counters, dtype=torch.int32, device=device)
    _require_gpu(out, "out")
    if out.dtype != torch.int32 or out.numel() != 4 * n_counters:
        raise ValueError("out must be int32 with 4*n_counters elements")
    with torch.cuda.device(out.device):
        _abi.asr_philox_4x32_fill(out.data_ptr(), n_counters, *args, _stream(out.device))
    return out


def _convert_args(x, out):
    _require_gpu(x, "x")
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _require_gpu(out, "out")
    if out.dtype != torch.bfloat16 or out.numel() != x.numel() or out.device != x.device:
        raise ValueError("out must be bfloat16 with x's size, on x's device")
    check_disjoint([_extent(x, "x"), _extent(out, "out")])
    return out


def cvt_f32_bf16_sr(x, seed, step, base_index=0, *, out=None):
    """Stochastic rounding f32 -> bf16 (element i at position base_index + i)."""
    key = (_u32("seed", seed), _u32("step", step), _u64("base_index", base_index))
    out = _convert_args(x, out)
    with torch.cuda.device(x.device):
        _abi.asr_cvt_f32_bf16_sr(x.data_ptr(), out.data_ptr(), x.numel(), *key, _stream(x.device))
    return out


def cvt_f32_bf16_rn(x, *, out=None):
    """Round-to-nearest-even f32 -> bf16."""
    out = _convert_args(x, out)
    with torch.cuda.device(x.device):
        _abi.asr_cvt_f32_bf16_rn(x.data_ptr(), out.data_ptr(), x.numel(), _stream(x.device))
    return out


def gemm_bf16(a, b, *, rounding="rn", seed=0, step=0, base_index=0, out=None, out_f32=None):
    """C = A B^T for bf16 A (M x K) and B (N x K), rounded to bf16.

    rounding "rn" (round to nearest even) or "sr" (stochastic: element
    (m, n) uses stream position base_index + m*N + n under key (seed,
    step)). ``out``: optional bf16 (M x N) destination, row stride >= N;
    ``out_f32``: optional float32 (M x N) tensor with the same strides as
    ``out`` that also receives the unrounded result. Returns ``out``.
    """
    if rounding not in ("rn", "sr"):
        raise ValueError("rounding must be 'rn' or 'sr'")
    key = (_u32("seed", seed), _u32("step", step), _u64("base_index", base_index))
    for t, name in ((a, "a"), (b, "b")):
        _require_gpu(t, name)
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise TypeError(f"{name} must be a 2-D bfloat16 tensor")
        if t.stride(1) != 1:
            raise ValueError(f"{name} must have unit stride along K")
    if a.device != b.device:
        raise ValueError("a and b must be on the same device")
    if a.shape[1] != b.shape[1]:
        raise ValueError(f"K mismatch: a is {tuple(a.shape)}, b is {tuple(b.shape)}")
    m, k = a.shape
    n = b.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (m, n) or out.device != a.device \
            or (m > 0 and n > 0 and out.stride(1) != 1):
        raise ValueError("out must be a bfloat16 (M, N) tensor with unit column stride")
    ldc = out.stride(0) if m > 1 else max(n, 1)
    f32_ptr = None
    if out_f32 is not None:
        if out_f32.dtype != torch.float32 or tuple(out_f32.shape) != (m, n) \
                or out_f32.device != a.device or out_f32.stride() != out.stride():
            raise ValueError("out_f32 must be a float32 (M, N) tensor with out's strides")
        f32_ptr = out_f32.data_ptr()
    outputs = [_extent(out, "out")] + ([_extent(out_f32, "out_f32")] if out_f32 is not None else [])
    check_disjoint(outputs)
    for o in outputs:
        for i in (_extent(a, "a"), _extent(b, "b")):
            check_disjoint([o, i])
    # a row stride only matters when there is a second row and a K to walk
    lda = a.stride(0) if m > 1 and k > 0 else max(k, 8)
    ldb = b.stride(0) if n > 1 and k > 0 else max(k, 8)
    code = ASR_ROUND_SR if rounding == "sr" else ASR_ROUND_RN
    with torch.cuda.device(a.device):
        _abi.asr_gemm_bf16(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, f32_ptr,
                           m, n, k, code, *key, _stream(a.device))
    return out


class RoundingMode:
    """Rounding modes of the f32 -> bf16 conversion ("Add stochastic rounding
    and philox RNG helpers", discussion: stochastic rounding as a rounding
    mode of the existing conversion, keyed by a seed)."""
    NEAREST = "rn"
    STOCHASTIC = "sr"


def to(x, dtype=torch.bfloat16, *, rounding=RoundingMode.NEAREST, seed=0, step=0, base_index=0,
       out=None):
    """x.to(dtype) with a choice of rounding, for float32 -> bfloat16.

    rounding NEAREST: round to nearest even. STOCHASTIC: element i uses the
    16 random bits of stream position base_index + i under key (seed, step)
    (asr_cvt_f32_bf16_sr). Any shape; x must be contiguous float32 on a GPU.
    A float32 -> float32 request returns x itself.
    """
    if dtype == x.dtype == torch.float32:
        return x
    if dtype != torch.bfloat16:
        raise NotImplementedError("to(): float32 -> bfloat16 only")
    if rounding in (RoundingMode.STOCHASTIC, "sr", "stochastic"):
        return cvt_f32_bf16_sr(x, seed, step, base_index, out=out)
    if rounding in (RoundingMode.NEAREST, "rn", "nearest"):
        return cvt_f32_bf16_rn(x, out=out)
    raise ValueError(f"unknown rounding {rounding!r}")


def f32_sqrt_div(a, b):
    """(sqrt(a), a / b) as the AdamW kernel evaluates them (test support)."""
    for t, name in ((a, "a"), (b, "b")):
        _require_gpu(t, name)
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if a.numel() != b.numel() or a.device != b.device:
        raise ValueError("a and b must match in size and device")
    s = torch.empty_like(a)
    d = torch.empty_like(a)
    with torch.cuda.device(a.device):
        _abi.asr_f32_sqrt_div(a.data_ptr(), b.data_ptr(), s.data_ptr(), d.data_ptr(), a.numel(),
                              _stream(a.device))
    return s, d


def sr_bf16_given_bits(x, r16, *, out=None):
    """SR f32 -> bf16 with caller-supplied random bits r16 (int16 tensor whose
    bit patterns are the 16-bit random values)."""
    _require_gpu(x, "x")
    _require_gpu(r16, "r16")
    if x.dtype != torch.float32 or r16.dtype != torch.int16 or r16.numel() != x.numel():
        raise ValueError("x must be float32 and r16 int16 of the same size")
    out = _convert_args(x, out)
    check_disjoint([_extent(r16, "r16"), _extent(out, "out")])
    with torch.cuda.device(x.device):
        _abi.asr_sr_bf16_given_bits(x.data_ptr(), r16.data_ptr(), out.data_ptr(), x.numel(),
                                    _stream(x.device))
    return out
