"""ctypes binding of the C ABI in include/adamw_sr.h (argument marshalling only).

Every function here has the name of the C entry point it calls and takes
plain integers for pointers and streams; it raises AsrError on a non-zero
status. Nothing here computes any part of the step: all of it runs in the
HIP kernels of libadamw_sr.so. The library is loaded on first use and its
absence is an error, never a fallback.
"""

import ctypes
import os
import threading

from ._build import LIB_PATH

ASR_OK, ASR_EINVAL, ASR_EDTYPE, ASR_EALIGN, ASR_EWORKSPACE, ASR_EHIP = range(6)
ASR_F32, ASR_BF16 = 0, 1
ASR_ROUND_SR, ASR_ROUND_RN = 0, 1
ASR_PROBE_READ, ASR_PROBE_WRITE, ASR_PROBE_COPY = 0, 1, 2
ABI_VERSION = 107

STATUS_NAMES = {ASR_OK: "ASR_OK", ASR_EINVAL: "ASR_EINVAL", ASR_EDTYPE: "ASR_EDTYPE",
                ASR_EALIGN: "ASR_EALIGN", ASR_EWORKSPACE: "ASR_EWORKSPACE",
                ASR_EHIP: "ASR_EHIP"}


class AsrError(RuntimeError):
    def __init__(self, status, func, message):
        self.status = status
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {message}")


class AsrTensor(ctypes.Structure):
    """asr_tensor (56 bytes)."""
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
        ("base_index", ctypes.c_uint64),
        ("param_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
    ]


# The same layout as a numpy structured dtype, so that a list's descriptors
# can be filled column by column.
ASR_TENSOR_DTYPE = None


def _tensor_dtype():
    import numpy as np
    dt = np.dtype([("param", np.uint64), ("grad", np.uint64), ("exp_avg", np.uint64),
                   ("exp_avg_sq", np.uint64), ("numel", np.int64), ("base_index", np.uint64),
                   ("param_dtype", np.int32), ("grad_dtype", np.int32)])
    assert dt.itemsize == ctypes.sizeof(AsrTensor)
    for name, _ in AsrTensor._fields_:
        assert dt.fields[name][1] == getattr(AsrTensor, name).offset, name
    return dt


ASR_TENSOR_DTYPE = _tensor_dtype()

_c = ctypes
_SIGNATURES = {
    "asr_abi_version": (_c.c_int, []),
    "asr_last_error": (_c.c_char_p, []),
    "asr_adamw_workspace_bytes": (_c.c_size_t, [_c.POINTER(AsrTensor), _c.c_int32]),
    "asr_adamw_host_scalars": (_c.c_int, [_c.c_double] * 5 + [_c.c_int64, _c.POINTER(_c.c_float)]),
    "asr_adamw_step": (_c.c_int, [_c.POINTER(AsrTensor), _c.c_int32] + [_c.c_double] * 5 +
                       [_c.c_int64, _c.c_uint32, _c.c_int32, _c.c_void_p, _c.c_size_t,
                        _c.c_void_p]),
    "asr_adamw_step_noalloc": (_c.c_int, [_c.POINTER(AsrTensor), _c.c_int32] + [_c.c_double] * 5 +
                               [_c.c_int64, _c.c_uint32, _c.c_int32, _c.c_void_p]),
    "asr_philox_4x32_fill": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_uint64, _c.c_uint64,
                                        _c.c_uint32, _c.c_uint32, _c.c_void_p]),
    "asr_cvt_f32_bf16_sr": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_uint32,
                                       _c.c_uint32, _c.c_uint64, _c.c_void_p]),
    "asr_cvt_f32_bf16_rn": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "asr_f32_sqrt_div": (_c.c_int, [_c.c_void_p] * 4 + [_c.c_int64, _c.c_void_p]),
    "asr_random_uniform": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_int64, _c.c_double,
                                      _c.c_double, _c.c_uint32, _c.c_uint32, _c.c_uint64,
                                      _c.c_void_p]),
    "asr_random_normal": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_int64, _c.c_double,
                                     _c.c_double, _c.c_uint32, _c.c_uint32, _c.c_uint64,
                                     _c.c_void_p]),
    "asr_dropout": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_int64,
                               _c.c_double, _c.c_uint32, _c.c_uint32, _c.c_uint64,
                               _c.c_void_p]),
    "asr_box_muller_given_words": (_c.c_int, [_c.c_void_p] * 4 + [_c.c_int64, _c.c_void_p]),
    "asr_stream_copy": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "asr_hbm_probe": (_c.c_int, [_c.c_int32, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "asr_adamw_stream_probe": (_c.c_int, [_c.POINTER(AsrTensor), _c.c_int32, _c.c_void_p,
                                          _c.c_size_t, _c.c_void_p]),
    "asr_gemm_bf16": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_int64, _c.c_void_p,
                                 _c.c_int64, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                                 _c.c_int32, _c.c_uint32, _c.c_uint32, _c.c_uint64,
                                 _c.c_void_p]),
    "asr_sr_bf16_given_bits": (_c.c_int, [_c.c_void_p] * 3 + [_c.c_int64, _c.c_void_p]),
}

_lock = threading.Lock()
_lib = None


def lib():
    """The loaded library (loads it on first call)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is not built; run __graft_entry__.build() "
                        "(or python -m adamw_optimizer_stochastic_amd._build)")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                if handle.asr_abi_version() != ABI_VERSION:
                    raise RuntimeError("libadamw_sr.so ABI version mismatch; rebuild it")
                # the step's entry points once more, taking the descriptor
                # array as a plain address (a numpy array's buffer)
                for name in ("asr_adamw_workspace_bytes", "asr_adamw_step"):
                    res, args = _SIGNATURES[name]
                    fn = handle[name]   # a separate function object for the same symbol
                    fn.restype = res
                    fn.argtypes = [_c.c_void_p] + args[1:]
                    _by_address[name] = fn
                _lib = handle
    return _lib


_by_address = {}


def _check(status, func):
    if status != ASR_OK:
        raise AsrError(status, func, lib().asr_last_error().decode(errors="replace"))


def asr_abi_version():
    return lib().asr_abi_version()


def asr_last_error():
    return lib().asr_last_error().decode(errors="replace")


def _tensor_array(tensors):
    n = len(tensors)
    arr = (AsrTensor * max(n, 1))()
    for i, t in enumerate(tensors):
        arr[i] = t if isinstance(t, AsrTensor) else AsrTensor(**t)
    return arr, n


def asr_adamw_workspace_bytes(tensors):
    """tensors: sequence of AsrTensor (or dicts); only numel is read."""
    arr, n = _tensor_array(tensors)
    return int(lib().asr_adamw_workspace_bytes(arr if n else None, n))


def array_address(arr):
    """The address of a numpy ASR_TENSOR_DTYPE array's descriptors, for the
    *_at entry points (None for an empty array). The array must stay alive
    while the address is used."""
    if arr.dtype != ASR_TENSOR_DTYPE or not arr.flags.c_contiguous:
        raise TypeError("descriptor array must be a C-contiguous ASR_TENSOR_DTYPE array")
    return arr.ctypes.data if arr.size else None


def asr_adamw_workspace_bytes_at(address, n):
    """asr_adamw_workspace_bytes for n descriptors at `address` (array_address)."""
    lib()
    return int(_by_address["asr_adamw_workspace_bytes"](address, n))


def asr_adamw_step_at(address, n, lr, beta1, beta2, eps, weight_decay, step, seed, rounding,
                      workspace, workspace_bytes, stream):
    """asr_adamw_step for n descriptors at `address` (array_address)."""
    lib()
    _check(_by_address["asr_adamw_step"](address, n, lr, beta1, beta2, eps, weight_decay, step,
                                         seed, rounding, workspace, workspace_bytes, stream),
           "asr_adamw_step")


def asr_adamw_host_scalars(lr, beta1, beta2, eps, weight_decay, step):
    """The eight binary32 constants (decay, b1, omb1, b2, omb2, step_size,
    inv_bc2_sqrt, eps32), as Python floats."""
    out = (ctypes.c_float * 8)()
    _check(lib().asr_adamw_host_scalars(lr, beta1, beta2, eps, weight_decay, step, out),
           "asr_adamw_host_scalars")
    return [float(x) for x in out]


def asr_adamw_step(tensors, lr, beta1, beta2, eps, weight_decay, step, seed, rounding,
                   workspace, workspace_bytes, stream):
    """tensors: sequence of AsrTensor (or of dicts with its field names)."""
    arr, n = _tensor_array(tensors)
    _check(lib().asr_adamw_step(arr if n else None, n, lr, beta1, beta2, eps, weight_decay,
                                step, seed, rounding, workspace, workspace_bytes, stream),
           "asr_adamw_step")


def asr_adamw_step_noalloc(tensors, lr, beta1, beta2, eps, weight_decay, step, seed, rounding,
                           stream):
    """asr_adamw_step on the library's static scratch (no workspace)."""
    arr, n = _tensor_array(tensors)
    _check(lib().asr_adamw_step_noalloc(arr if n else None, n, lr, beta1, beta2, eps,
                                        weight_decay, step, seed, rounding, stream),
           "asr_adamw_step_noalloc")


def asr_philox_4x32_fill(out, n_counters, counter_base, counter_upper, seed, step, stream):
    _check(lib().asr_philox_4x32_fill(out, n_counters, counter_base, counter_upper, seed, step,
                                      stream), "asr_philox_4x32_fill")


def asr_cvt_f32_bf16_sr(inp, out, n, seed, step, base_index, stream):
    _check(lib().asr_cvt_f32_bf16_sr(inp, out, n, seed, step, base_index, stream),
           "asr_cvt_f32_bf16_sr")


def asr_cvt_f32_bf16_rn(inp, out, n, stream):
    _check(lib().asr_cvt_f32_bf16_rn(inp, out, n, stream), "asr_cvt_f32_bf16_rn")


def asr_f32_sqrt_div(a, b, sqrt_out, div_out, n, stream):
    _check(lib().asr_f32_sqrt_div(a, b, sqrt_out, div_out, n, stream), "asr_f32_sqrt_div")


def asr_gemm_bf16(a, lda, b, ldb, c, ldc, c_f32, m, n, k, rounding, seed, step, base_index,
                  stream):
    _check(lib().asr_gemm_bf16(a, lda, b, ldb, c, ldc, c_f32, m, n, k, rounding, seed, step,
                               base_index, stream), "asr_gemm_bf16")


def asr_random_uniform(out, dtype, n, low, high, seed, step, base_index, stream):
    _check(lib().asr_random_uniform(out, dtype, n, low, high, seed, step, base_index, stream),
           "asr_random_uniform")


def asr_random_normal(out, dtype, n, mean, std, seed, step, base_index, stream):
    _check(lib().asr_random_normal(out, dtype, n, mean, std, seed, step, base_index, stream),
           "asr_random_normal")


def asr_dropout(x, y, mask, dtype, n, p, seed, step, base_index, stream):
    _check(lib().asr_dropout(x, y, mask, dtype, n, p, seed, step, base_index, stream),
           "asr_dropout")


def asr_box_muller_given_words(w_even, w_odd, zc, zs, n, stream):
    _check(lib().asr_box_muller_given_words(w_even, w_odd, zc, zs, n, stream),
           "asr_box_muller_given_words")


def asr_stream_copy(dst, src, nbytes, stream):
    _check(lib().asr_stream_copy(dst, src, nbytes, stream), "asr_stream_copy")


def asr_sr_bf16_given_bits(x, r16, out, n, stream):
    _check(lib().asr_sr_bf16_given_bits(x, r16, out, n, stream), "asr_sr_bf16_given_bits")


def asr_hbm_probe(kind, dst, src, nbytes, stream):
    _check(lib().asr_hbm_probe(kind, dst, src, nbytes, stream), "asr_hbm_probe")


def asr_adamw_stream_probe(tensors, workspace, workspace_bytes, stream):
    """tensors: sequence of AsrTensor (or dicts); destroys the params."""
    arr, n = _tensor_array(tensors)
    _check(lib().asr_adamw_stream_probe(arr if n else None, n, workspace, workspace_bytes,
                                        stream), "asr_adamw_stream_probe")
