"""The AdamW step with fp32 states and an optional bf16 write-back (oracle side).

What the pages fix ("adamw-sr" kernels hub page):
  * intro: one decoupled-weight-decay Adam step per parameter, bf16
    write-back by unbiased stochastic rounding, no fp32 master copy;
  * Usage: a drop-in for torch.optim.AdamW; optimizer states are float32;
    parameters and gradients are f32 or bf16; stochastic rounding is on by
    default for bf16 parameters;
  * Correctness: f32 parameters track torch.optim.AdamW to < 1e-4 over 100
    steps; References: decoupled weight decay (Loshchilov and Hutter).

The pages print no update equation. Reading: the algorithm documented for
torch.optim.AdamW with amsgrad and maximize off (weight decay scaled by lr,
bias correction on, eps outside the square root), evaluated in binary32 in
this fixed order, every operation rounded to nearest even, no fused
multiply-add:

    m   = b1 * m + omb1 * g
    v   = b2 * v + omb2 * (g * g)
    den = sqrt(v) * inv_bc2_sqrt + eps
    upd = m / den
    p   = p * decay - step_size * upd

with the per-call constants formed once in binary64 and rounded to binary32:

    bc1 = 1 - beta1**t,  bc2 = 1 - beta2**t   (t >= 1, integer powers by
                                              binary powering from the low bit)
    decay = f32(1 - lr*wd); b1 = f32(beta1); omb1 = f32(1 - beta1)
    b2 = f32(beta2); omb2 = f32(1 - beta2); step_size = f32(lr / bc1)
    inv_bc2_sqrt = f32(1 / sqrt(bc2)); eps = f32(eps)

The decay acts on the current parameter value (the upcast bf16 value when
there is no master copy). sqrt(v) * (1/sqrt(bc2)) is the same real number
as torch's sqrt(v) / sqrt(bc2) with one division fewer per element.

Precision: the arithmetic is binary32 because the pages fix the states as
float32 and the bf16 result is decided from the binary32 bits of the new
parameter, so both sides must take that decision in the same precision.
"""

import math
from dataclasses import dataclass

import numpy as np

from .bf16 import bf16_to_f32, f32_bits, bits_f32, sr_bf16, rn_bf16, \
    sr_bf16_scalar, rn_bf16_scalar, f32_pattern
from .stream import random16, random16_scalar

F32, BF16 = 0, 1
ROUND_SR, ROUND_RN = 0, 1

# The float environment must keep subnormals: a flush-to-zero mode set by
# some loaded library would silently change results.
if np.float32(1e-40) * np.float32(1.0) == 0:
    raise RuntimeError("oracle: float32 subnormals are flushed on this host")


def powi(base, t):
    """base**t for an integer t >= 0 in binary64, by binary powering from the
    low bit: r *= b when the bit is set, then b *= b."""
    r, b, t = 1.0, float(base), int(t)
    while t:
        if t & 1:
            r *= b
        b *= b
        t >>= 1
    return r


@dataclass(frozen=True)
class HostScalars:
    decay: np.float32
    b1: np.float32
    omb1: np.float32
    b2: np.float32
    omb2: np.float32
    step_size: np.float32
    inv_bc2_sqrt: np.float32
    eps: np.float32


def host_scalars(lr, beta1, beta2, eps, weight_decay, step):
    """The eight binary32 constants of one step (formed in binary64), for the
    AdamW update torch.optim.AdamW documents ("adamw-sr" page, Usage: a
    drop-in for it; the page prints no formula, so its documented algorithm is
    the reading)."""
    if int(step) < 1:
        raise ValueError("step counts from 1")
    lr, beta1, beta2 = float(lr), float(beta1), float(beta2)
    bc1 = 1.0 - powi(beta1, step)
    bc2 = 1.0 - powi(beta2, step)
    f = np.float32
    return HostScalars(
        decay=f(1.0 - lr * float(weight_decay)),
        b1=f(beta1), omb1=f(1.0 - beta1),
        b2=f(beta2), omb2=f(1.0 - beta2),
        step_size=f(lr / bc1),
        inv_bc2_sqrt=f(1.0 / math.sqrt(bc2)),
        eps=f(eps),
    )


def adamw_f32(p, g, m, v, sc):
    """One element-wise AdamW update on float32 arrays ("adamw-sr" page, intro
    and Usage: decoupled-weight-decay Adam with float32 states), with numpy
    float32 ufuncs, each rounded to nearest even (numpy never fuses a
    multiply and an add). Returns (p, m, v) as new float32 arrays."""
    p, g, m, v = (np.asarray(x, dtype=np.float32) for x in (p, g, m, v))
    with np.errstate(all="ignore"):
        m = np.add(np.multiply(sc.b1, m), np.multiply(sc.omb1, g))
        v = np.add(np.multiply(sc.b2, v), np.multiply(sc.omb2, np.multiply(g, g)))
        den = np.add(np.multiply(np.sqrt(v), sc.inv_bc2_sqrt), sc.eps)
        upd = np.divide(m, den)
        p = np.subtract(np.multiply(p, sc.decay), np.multiply(sc.step_size, upd))
    return (p.astype(np.float32, copy=False), m.astype(np.float32, copy=False),
            v.astype(np.float32, copy=False))


# ---- scalar form: binary64 arithmetic, rounded to binary32 after every op.
# For +, -, *, / and sqrt of binary32 operands, computing in binary64 and
# rounding once more to binary32 gives the correctly rounded binary32 result
# (binary64 has more than 2*24+2 bits), so this form is exact without
# relying on numpy's float32 kernels.

def _r(x):
    with np.errstate(over="ignore"):
        return float(np.float32(x))


def _div(a, b):
    if b == 0.0:
        if a == 0.0 or math.isnan(a):
            return math.nan
        return math.copysign(math.inf, a) * math.copysign(1.0, b)
    return a / b


def _sqrt(x):
    if math.isnan(x) or x < 0:
        return math.nan
    return math.sqrt(x)


def adamw_f32_scalar(p, g, m, v, sc):
    """The same update on Python floats holding binary32 values."""
    b1, omb1, b2, omb2 = float(sc.b1), float(sc.omb1), float(sc.b2), float(sc.omb2)
    m = _r(_r(b1 * m) + _r(omb1 * g))
    v = _r(_r(b2 * v) + _r(omb2 * _r(g * g)))
    den = _r(_r(_r(_sqrt(v)) * float(sc.inv_bc2_sqrt)) + float(sc.eps))
    upd = _r(_div(m, den))
    p = _r(_r(p * float(sc.decay)) - _r(float(sc.step_size) * upd))
    return p, m, v


def _check_codes(param_dtype, grad_dtype, rounding):
    if param_dtype not in (F32, BF16) or grad_dtype not in (F32, BF16):
        raise ValueError("dtype codes are F32=0 or BF16=1")
    if rounding not in (ROUND_SR, ROUND_RN):
        raise ValueError("rounding is ROUND_SR=0 or ROUND_RN=1")


def _upcast(x, dtype):
    if dtype == BF16:
        return bf16_to_f32(np.asarray(x, dtype=np.uint16))
    return np.asarray(x, dtype=np.float32)


def step_tensor(param, grad, m, v, *, param_dtype, grad_dtype, base_index,
                lr, beta1, beta2, eps, weight_decay, step, seed, rounding=ROUND_SR):
    """One AdamW step of one tensor (numpy). ("adamw-sr" page, Method: the bf16
    write-back draws the random bits of each element from Philox keyed by
    (seed, step) at the element's global position base_index + i.)

    ``param``/``grad``: uint16 bf16 patterns when their dtype is BF16, else
    float32; ``m``/``v``: float32. Inputs are not modified.
    Returns (param_new, m_new, v_new) in the same representations.
    A bf16 parameter is written back by SR (random value of element i from
    global position base_index + i) or by RN; an f32 parameter is stored as
    computed and the rounding mode does not apply.
    """
    _check_codes(param_dtype, grad_dtype, rounding)
    sc = host_scalars(lr, beta1, beta2, eps, weight_decay, step)
    p32 = _upcast(param, param_dtype)
    g32 = _upcast(grad, grad_dtype)
    p_new, m_new, v_new = adamw_f32(p32, g32, m, v, sc)
    if param_dtype == F32:
        return p_new, m_new, v_new
    bits = f32_bits(p_new)
    if rounding == ROUND_RN:
        return rn_bf16(bits), m_new, v_new
    n = bits.size
    positions = (np.uint64(base_index) + np.arange(n, dtype=np.uint64))
    r16 = random16(positions, seed, step)
    return sr_bf16(bits, r16), m_new, v_new


def step_tensor_scalar(param, grad, m, v, *, param_dtype, grad_dtype, base_index,
                       lr, beta1, beta2, eps, weight_decay, step, seed,
                       rounding=ROUND_SR):
    """Pure-Python loop form of :func:`step_tensor` (tiny inputs only).
    Takes and returns Python lists (ints for bf16 patterns, floats for f32)."""
    _check_codes(param_dtype, grad_dtype, rounding)
    sc = host_scalars(lr, beta1, beta2, eps, weight_decay, step)

    def up(x, dt):
        if dt == BF16:
            return float(np.uint32(int(x) << 16).view(np.float32))
        return _r(float(x))

    out_p, out_m, out_v = [], [], []
    for i in range(len(param)):
        p, mm, vv = adamw_f32_scalar(up(param[i], param_dtype), up(grad[i], grad_dtype),
                                     _r(float(m[i])), _r(float(v[i])), sc)
        out_m.append(mm)
        out_v.append(vv)
        if param_dtype == F32:
            out_p.append(p)
            continue
        u = f32_pattern(p)
        if rounding == ROUND_RN:
            out_p.append(rn_bf16_scalar(u))
        else:
            pos = (int(base_index) + i) & 0xFFFFFFFFFFFFFFFF
            out_p.append(sr_bf16_scalar(u, random16_scalar(pos, seed, step)))
    return out_p, out_m, out_v


def step_list(tensors, *, lr, beta1, beta2, eps, weight_decay, step, seed,
              rounding=ROUND_SR):
    """One step over a list of tensors, each a dict with keys param, grad, m,
    v, param_dtype, grad_dtype, base_index. Tensors are independent ("adamw-sr"
    page, Correctness: pieces with their own base_index give the one-piece
    result); returns a list of (param_new, m_new, v_new)."""
    return [step_tensor(t["param"], t["grad"], t["m"], t["v"],
                        param_dtype=t["param_dtype"], grad_dtype=t["grad_dtype"],
                        base_index=t["base_index"], lr=lr, beta1=beta1,
                        beta2=beta2, eps=eps, weight_decay=weight_decay,
                        step=step, seed=seed, rounding=rounding)
            for t in tensors]


def bits_of(x):
    """Helper for comparisons: float32 array -> uint32 patterns."""
    return f32_bits(x)


def floats_of(u):
    return bits_f32(u)
