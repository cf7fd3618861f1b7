"""Pins of the oracle's AdamW step (CPU only).

What pins it:
  * the pure-Python form (binary64 rounded to binary32 after each op)
    against the numpy float32 form, on random and extreme inputs;
  * closed forms: the first step, where the bias-corrected moments are g and
    g**2 exactly, and a constant gradient, where every step moves by the
    same amount and the decay compounds geometrically;
  * torch.optim.AdamW on the CPU over 100 f32 steps, to the page's bound
    (adamw-sr page, Correctness section: < 1e-4 over 100 steps);
  * the sub-ULP example of the adamw-sr page's intro (6,000 steps of 1e-4
    from 1.0 toward 1.5): round-to-nearest never moves, stochastic rounding
    climbs, and repeats are bitwise identical;
  * shard invariance (adamw-sr page, Correctness section) and the
    composition "step in f32, then convert with SR" == "step with SR";
  * the binary64 powers behind the bias corrections against exact rationals.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.adamw import powi, F32, BF16, ROUND_SR, ROUND_RN

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _bf16(x):
    return oracle.rn_bf16(oracle.f32_bits(np.asarray(x, dtype=np.float32)))


def _ulp32(x):
    x = abs(float(x))
    if x < 2.0 ** -126:
        return 2.0 ** -149
    return 2.0 ** (math.floor(math.log2(x)) - 23)


# ---------------------------------------------------------------- host scalars

def test_powi_against_exact_rationals():
    rng = np.random.default_rng(0)
    for b in [0.9, 0.999, 0.95, 0.5, 0.0, 0.99999] + rng.uniform(0, 1, 20).tolist():
        for t in [1, 2, 3, 7, 10, 100, 1000, 6000]:
            got = powi(b, t)
            exact = Fraction(b) ** t
            if exact < Fraction(1, 1 << 1000):   # below binary64's normal range
                assert 0.0 <= got < 2.0 ** -1000
                continue
            # Any multiplication chain for b**t carries each rounding error
            # (at most 2**-53 relative) to a total power of at most t - 1.
            rel = abs(Fraction(got) - exact) / exact
            assert rel <= Fraction(t, 1 << 53) * Fraction(101, 100), (b, t)


def test_host_scalars_values():
    sc = oracle.host_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    assert sc.step_size == np.float32(1e-3 / (1 - 0.9))
    assert sc.decay == np.float32(1 - 1e-5)
    assert sc.inv_bc2_sqrt == np.float32(1 / math.sqrt(1 - 0.999))
    assert sc.omb1 == np.float32(1 - 0.9) and sc.omb2 == np.float32(1 - 0.999)
    with pytest.raises(ValueError):
        oracle.host_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 0)


# ------------------------------------------------------------- scalar vs numpy

def _edge_floats(rng, n):
    """f32 values spanning the exponent range, subnormals, zeros of both signs."""
    mant = rng.uniform(1, 2, n)
    exp = rng.integers(-149, 60, n)
    sign = rng.choice([-1.0, 1.0], n)
    x = (sign * mant * np.exp2(exp.astype(np.float64))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1e-45, -3e-39]
    return x


@pytest.mark.parametrize("pd,gd", [(F32, F32), (BF16, BF16), (BF16, F32), (F32, BF16)])
@pytest.mark.parametrize("rounding", [ROUND_SR, ROUND_RN])
def test_scalar_equals_numpy(pd, gd, rounding):
    rng = np.random.default_rng(pd * 4 + gd * 2 + rounding)
    n = 3000
    p = _edge_floats(rng, n)
    g = _edge_floats(rng, n)
    m = _edge_floats(rng, n)
    v = np.abs(_edge_floats(rng, n))
    param = _bf16(p) if pd == BF16 else p
    grad = _bf16(g) if gd == BF16 else g
    kw = dict(param_dtype=pd, grad_dtype=gd, base_index=(1 << 32) - 5, step=37, seed=123,
              rounding=rounding, lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-6, weight_decay=0.1)
    vp, vm, vv = oracle.step_tensor(param, grad, m, v, **kw)
    sp, sm, sv = oracle.step_tensor_scalar(param.tolist(), grad.tolist(), m.tolist(), v.tolist(), **kw)
    assert np.array_equal(oracle.f32_bits(vm), oracle.f32_bits(np.array(sm, np.float32)))
    assert np.array_equal(oracle.f32_bits(vv), oracle.f32_bits(np.array(sv, np.float32)))
    if pd == BF16:
        assert np.array_equal(vp, np.array(sp, np.uint16))
    else:
        assert np.array_equal(oracle.f32_bits(vp), oracle.f32_bits(np.array(sp, np.float32)))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("lr,wd,eps", [(1e-3, 0.01, 1e-8), (1e-2, 0.1, 1e-3), (5e-4, 0.0, 1e-5)])
def test_first_step_closed_form(lr, wd, eps):
    """t = 1 from m = v = 0: m/(1-b1) = g and v/(1-b2) = g**2 exactly, so
    p1 = p0 (1 - lr wd) - lr g / (|g| + eps). Binary32 evaluation error:
    half an ulp of p0 (1 - lr wd) and half an ulp of p1 from the last two
    roundings, plus about ten roundings of 2**-24 relative each in the update
    term, which is at most lr in size."""
    rng = np.random.default_rng(1)
    n = 20000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g[:100] = (rng.standard_normal(100) * 1e-4).astype(np.float32)  # eps matters here
    z = np.zeros(n, np.float32)
    p1, m1, v1 = oracle.step_tensor(p0, g, z, z, param_dtype=F32, grad_dtype=F32, base_index=0,
                                    lr=lr, beta1=0.9, beta2=0.999, eps=eps, weight_decay=wd,
                                    step=1, seed=0)
    exact = p0.astype(np.float64) * (1 - lr * wd) - lr * g / (np.abs(g.astype(np.float64)) + eps)
    decayed = p0.astype(np.float64) * (1 - lr * wd)
    tol = (0.5 * np.array([_ulp32(x) for x in decayed]) + 0.5 * np.array([_ulp32(x) for x in exact])
           + 16 * 2.0 ** -24 * lr)
    assert np.all(np.abs(p1.astype(np.float64) - exact) <= tol)


def test_constant_gradient_closed_form():
    """Constant g: the bias-corrected moments equal g and g**2 at every
    step, so every step subtracts u = lr g/(|g| + eps) after decaying by
    d = 1 - lr wd: p_t = d**t p0 - u (1 - d**t)/(1 - d). Binary32 error
    over 100 steps stays within ~100 roundings of the largest terms."""
    lr, wd, eps, T = 1e-3, 0.05, 1e-8, 100
    rng = np.random.default_rng(2)
    n = 4096
    p = (rng.standard_normal(n) * 0.05).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    p0 = p.astype(np.float64)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, T + 1):
        p, m, v = oracle.step_tensor(p, g, m, v, param_dtype=F32, grad_dtype=F32, base_index=0,
                                     lr=lr, beta1=0.9, beta2=0.999, eps=eps, weight_decay=wd,
                                     step=t, seed=0)
    d = 1 - lr * wd
    u = lr * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps)
    exact = d ** T * p0 - u * (1 - d ** T) / (1 - d)
    err = np.abs(p.astype(np.float64) - exact)
    assert np.all(err <= 200 * 2.0 ** -24 * (np.abs(p0) + T * lr)), err.max()


def test_tracks_torch_adamw_100_steps():
    claim = json.load(open(os.path.join(GOLDEN, "pages_claims.json")))["fp32_tracking"]
    n, T = 1 << 18, claim["steps"]
    gen = np.random.default_rng(3)
    p = (gen.standard_normal(n) * 0.02).astype(np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                            foreach=False)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, T + 1):
        g = (gen.standard_normal(n) * 1e-2).astype(np.float32)
        p, m, v = oracle.step_tensor(p, g, m, v, param_dtype=F32, grad_dtype=F32, base_index=0,
                                     step=t, seed=0, **HP)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
    diff = np.abs(p - tp.detach().numpy()).max()
    assert diff < claim["max_abs_diff"], diff
    assert diff < 1e-6  # the same algorithm: only rounding-order differences


# -------------------------------------------------------- sub-ULP accumulation

def _subulp_run(n, steps, rounding, seed, lr):
    w = np.full(n, 0x3F80, np.uint16)            # bf16 1.0
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, steps + 1):
        g = oracle.bf16_to_f32(w) - np.float32(1.5)   # exact in binary32
        w, m, v = oracle.step_tensor(w, g, m, v, param_dtype=BF16, grad_dtype=F32,
                                     base_index=0, lr=lr, beta1=0.9, beta2=0.999, eps=1e-8,
                                     weight_decay=0.0, step=t, seed=seed, rounding=rounding)
    return w


def _f32_trajectory(steps, lr):
    p = np.array([1.0], np.float32)
    m = np.zeros(1, np.float32)
    v = np.zeros(1, np.float32)
    for t in range(1, steps + 1):
        g = p - np.float32(1.5)
        p, m, v = oracle.step_tensor(p, g, m, v, param_dtype=F32, grad_dtype=F32, base_index=0,
                                     lr=lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                                     step=t, seed=0)
    return float(p[0])


def test_subulp_accumulation_example():
    ex = json.load(open(os.path.join(GOLDEN, "pages_claims.json")))["subulp_demo"]
    steps, lr, n = ex["steps"], ex["update_per_step"], 1024
    rn = _subulp_run(n, steps, ROUND_RN, 0, lr)
    assert np.all(rn == 0x3F80)                    # mean stays at the start exactly
    assert float(oracle.bf16_to_f32(rn).mean()) == ex["start"]
    sr = _subulp_run(n, steps, ROUND_SR, 0, lr)
    sr_again = _subulp_run(n, steps, ROUND_SR, 0, lr)
    assert np.array_equal(sr, sr_again)            # bitwise repeatable
    mean = float(oracle.bf16_to_f32(sr).astype(np.float64).mean())
    f32_end = _f32_trajectory(steps, lr)
    assert ex["start"] < mean < ex["target"]
    assert mean > 1.40 and abs(mean - f32_end) < 0.01, (mean, f32_end)
    other = _subulp_run(n, steps, ROUND_SR, 1, lr)
    assert not np.array_equal(other, sr)
    assert abs(float(oracle.bf16_to_f32(other).astype(np.float64).mean()) - mean) < 0.005


# ------------------------------------------------ sharding and composition

def _state(n, seed):
    rng = np.random.default_rng(seed)
    p = _bf16(rng.standard_normal(n) * 0.02)
    g = _bf16(rng.standard_normal(n) * 1e-3)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-7).astype(np.float32)
    return p, g, m, v


@pytest.mark.parametrize("base", [0, 1, 3, 5, (1 << 32) - 3, (1 << 32) + 5, (1 << 34) - 3, (1 << 34) + 5])
def test_whole_equals_shards(base):
    n = 10007
    p, g, m, v = _state(n, 4)
    kw = dict(param_dtype=BF16, grad_dtype=BF16, step=4, seed=2, **HP)
    whole = oracle.step_tensor(p, g, m, v, base_index=base, **kw)
    cuts = [0, 1, 7, 1000, 4093, 4096, 9000, n]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = oracle.step_tensor(p[a:b], g[a:b], m[a:b], v[a:b], base_index=base + a, **kw)
        for x, y in zip(part, whole):
            assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y[a:b]).view(np.uint8))


def test_list_order_does_not_matter():
    sizes = [5, 4096, 33, 8, 1000]
    tensors, base = [], 0
    for i, s in enumerate(sizes):
        p, g, m, v = _state(s, 10 + i)
        tensors.append(dict(param=p, grad=g, m=m, v=v, param_dtype=BF16, grad_dtype=BF16,
                            base_index=base))
        base += s
    kw = dict(step=2, seed=5, **HP)
    out = oracle.step_list(tensors, **kw)
    perm = [3, 0, 4, 2, 1]
    out_perm = oracle.step_list([tensors[i] for i in perm], **kw)
    for k, i in enumerate(perm):
        for x, y in zip(out_perm[k], out[i]):
            assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


def test_sr_step_is_f32_step_then_sr_convert():
    n = 5000
    p, g, m, v = _state(n, 6)
    base = (1 << 33) + 2
    kw = dict(grad_dtype=BF16, step=9, seed=77, **HP)
    got_p, got_m, got_v = oracle.step_tensor(p, g, m, v, param_dtype=BF16, base_index=base, **kw)
    f_p, f_m, f_v = oracle.step_tensor(oracle.bf16_to_f32(p), g, m, v, param_dtype=F32,
                                       base_index=base, **kw)
    assert np.array_equal(got_p, oracle.cvt_f32_bf16_sr(f_p, 77, 9, base))
    assert np.array_equal(got_m, f_m) and np.array_equal(got_v, f_v)
    rn_p, rn_m, _ = oracle.step_tensor(p, g, m, v, param_dtype=BF16, base_index=base,
                                       rounding=ROUND_RN, **kw)
    assert np.array_equal(rn_p, oracle.cvt_f32_bf16_rn(f_p))
    assert np.array_equal(rn_m, got_m)   # the moments do not depend on the rounding
