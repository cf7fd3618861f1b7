"""Random numbers beyond rounding (asr_random_uniform, asr_random_normal,
asr_dropout) and the to() conversion surface, against the oracle.

Uniform draws and dropout are integer decisions and exact binary32
operations on the stream words: bit-exact. Normal draws go through the
hardware log2, sin and cos units: test_box_muller_exhaustive measures, over
every input those units can receive here (2**24 values of u1, 2**24 of u2),
a radius error below 2**-22 relative and a sin/cos error below 2**-22
absolute. So |z - z_exact| <= r * (2**-22 + 2**-22 + 2**-44) + 2**-24 |z|.
After the final binary32 multiply and add, the normal draws are compared
within 2**-20 * (std * r + |mean| + |y|), about 2x that. The bf16 form must
be the round-to-nearest of the kernel's own f32 value.
Sizes cover one element, ragged tails, several workgroups and unaligned
starting positions (a pair split across pieces for the normal draws).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import rng as orng
from adamw_optimizer_stochastic_amd import random as arng, ops, RoundingMode, to
from _gpu_util import (gpu, require_gpu, announce, to_host, assert_bits_equal, f32_tensor,
                       bf16_tensor)

pytestmark = gpu

SIZES = [1, 3, 1023, 1025, 65537, (1 << 20) + 3]
BASES = [0, 1, 2, 3, (1 << 40) + 5]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("base", BASES)
def test_uniform_bit_exact(n, base):
    announce("uniform", n, base)
    seed, step = 1234, 5
    for low, high in ((0.0, 1.0), (-2.5, 7.25)):
        got = arng.uniform(n, low, high, seed=seed, step=step, base_index=base)
        want = orng.uniform_f32(n, seed, step, base, low, high)
        assert_bits_equal(to_host(got), want, f"uniform f32 n={n} base={base}")
        gotb = arng.uniform(n, low, high, seed=seed, step=step, base_index=base,
                            dtype=torch.bfloat16)
        assert_bits_equal(to_host(gotb), oracle.rn_bf16(oracle.f32_bits(want)),
                          f"uniform bf16 n={n} base={base}")


def test_uniform_pieces_reproduce_whole():
    announce("uniform pieces")
    n = 300001
    whole = to_host(arng.uniform(n, seed=9, step=2, base_index=10))
    cuts = [0, 1, 4099, 77777, 200002, n]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = to_host(arng.uniform(b - a, seed=9, step=2, base_index=10 + a))
        assert np.array_equal(part.view(np.uint32), whole[a:b].view(np.uint32))


def _normal_bound(y64, r, mean, std):
    # |z_f32 - z| <= r * 2**-21 (radius and sincos errors), then the binary32
    # multiply-add: half an ulp of |std z| and of |y| each, with slack
    return 2.0 ** -20 * (abs(std) * r + abs(mean) + np.abs(y64)) + 1e-30


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("base", [0, 1, 3, (1 << 40) + 5])
def test_normal_within_bound(n, base):
    announce("normal", n, base)
    seed, step = 77, 3
    for mean, std in ((0.0, 1.0), (1.5, 0.02)):
        got = to_host(arng.normal(n, mean, std, seed=seed, step=step, base_index=base))
        y64, r = orng.normal_f64(n, seed, step, base, mean, std)
        err = np.abs(got.astype(np.float64) - y64)
        bound = _normal_bound(y64, r, mean, std)
        assert np.all(err <= bound), f"max err/bound {np.max(err / bound)}"
        gotb = to_host(arng.normal(n, mean, std, seed=seed, step=step, base_index=base,
                                   dtype=torch.bfloat16))
        assert_bits_equal(gotb, to_host(ops.cvt_f32_bf16_rn(f32_tensor(got))),
                          "normal bf16 = rn(f32)")


E_RADIUS = 2.0 ** -22   # relative error of r = sqrt(-2 ln u1)
E_TRIG = 2.0 ** -22     # absolute error of cos(2 pi u2), sin(2 pi u2), incl. the product's rounding


def test_box_muller_exhaustive():
    """The Box-Muller pair (asr_box_muller_given_words, the device function
    the normal kernel runs) over every u1 (with u2 = 0) and every u2 (with
    u1 = 2**-24, the largest radius) against binary64."""
    announce("box-muller exhaustive")
    from adamw_optimizer_stochastic_amd import _abi
    dev = torch.device("cuda", 0)
    n = 1 << 24
    words = (torch.arange(n, dtype=torch.int64, device=dev) << 8).to(torch.int32)  # top 24 bits = k
    zeros = torch.zeros(n, dtype=torch.int32, device=dev)
    zc = torch.empty(n, dtype=torch.float32, device=dev)
    zs = torch.empty(n, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    k = np.arange(n, dtype=np.float64)
    # every u1 = (k + 1) * 2**-24, u2 = 0: zc = r, zs = 0
    _abi.asr_box_muller_given_words(words.data_ptr(), zeros.data_ptr(), zc.data_ptr(),
                                    zs.data_ptr(), n, st)
    torch.cuda.synchronize()
    r_dev = to_host(zc).astype(np.float64)
    assert np.all(to_host(zs) == 0)
    r64 = np.sqrt(-2.0 * np.log((k + 1) * 2.0 ** -24))
    assert r_dev[-1] == 0.0 and np.signbit(np.float32(r_dev[-1])) == False  # u1 = 1: r = +0
    e_r = np.max(np.abs(r_dev[:-1] - r64[:-1]) / r64[:-1])
    # every u2 = k * 2**-24 at u1 = 2**-24
    _abi.asr_box_muller_given_words(zeros.data_ptr(), words.data_ptr(), zc.data_ptr(),
                                    zs.data_ptr(), n, st)
    torch.cuda.synchronize()
    rd = r_dev[0]
    theta = 2.0 * np.pi * k * 2.0 ** -24
    e_t = max(np.max(np.abs(to_host(zc).astype(np.float64) / rd - np.cos(theta))),
              np.max(np.abs(to_host(zs).astype(np.float64) / rd - np.sin(theta))))
    announce(f"radius error 2**{np.log2(e_r):.2f} relative, sin/cos error 2**{np.log2(e_t):.2f}")
    assert e_r <= E_RADIUS
    assert e_t <= E_TRIG


def test_normal_pieces_and_statistics():
    announce("normal pieces/stats")
    n = 1 << 22
    whole = to_host(arng.normal(n, seed=5, step=1, base_index=3))
    part = to_host(arng.normal(n - 1001, seed=5, step=1, base_index=3 + 1001))  # odd cut
    assert np.array_equal(part.view(np.uint32), whole[1001:].view(np.uint32))
    z = whole.astype(np.float64)
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / n)


SPECIALS = np.array([np.inf, -np.inf, np.nan, -3.0, 0.0, -0.0, 1e-40, 3.4e38], dtype=np.float32)


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.9, 0.999])
@pytest.mark.parametrize("n,base", [(1, 0), (1023, 1), (65537, 2), ((1 << 20) + 3, (1 << 40) + 5)])
def test_dropout_bit_exact(p, n, base):
    announce("dropout", p, n, base)
    g = np.random.default_rng(n)
    x = g.standard_normal(n).astype(np.float32)
    x[: min(n, SPECIALS.size)] = SPECIALS[: min(n, SPECIALS.size)]
    seed, step = 31, 8
    y, mask = arng.dropout(f32_tensor(x), p, seed=seed, step=step, base_index=base,
                           return_mask=True)
    wy, wk = orng.dropout_f32(x, p, seed, step, base)
    assert_bits_equal(to_host(y), wy, f"dropout f32 p={p}")
    assert np.array_equal(to_host(mask.view(torch.uint8)).astype(bool), wk)
    xb = oracle.rn_bf16(oracle.f32_bits(x)).astype(np.uint16)
    yb = arng.dropout(bf16_tensor(xb), p, seed=seed, step=step, base_index=base)
    wyb, _ = orng.dropout_bf16(xb, p, seed, step, base)
    assert_bits_equal(to_host(yb), wyb, f"dropout bf16 p={p}")


def test_dropout_in_place_and_eval():
    announce("dropout in place")
    x = np.linspace(-3, 3, 4099, dtype=np.float32)
    t = f32_tensor(x)
    want, _ = orng.dropout_f32(x, 0.3, 4, 4, 0)
    out = arng.dropout(t, 0.3, seed=4, step=4, inplace=True)
    assert out.data_ptr() == t.data_ptr()
    assert_bits_equal(to_host(t), want, "in place")
    same = arng.dropout(t, 0.3, seed=4, step=4, training=False)
    assert same is t


def test_to_surface():
    announce("to()")
    g = np.random.default_rng(2)
    x = g.standard_normal((37, 129)).astype(np.float32)
    t = f32_tensor(x)
    rn = to(t, torch.bfloat16)
    assert rn.shape == t.shape and rn.dtype == torch.bfloat16
    assert_bits_equal(to_host(rn).reshape(-1), oracle.cvt_f32_bf16_rn(x), "to rn")
    sr = to(t, torch.bfloat16, rounding=RoundingMode.STOCHASTIC, seed=3, step=1, base_index=11)
    assert_bits_equal(to_host(sr).reshape(-1), oracle.cvt_f32_bf16_sr(x, 3, 1, 11), "to sr")
    assert to(t, torch.float32) is t
    with pytest.raises(NotImplementedError):
        to(t, torch.float16)


def test_full_size_sampled():
    """Dropout and normal draws over 2**30 elements in the launch
    configuration the benchmark times; sampled positions against the oracle."""
    announce("rng full size 2**30")
    n = 1 << 30
    dev = torch.device("cuda", 0)
    x = torch.empty(n, dtype=torch.float32, device=dev)
    arng.normal_(x, seed=1, step=0)
    idx = np.unique(np.concatenate([np.random.default_rng(0).integers(0, n, 4096),
                                    [0, 1, 2, 3, n - 4, n - 3, n - 2, n - 1]]))
    xi = to_host(x[torch.from_numpy(idx).to(dev)])
    # each sampled element on its own: the oracle at base = its position
    y64 = np.array([orng.normal_f64(1, 1, 0, int(i))[0][0] for i in idx])
    r = np.array([orng.normal_f64(1, 1, 0, int(i))[1][0] for i in idx])
    assert np.all(np.abs(xi.astype(np.float64) - y64) <= _normal_bound(y64, r, 0.0, 1.0))
    y = torch.empty_like(x)
    mask = torch.empty(n, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        from adamw_optimizer_stochastic_amd import _abi
        _abi.asr_dropout(x.data_ptr(), y.data_ptr(), mask.data_ptr(), _abi.ASR_F32, n, 0.1, 2, 0,
                         0, ops._stream(dev))
    torch.cuda.synchronize()
    yi = to_host(y[torch.from_numpy(idx).to(dev)])
    mi = to_host(mask[torch.from_numpy(idx).to(dev)])
    for k, i in enumerate(idx):
        wy, wk = orng.dropout_f32(xi[k:k + 1], 0.1, 2, 0, int(i))
        assert yi[k].view(np.uint32) == wy[0].view(np.uint32) and bool(mi[k]) == bool(wk[0])
    del x, y, mask


@pytest.mark.parametrize("offset", [1, 2, 3, 6])
@pytest.mark.parametrize("base", [7, (1 << 64) - 3])
def test_unaligned_views_and_wrap_with_guards(offset, base):
    """Dropout (with mask) and uniform fills into views that start `offset`
    elements into their storage and end 3 before its end, f32 and bf16;
    positions that cross 2**64. Bit-exact against the oracle, and nothing
    outside the views is written."""
    from adamw_optimizer_stochastic_amd import _abi
    announce("rng unaligned", offset, base)
    n, tail, seed, step, p = 5000, 3, 17, 3, 0.3
    total = n + offset + tail
    stream = torch.cuda.current_stream().cuda_stream
    x = np.random.default_rng(offset).standard_normal(total).astype(np.float32)
    for dtype, code in ((torch.float32, _abi.ASR_F32), (torch.bfloat16, _abi.ASR_BF16)):
        if dtype == torch.float32:
            xd, xs = f32_tensor(x), x[offset:offset + n]
        else:
            xb = oracle.rn_bf16(oracle.f32_bits(x)).astype(np.uint16)
            xd, xs = bf16_tensor(xb), xb[offset:offset + n]
        y = torch.zeros(total, dtype=dtype, device="cuda")
        mk = torch.full((total,), 7, dtype=torch.uint8, device="cuda")
        _abi.asr_dropout(xd[offset:].data_ptr(), y[offset:].data_ptr(), mk[offset:].data_ptr(),
                         code, n, p, seed, step, base, stream)
        wy, wk = (orng.dropout_f32 if code == _abi.ASR_F32 else orng.dropout_bf16)(
            xs, p, seed, step, base)
        gy, gm = to_host(y), to_host(mk)
        assert_bits_equal(gy[offset:offset + n], wy, f"dropout {dtype}")
        assert np.array_equal(gm[offset:offset + n].astype(bool), wk)
        assert not gy[:offset].any() and not gy[offset + n:].any()
        assert np.all(gm[:offset] == 7) and np.all(gm[offset + n:] == 7)
        u = torch.zeros(total, dtype=dtype, device="cuda")
        _abi.asr_random_uniform(u[offset:].data_ptr(), code, n, -1.0, 2.0, seed, step, base,
                                stream)
        wu = orng.uniform_f32(n, seed, step, base, -1.0, 2.0)
        if code == _abi.ASR_BF16:
            wu = oracle.rn_bf16(oracle.f32_bits(wu))
        gu = to_host(u)
        assert_bits_equal(gu[offset:offset + n], wu, f"uniform {dtype}")
        assert not gu[:offset].any() and not gu[offset + n:].any()
