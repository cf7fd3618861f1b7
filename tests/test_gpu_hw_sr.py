"""The device SR rounding (gfx950's v_cvt_sr_bf16_f32, fed its 16 random bits
in the high half of its random operand) against the oracle's rule, through
asr_sr_bf16_given_bits:

  * every one of the 2**32 f32 patterns at four random values that sit on the
    carry boundaries (0, 0x7FFF, 0x8000, 0xFFFF);
  * every one of the 2**16 random values at 4,096 sampled inputs (random
    patterns, NaN payloads, Inf, FLT_MAX, subnormals, zeros, ties);
  * 2**24 random (x, r) pairs.

Bit-exact. This is the condition for letting the step and the conversion
kernels round with the hardware instruction instead of the integer form
(add the bits to the dropped half, truncate; NaN kept quiet)."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from adamw_optimizer_stochastic_amd import ops
from _gpu_util import gpu, require_gpu, announce, f32_tensor, to_host, assert_bits_equal

pytestmark = gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _r16_tensor(values, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(values, dtype=np.uint16).view(np.int16)).to(device)


def _mismatches(start, got, r16):
    u = np.arange(start, start + got.size, dtype=np.uint64).astype(np.uint32)
    want = oracle.sr_bf16(u, np.uint32(r16))
    return int(np.count_nonzero(want != got))


@pytest.mark.parametrize("r16", [0x0000, 0x7FFF, 0x8000, 0xFFFF])
def test_every_f32_at_fixed_random_value(r16):
    announce("hw sr exhaustive, r16 =", hex(r16))
    dev = torch.device("cuda", 0)
    big, sub = 1 << 28, 1 << 24
    r = torch.full((big,), np.uint16(r16).view(np.int16).item(), dtype=torch.int16, device=dev)
    bad = 0
    with ThreadPoolExecutor(max_workers=16) as pool:
        for start in range(0, 1 << 32, big):
            bits = torch.arange(start, start + big, dtype=torch.int64, device=dev)
            x = bits.to(torch.int32).view(torch.float32)    # low 32 bits: the pattern
            got = to_host(ops.sr_bf16_given_bits(x, r))
            futs = [pool.submit(_mismatches, start + k, got[k:k + sub], r16)
                    for k in range(0, big, sub)]
            bad += sum(f.result() for f in futs)
    assert bad == 0, f"{bad} patterns differ at r16={r16:#x}"


def _sampled_inputs(rng, k):
    u = rng.integers(0, 1 << 32, size=k, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FFFFFFF,
                        0xFFFFFFFF, 0xFF800001, 0x7FBFFFFF, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F0000,
                        0x7F7F8000, 0x00000000, 0x80000000, 0x00000001, 0x0000FFFF, 0x00010000,
                        0x007FFFFF, 0x807FFFFF, 0x3F808000, 0x3F818000, 0x3FFFFFFF, 0xBFFFFFFF],
                       dtype=np.uint32)
    u[:special.size] = special
    return u


def test_every_random_value_at_sampled_inputs():
    announce("hw sr: all r16 at sampled x")
    rng = np.random.default_rng(950)
    k = 4096
    u = _sampled_inputs(rng, k)
    r = np.arange(1 << 16, dtype=np.uint32)
    U = np.repeat(u, r.size)
    R = np.tile(r, k)
    got = to_host(ops.sr_bf16_given_bits(f32_tensor(U.view(np.float32)), _r16_tensor(R)))
    with ThreadPoolExecutor(max_workers=16) as pool:
        parts = [pool.submit(lambda a, b: oracle.sr_bf16(a, b), U[s:s + (1 << 24)],
                             R[s:s + (1 << 24)]) for s in range(0, U.size, 1 << 24)]
        want = np.concatenate([p.result() for p in parts])
    assert_bits_equal(got, want, "all random values at sampled inputs")


def test_random_pairs():
    announce("hw sr: random pairs")
    rng = np.random.default_rng(1)
    n = 1 << 24
    u = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    r = rng.integers(0, 1 << 16, size=n, dtype=np.uint32)
    got = to_host(ops.sr_bf16_given_bits(f32_tensor(u.view(np.float32)), _r16_tensor(r)))
    assert_bits_equal(got, oracle.sr_bf16(u, r), "random pairs")
    # an unaligned view takes the same path
    got2 = to_host(ops.sr_bf16_given_bits(f32_tensor(u.view(np.float32))[1:], _r16_tensor(r)[1:]))
    assert_bits_equal(got2, oracle.sr_bf16(u[1:], r[1:]), "random pairs, offset views")
