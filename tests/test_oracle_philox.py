"""Pins of the oracle's Philox4x32-10 (CPU only).

What pins it, none of which re-types the oracle's code:
  * Triton's own Philox (``tl.philox`` with 10 rounds, run by Triton's CPU
    interpreter), the generator behind ``tl.rand`` that the FlyDSL page's
    discussion section names as prior art. Constants, round structure, key
    schedule and word order must all agree for random counters and keys.
  * The pure-Python form against the numpy form.
  * Bijection: every round is invertible (both multipliers are odd), so an
    inverse written here from the round definition must undo the oracle.
  * Statistics the FlyDSL page's Tests section asks of the device generator:
    uniform words and no collisions.
"""

import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle
from oracle.philox import MUL_A, MUL_B, WEYL_A, WEYL_B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
M32 = 0xFFFFFFFF

_TRITON_SCRIPT = textwrap.dedent(r"""
    import os, sys
    os.environ["TRITON_INTERPRET"] = "1"
    import numpy as np, torch, triton, triton.language as tl

    @triton.jit
    def _kern(c0p, c1p, c2p, c3p, keyp, out, N: tl.constexpr):
        i = tl.arange(0, N)
        k = tl.load(keyp + i)
        a, b, c, d = tl.philox(k, tl.load(c0p + i), tl.load(c1p + i),
                               tl.load(c2p + i), tl.load(c3p + i), 10)
        tl.store(out + i * 4 + 0, a)
        tl.store(out + i * 4 + 1, b)
        tl.store(out + i * 4 + 2, c)
        tl.store(out + i * 4 + 3, d)

    src = np.load(sys.argv[1])
    ctr, key = src["ctr"], src["key"]
    n = ctr.shape[1]
    blk = 4096
    out = np.empty((n, 4), dtype=np.uint32)
    for s in range(0, n, blk):
        cs = [torch.from_numpy(np.ascontiguousarray(ctr[w, s:s + blk]).view(np.int32)).view(torch.uint32)
              for w in range(4)]
        ks = torch.from_numpy(np.ascontiguousarray(key[s:s + blk]).view(np.int64))
        o = torch.zeros(4 * blk, dtype=torch.uint32)
        _kern[(1,)](*cs, ks, o, N=blk)
        out[s:s + blk] = o.view(torch.int32).numpy().view(np.uint32).reshape(blk, 4)
    np.save(sys.argv[2], out)
""")


def _triton_available():
    try:
        import triton  # noqa: F401
        return True
    except Exception:
        return False


@pytest.mark.skipif(not _triton_available(), reason="triton not importable")
def test_matches_triton_interpreter(tmp_path):
    n = 1 << 16
    rng = np.random.default_rng(20241202)
    ctr = rng.integers(0, 1 << 32, size=(4, n), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 1 << 64, size=n, dtype=np.uint64, endpoint=False)
    # Structured corners: zero counter and key, all-ones words, one-hot words.
    ctr[:, 0] = 0
    key[0] = 0
    ctr[:, 1] = M32
    key[1] = (1 << 64) - 1
    for w in range(4):
        ctr[:, 2 + w] = 0
        ctr[w, 2 + w] = 1
    src = tmp_path / "in.npz"
    dst = tmp_path / "out.npy"
    np.savez(src, ctr=ctr, key=key)
    script = tmp_path / "tri.py"
    script.write_text(_TRITON_SCRIPT)
    env = dict(os.environ, TRITON_INTERPRET="1")
    subprocess.run([sys.executable, str(script), str(src), str(dst)], check=True,
                   env=env, cwd=ROOT, timeout=600)
    want = np.load(dst)
    got = np.stack(oracle.philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3],
                                        key & np.uint64(M32), key >> np.uint64(32)), -1)
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} mismatching calls, first at {bad[:5]}"


def test_scalar_equals_vectorized():
    """The pure-Python scalar form against the numpy form on 2**20 random
    (counter, key) pairs."""
    rng = np.random.default_rng(7)
    n = 1 << 20
    ctr = rng.integers(0, 1 << 32, size=(4, n), dtype=np.uint64)
    key = rng.integers(0, 1 << 32, size=(2, n), dtype=np.uint64)
    vec = np.stack(oracle.philox4x32_10(*ctr, *key), -1)
    for i in range(n):
        s = oracle.philox4x32_10_scalar(ctr[:, i], key[:, i])
        assert tuple(int(x) for x in vec[i]) == s, i


def _inverse_round(d, k0, k1):
    """Undo one round, from the round's definition: word 3 is the low half
    of MUL_A*c0 and word 1 the low half of MUL_B*c2, so c0 and c2 come back
    through the multiplicative inverses; the high halves then unmask c3, c1."""
    inv_a = pow(MUL_A, -1, 1 << 32)
    inv_b = pow(MUL_B, -1, 1 << 32)
    d0, d1, d2, d3 = d
    c0 = (d3 * inv_a) & M32
    c2 = (d1 * inv_b) & M32
    c3 = d2 ^ ((MUL_A * c0) >> 32) ^ k1
    c1 = d0 ^ ((MUL_B * c2) >> 32) ^ k0
    return c0, c1, c2, c3


def test_bijection_inverse():
    rng = np.random.default_rng(11)
    for _ in range(2000):
        ctr = tuple(int(x) for x in rng.integers(0, 1 << 32, size=4, dtype=np.uint64))
        key = tuple(int(x) for x in rng.integers(0, 1 << 32, size=2, dtype=np.uint64))
        out = oracle.philox4x32_10_scalar(ctr, key)
        keys = [((key[0] + r * WEYL_A) & M32, (key[1] + r * WEYL_B) & M32) for r in range(10)]
        d = out
        for k0, k1 in reversed(keys):
            d = _inverse_round(d, k0, k1)
        assert d == ctr


def test_collision_free_128bit_and_birthday_32bit():
    n = 1 << 20
    words = oracle.philox_fill(n, 0, 1234, 5).reshape(n, 4)
    as_bytes = np.ascontiguousarray(words).view(np.dtype((np.void, 16)))
    assert np.unique(as_bytes).size == n  # distinct counters -> distinct outputs
    # Word 0 alone: collisions among n 32-bit values follow the birthday
    # count, expectation n(n-1)/2**33 = 128 here (Poisson, sd ~11.3).
    collisions = n - np.unique(words[:, 0]).size
    assert 128 - 6 * 11.3 < collisions < 128 + 6 * 11.3, collisions


def test_uniform_16bit_values():
    # 2**22 calls -> 2**24 random 16-bit values; chi-square over 65,536 bins.
    words = oracle.philox_fill(1 << 22, 1 << 40, 99, 3)
    r16 = words & np.uint32(0xFFFF)
    counts = np.bincount(r16, minlength=1 << 16)
    expected = r16.size / (1 << 16)
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    dof = (1 << 16) - 1
    assert abs(chi2 - dof) < 6 * np.sqrt(2 * dof), chi2
    # Per-bit balance of the full 32-bit words.
    n = words.size
    for b in range(32):
        ones = int(((words >> np.uint32(b)) & np.uint32(1)).sum())
        assert abs(ones - n / 2) < 5 * np.sqrt(n / 4), (b, ones)


def test_fill_layout_and_stream_words():
    # philox_fill(k) words == per-call words; random16 picks word p & 3 of
    # call p >> 2 (checked with the pure-Python forms).
    base = (1 << 34) - 3
    words = oracle.philox_fill(5, base, 17, 9, counter_upper=(3 << 32) | 2)
    for k in range(5):
        c = base + k
        want = oracle.philox4x32_10_scalar((c & M32, c >> 32, 2, 3), (17, 9))
        assert tuple(int(x) for x in words[4 * k:4 * k + 4]) == want
    pos = np.array([0, 1, 2, 3, 4, 5, (1 << 32) - 1, 1 << 32, (1 << 34) + 5], dtype=np.uint64)
    vec = oracle.random16(pos, 17, 9)
    for p, r in zip(pos.tolist(), vec.tolist()):
        j = p >> 2
        w = oracle.philox4x32_10_scalar((j & M32, j >> 32, 0, 0), (17, 9))
        assert r == (w[p & 3] & 0xFFFF) == oracle.random16_scalar(p, 17, 9)
