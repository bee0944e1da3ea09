"""Pins of the oracle's Philox4x32-10 and of its element -> random-bits mapping.

Philox4x32-10 is defined by Salmon et al., "Parallel Random Numbers: As Easy
as 1, 2, 3" (SC'11).  The oracle's implementation is checked against two
independent ones:
* the definition written out here with Python integers (and, for a million
  counters, the same definition over numpy uint64 arrays);
* rocRAND's philox4x32_10 engine, whose header-only engine is host-callable.
  A tiny host program (built here with hipcc, host code only, no GPU call)
  prints the engine's outputs for chosen keys and counters; the engine's
  (seed, subsequence, offset) arguments map to key = seed and counter =
  (offset/4 as 64 bits, subsequence as 64 bits).
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

PROG = r"""
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>
int main() {
  unsigned long long cases[][3] = {
    {0ull, 0ull, 0ull}, {0ull, 0ull, 1ull}, {0ull, 1ull, 0ull}, {1ull, 0ull, 0ull},
    {0xdeadbeefcafef00dull, 123456789ull, 987654321ull},
    {0xffffffffffffffffull, 0xffffffffffffffffull, 0x3fffffffffffffffull},
    {42ull, 2047ull, 8388607ull}, {0x0123456789abcdefull, 1ull << 40, (1ull << 33) + 5ull},
  };
  for (auto& c : cases) {
    rocrand_device::philox4x32_10_engine eng(c[0], c[1], c[2] * 4ull);
    unsigned a = eng(), b = eng(), d = eng(), e = eng();
    std::printf("%llu %llu %llu %u %u %u %u\n", c[0], c[1], c[2], a, b, d, e);
  }
  return 0;
}
"""


def _rocrand_outputs():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc or rocRAND headers not available")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "kat.cpp")
        exe = os.path.join(d, "kat")
        with open(src, "w") as f:
            f.write(PROG)
        subprocess.run([hipcc, "-x", "c++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src,
                        "-o", exe], check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    rows = []
    for line in out.strip().splitlines():
        seed, sub, off, *w = (int(x) for x in line.split())
        rows.append((seed, sub, off, w))
    return rows


def test_philox_matches_rocrand_engine():
    rows = _rocrand_outputs()
    assert len(rows) == 8
    for seed, sub, grp, words in rows:
        key = (seed & 0xFFFFFFFF, seed >> 32)
        ctr = (grp & 0xFFFFFFFF, grp >> 32, sub & 0xFFFFFFFF, sub >> 32)
        assert oracle.philox(ctr, key) == words, (seed, sub, grp)


# The definition (SC'11, the Philox family): a round multiplies counter words
# 0 and 2 by the two multipliers; the new word 0 is the high half of the
# second product xored with word 1 and key word 0, the new word 2 the high
# half of the first product xored with word 3 and key word 1, and the low
# halves become words 1 and 3 (second product, then first).  The key is
# bumped by the two Weyl constants after each round; ten rounds.
_M = (0xD2511F53, 0xCD9E8D57)
_W = (0x9E3779B9, 0xBB67AE85)
_MASK = (1 << 32) - 1


def philox_int(ctr, key, rounds=10):
    x0, x1, x2, x3 = (int(c) & _MASK for c in ctr)
    k0, k1 = (int(k) & _MASK for k in key)
    for _ in range(rounds):
        p0, p1 = _M[0] * x0, _M[1] * x2
        x0, x1, x2, x3 = (p1 >> 32) ^ x1 ^ k0, p1 & _MASK, (p0 >> 32) ^ x3 ^ k1, p0 & _MASK
        k0, k1 = (k0 + _W[0]) & _MASK, (k1 + _W[1]) & _MASK
    return [x0, x1, x2, x3]


def philox_np(ctr, key, rounds=10):
    """The same over uint64 arrays (a 32 x 32-bit product fits exactly)."""
    x = [np.asarray(c, np.uint64) & np.uint64(_MASK) for c in ctr]
    k0 = np.asarray(key[0], np.uint64) & np.uint64(_MASK)
    k1 = np.asarray(key[1], np.uint64) & np.uint64(_MASK)
    m, s32 = np.uint64(_MASK), np.uint64(32)
    for _ in range(rounds):
        p0, p1 = np.uint64(_M[0]) * x[0], np.uint64(_M[1]) * x[2]
        x = [(p1 >> s32) ^ x[1] ^ k0, p1 & m, (p0 >> s32) ^ x[3] ^ k1, p0 & m]
        k0, k1 = (k0 + np.uint64(_W[0])) & m, (k1 + np.uint64(_W[1])) & m
    return x


def _counters(n, seed):
    """Counters and keys spanning every word: random, plus all-zero, all-one
    and single-bit words."""
    r = np.random.default_rng(seed)
    ctr = r.integers(0, 1 << 32, (n, 4), dtype=np.uint64)
    key = r.integers(0, 1 << 32, (n, 2), dtype=np.uint64)
    special = np.array([0, 1, _MASK, 1 << 31, 0x80000001], np.uint64)
    ctr[:200] = special[r.integers(0, special.size, (200, 4))]
    key[:200] = special[r.integers(0, special.size, (200, 2))]
    return ctr, key


def _oracle_many(ctr, key):
    import ctypes
    f = oracle.lib().orc_philox4x32_10
    c, k, o = (ctypes.c_uint32 * 4)(), (ctypes.c_uint32 * 2)(), (ctypes.c_uint32 * 4)()
    out = np.zeros(ctr.shape, np.uint64)
    for i in range(ctr.shape[0]):
        c[0], c[1], c[2], c[3] = (int(x) for x in ctr[i])
        k[0], k[1] = int(key[i, 0]), int(key[i, 1])
        f(c, k, o)
        out[i] = tuple(o)
    return out


def test_philox_matches_python_definition():
    ctr, key = _counters(20000, 1)
    got = _oracle_many(ctr, key)
    for i in range(ctr.shape[0]):
        assert list(got[i]) == philox_int(ctr[i], key[i]), (ctr[i], key[i])


def test_philox_matches_definition_on_a_million_counters():
    ctr, key = _counters(1_000_000, 2)
    got = _oracle_many(ctr, key)
    want = np.stack(philox_np(ctr.T, key.T), 1)
    assert np.array_equal(got, want)
    # and the two written-out forms agree with each other on a sample
    for i in range(0, 1_000_000, 50_000):
        assert list(want[i]) == philox_int(ctr[i], key[i])


def test_random_bits_mapping_16():
    """Element e takes half (e&1) of word (e>>1)&3 of block e>>3 (documented mapping)."""
    cfg = oracle.Cfg(seed=0x1234_5678_9ABC_DEF0, sr_bits=16)
    step = (7 << 32) | 99
    for e in [0, 1, 2, 3, 7, 8, 15, 16, 12345, (1 << 35) + 11]:
        g = e >> 3
        w = oracle.philox((g & 0xFFFFFFFF, g >> 32, step & 0xFFFFFFFF, step >> 32),
                          (cfg.seed & 0xFFFFFFFF, cfg.seed >> 32))[(e >> 1) & 3]
        expect = (w >> 16) if (e & 1) else (w & 0xFFFF)
        assert oracle.random_bits(cfg, e, step) == expect


def test_random_bits_mapping_8():
    cfg = oracle.Cfg(seed=5, sr_bits=8)
    for e in [0, 1, 2, 3, 4, 5, 15, 16, 17, 999]:
        g = e >> 4
        w = oracle.philox((g, 0, 3, 0), (5, 0))[(e >> 2) & 3]
        assert oracle.random_bits(cfg, e, 3) == (w >> (8 * (e & 3))) & 0xFF


def test_random_bits_uniform_and_step_dependent():
    """Counts over 2^16 elements are uniform at the chi-square level; other steps differ."""
    cfg = oracle.Cfg(seed=0, sr_bits=8)
    vals = np.array([oracle.random_bits(cfg, e, 0) for e in range(1 << 14)])
    counts = np.bincount(vals, minlength=256)
    expect = vals.size / 256
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert chi2 < 400  # 255 dof: mean 255, sd ~22.6
    other = np.array([oracle.random_bits(cfg, e, 1) for e in range(256)])
    assert (other != vals[:256]).mean() > 0.9
