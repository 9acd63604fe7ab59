"""Pins for the oracle's sampler-noise generator (CPU only).

The DDIM step with eta > 0 adds sigma * z with z ~ N(0, 1) ("AIGC 文生图系统
如何优化扩散模型推理速度", section 3).  The oracle draws z from Philox4x64-10
(Salmon et al., SC'11) and the Box-Muller transform.  The pins:
  * every Philox block equals numpy's independent Philox4x64-10 bit
    generator (numpy.random.Philox advances its counter before each block,
    so its block for counter c is produced from state counter c - 1);
  * inverting Box-Muller on the oracle's normals recovers exactly the
    32-bit halves of numpy's words, in the documented order;
  * the normals pass distribution tests (Kolmogorov-Smirnov against N(0,1),
    the pair radius against its exponential law, no pair correlation), and
    blocks depend only on their own counter.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle

MASK = 2**64 - 1


def _numpy_block(counter, key):
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    k = int(key[0]) | (int(key[1]) << 64)
    bg = np.random.Philox(key=k, counter=(c - 1) % 2**256)
    return bg.random_raw(4)


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((MASK, MASK, MASK, MASK), (MASK, MASK)),
    ((7, 3, 0, 0), (5, 1)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
])
def test_philox_block_matches_numpy(counter, key):
    np.testing.assert_array_equal(oracle.philox4x64_10(counter, key),
                                  _numpy_block(counter, key))


def test_philox_random_blocks_match_numpy():
    r = np.random.Generator(np.random.PCG64(11))
    for _ in range(200):
        counter = [int(x) for x in r.integers(0, 2**64, size=4, dtype=np.uint64)]
        key = [int(x) for x in r.integers(0, 2**64, size=2, dtype=np.uint64)]
        np.testing.assert_array_equal(oracle.philox4x64_10(counter, key),
                                      _numpy_block(counter, key))


@pytest.mark.parametrize("seed,step,image", [(0, 0, 0), (1234, 17, 1), (2**63 + 5, 49, 3)])
def test_box_muller_inverts_to_numpy_words(seed, step, image):
    n = 8 * 64
    z = oracle.philox_normals(n, seed, step, image).reshape(-1, 4, 2)
    for j in range(z.shape[0]):
        w = _numpy_block((j, image, 0, 0), (seed, step))
        for k in range(4):
            z0, z1 = z[j, k]
            u1 = math.exp(-(z0 * z0 + z1 * z1) / 2)
            u2 = (math.atan2(z1, z0) / (2 * math.pi)) % 1.0
            lo, hi = int(w[k]) & 0xFFFFFFFF, int(w[k]) >> 32
            # u = (h + 1/2) / 2^32; the round trip is exact to well under a unit of h
            # except where u1 is within rounding of 1 (radius ~ 0)
            assert abs(u1 * 2**32 - 0.5 - lo) < max(1e-3, 1e-9 * lo)
            if z0 * z0 + z1 * z1 > 1e-12:
                d = abs(u2 * 2**32 - 0.5 - hi)
                assert min(d, 2**32 - d) < 2e-3 * max(1.0, 1.0 / math.sqrt(z0 * z0 + z1 * z1))


def test_normals_distribution():
    z = oracle.philox_normals(1 << 20, 42, 3, 0)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    r2 = z[0::2] ** 2 + z[1::2] ** 2           # radius^2 of a Box-Muller pair ~ Exp(mean 2)
    assert stats.kstest(r2, "expon", args=(0, 2)).pvalue > 1e-3
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 5e-3
    assert abs(z.mean()) < 5e-3 and abs(z.var() - 1) < 5e-3


def test_blocks_depend_only_on_their_counter():
    a = oracle.philox_normals(8 * 10 + 3, 9, 2, 1)
    b = oracle.philox_normals(8 * 20, 9, 2, 1)
    np.testing.assert_array_equal(a, b[:a.size])
    # another step, image or seed is another stream
    for other in (oracle.philox_normals(80, 9, 3, 1), oracle.philox_normals(80, 9, 2, 0),
                  oracle.philox_normals(80, 10, 2, 1)):
        assert abs(np.corrcoef(other, b[:80])[0, 1]) < 0.5
        assert not np.array_equal(other, b[:80])
