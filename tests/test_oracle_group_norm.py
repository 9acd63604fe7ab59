"""Pins of the oracle's displaced GroupNorm (the corrected_async_gn mode on the
DistriFusion tutorial page, given there by name only; the reading is in the
oracle's header): each check compares it with something other than itself --
PyTorch's GroupNorm on the CPU in float64, numpy reductions, a hand-worked
case and invariants."""
import numpy as np
import pytest
import torch

import oracle


def _full_image_case(seed, B=2, C=12, G=3, n=10, P=4):
    rng = np.random.default_rng(seed)
    full = rng.standard_normal((B, C, P * n)) * 2.0 + 0.5
    # every patch's sums over the current activations: stale == fresh
    stats = np.empty((B, G, P, 2))
    cg = C // G
    for q in range(P):
        part = full[:, :, q * n:(q + 1) * n].reshape(B, G, cg * n)
        stats[:, :, q, 0] = part.sum(-1)
        stats[:, :, q, 1] = (part * part).sum(-1)
    return full, stats


@pytest.mark.parametrize("p", [0, 2, 3])
def test_all_fresh_is_groupnorm_of_the_full_image(p):
    """With every patch's sums current, the patch's output is its slice of
    plain GroupNorm over the whole image (torch.nn.functional.group_norm,
    float64, biased variance)."""
    B, C, G, n, P = 2, 12, 3, 10, 4
    full, stats = _full_image_case(7 + p, B, C, G, n, P)
    rng = np.random.default_rng(1)
    gamma, beta = rng.standard_normal(C), rng.standard_normal(C)
    want = torch.nn.functional.group_norm(torch.from_numpy(full), G, torch.from_numpy(gamma),
                                          torch.from_numpy(beta), eps=1e-5).numpy()
    y, _ = oracle.displaced_group_norm(full[:, :, p * n:(p + 1) * n], stats, G, p, 1e-5,
                                       gamma, beta)
    np.testing.assert_allclose(y, want[:, :, p * n:(p + 1) * n], rtol=1e-12, atol=1e-12)


def test_one_patch_is_plain_groupnorm():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 8, 33)) * 3.0 - 1.0
    want = torch.nn.functional.group_norm(torch.from_numpy(x), 4, eps=1e-6).numpy()
    y, _ = oracle.displaced_group_norm(x, np.full((3, 4, 1, 2), np.nan), 4, 0, 1e-6)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_the_local_stale_sums_are_replaced():
    """The correction: this patch's own stale sums never enter."""
    full, stats = _full_image_case(11)
    n, p = 10, 1
    x = full[:, :, p * n:(p + 1) * n]
    y1, f1 = oracle.displaced_group_norm(x, stats, 3, p, 1e-5)
    bad = stats.copy()
    bad[:, :, p, :] = [1e6, -3.0]
    y2, f2 = oracle.displaced_group_norm(x, bad, 3, p, 1e-5)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(f1, f2)


def test_fresh_sums_are_the_group_sums():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 6, 7))
    _, f = oracle.displaced_group_norm(x, np.zeros((2, 3, 2, 2)), 3, 0, 1e-5)
    grp = x.reshape(2, 3, 14)
    np.testing.assert_allclose(f[..., 0], grp.sum(-1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(f[..., 1], (grp * grp).sum(-1), rtol=1e-13)


def test_hand_worked_case():
    """One group of 2 channels x 2 positions, two patches: x = [[1, 3], [5, 7]]
    in patch 1, the other patch's sums (4, 10).  S1 = 16 + 4 = 20,
    S2 = 84 + 10 = 94, N = 8, mean = 5/2, var = 94/8 - 25/4 = 11/2."""
    x = np.array([[[1.0, 3.0], [5.0, 7.0]]])
    stats = np.array([[[[4.0, 10.0], [123.0, 456.0]]]])
    y, f = oracle.displaced_group_norm(x, stats, 1, 1, 0.0)
    np.testing.assert_allclose(y, (x - 2.5) / np.sqrt(5.5), rtol=1e-15)
    np.testing.assert_array_equal(f, [[[16.0, 84.0]]])


def test_whole_image_statistics_and_affine():
    """All patches normalized with current statistics: every group of the
    reassembled image has mean 0 and variance var/(var + eps); gamma, beta
    act per channel."""
    B, C, G, n, P = 2, 12, 3, 10, 4
    full, stats = _full_image_case(13, B, C, G, n, P)
    eps = 1e-3
    ys = [oracle.displaced_group_norm(full[:, :, q * n:(q + 1) * n], stats, G, q, eps)[0]
          for q in range(P)]
    img = np.concatenate(ys, axis=-1).reshape(B, G, -1)
    var = full.reshape(B, G, -1).var(-1)
    np.testing.assert_allclose(img.mean(-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(img.var(-1), var / (var + eps), rtol=1e-12)
    gamma = np.linspace(-2.0, 2.0, C)
    beta = np.linspace(1.0, 3.0, C)
    y_aff, _ = oracle.displaced_group_norm(full[:, :, :n], stats, G, 0, eps, gamma, beta)
    np.testing.assert_allclose(y_aff, ys[0] * gamma[None, :, None] + beta[None, :, None],
                               rtol=1e-12, atol=1e-12)


def test_stale_sums_shift_the_statistics():
    """Changing another patch's stale sum by d moves the mean by d / N."""
    full, stats = _full_image_case(17)
    n, p, N = 10, 0, 4 * 10 * 4
    x = full[:, :, :n]
    y1, _ = oracle.displaced_group_norm(x, stats, 3, p, 0.0)
    s2 = stats.copy()
    s2[:, :, 2, 0] += 8.0      # sum only: mean up by 8/N, E[x^2] unchanged
    y2, _ = oracle.displaced_group_norm(x, s2, 3, p, 0.0)
    grp = full.reshape(2, 3, -1)
    m1 = grp.mean(-1)
    m2 = m1 + 8.0 / N
    v2 = (grp * grp).mean(-1) - m2 * m2
    want = (x.reshape(2, 3, 4 * n) - m2[..., None]) / np.sqrt(v2[..., None])
    np.testing.assert_allclose(y2.reshape(2, 3, -1), want, rtol=1e-11, atol=1e-11)
    assert not np.allclose(y1, y2)
