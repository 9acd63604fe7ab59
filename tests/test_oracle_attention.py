"""Pins for the oracle's displaced patch attention (CPU only).

Every check here comes from something other than the oracle's own formula:
an independent numpy formulation (explicit probability matrix), closed forms
(two keys -> logistic weights; hard-attention and zero-scale limits),
invariants (rows sum to 1, key/value permutation), and the special cases the
DistriFusion page's synchronous warm-up implies (stale == fresh, or a single
patch, gives plain full attention).
"""
import math

import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import inputs


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _numpy_attention(q, k, v, scale):
    """Independent formulation: build the whole probability matrix with
    numpy broadcasting and multiply it into V."""
    s = np.einsum("...id,...jd->...ij", q, k) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v


def test_brute_force_matches_numpy():
    r = _rng(1)
    q = r.standard_normal((2, 3, 5, 8))
    k = r.standard_normal((2, 3, 11, 8))
    v = r.standard_normal((2, 3, 11, 8))
    o = oracle.attention(q, k, v, 1 / math.sqrt(8))
    np.testing.assert_allclose(o, _numpy_attention(q, k, v, 1 / math.sqrt(8)),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("N,d", [(1, 4), (7, 3), (64, 64), (200, 16)])
def test_brute_force_shapes(N, d):
    r = _rng(N * 100 + d)
    q = r.standard_normal((1, 2, 9, d)) * 2
    k = r.standard_normal((1, 2, N, d))
    v = r.standard_normal((1, 2, N, d))
    o = oracle.attention(q, k, v, 0.3)
    np.testing.assert_allclose(o, _numpy_attention(q, k, v, 0.3), rtol=0, atol=1e-12)


def test_two_keys_logistic_closed_form():
    # With two keys the weights are the logistic function of the score gap.
    q = np.array([[[[1.0, 2.0]]]])
    k = np.array([[[[0.5, -1.0], [2.0, 0.25]]]])
    v = np.array([[[[1.0, 10.0], [-3.0, 4.0]]]])
    scale = 0.7
    s0 = scale * (1.0 * 0.5 + 2.0 * -1.0)
    s1 = scale * (1.0 * 2.0 + 2.0 * 0.25)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    expect = w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1]
    np.testing.assert_allclose(oracle.attention(q, k, v, scale)[0, 0, 0], expect,
                               rtol=0, atol=1e-15)


def _numpy_probs(q, k, scale):
    """The probability matrix of _numpy_attention, on its own."""
    s = np.einsum("...id,...jd->...ij", q, k) * scale
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    return p / p.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("shape,scale", [((2, 2, 6, 16, 33), 0.25), ((1, 3, 4, 8, 1), 1.0),
                                         ((1, 1, 9, 5, 70), 3.0)])
def test_probability_matrix_matches_numpy(shape, scale):
    B, H, nq, d, N = shape
    r = _rng(nq * 31 + N)
    q = r.standard_normal((B, H, nq, d))
    k = r.standard_normal((B, H, N, d))
    np.testing.assert_allclose(oracle.attention_probs(q, k, scale), _numpy_probs(q, k, scale),
                               rtol=1e-13, atol=1e-15)


def test_probability_matrix_two_keys_and_order():
    # two keys: logistic weights of the score gap, in key order
    q = np.array([[[[1.0, 2.0], [0.0, 0.0]]]])
    k = np.array([[[[0.5, -1.0], [2.0, 0.25]]]])
    p = oracle.attention_probs(q, k, 0.7)
    s0, s1 = 0.7 * (0.5 - 2.0), 0.7 * (2.0 + 0.5)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(p[0, 0, 0], [w0, 1 - w0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(p[0, 0, 1], [0.5, 0.5], rtol=0, atol=0)   # q = 0: uniform


def test_probability_rows_sum_to_one():
    r = _rng(3)
    q = r.standard_normal((2, 2, 6, 16)) * 3
    k = r.standard_normal((2, 2, 33, 16))
    p = oracle.attention_probs(q, k, 0.25)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)


def test_constant_values_give_constant_output():
    r = _rng(4)
    q = r.standard_normal((1, 2, 5, 8))
    k = r.standard_normal((1, 2, 17, 8))
    c = r.standard_normal(8)
    v = np.broadcast_to(c, (1, 2, 17, 8)).copy()
    np.testing.assert_allclose(oracle.attention(q, k, v, 0.5),
                               np.broadcast_to(c, (1, 2, 5, 8)), rtol=0, atol=1e-14)
    ones = np.ones((1, 2, 17, 8))
    np.testing.assert_allclose(oracle.attention(q, k, ones, 0.5), 1.0, rtol=0, atol=1e-14)


def test_zero_query_or_equal_keys_give_mean_of_values():
    r = _rng(5)
    k = r.standard_normal((1, 1, 13, 8))
    v = r.standard_normal((1, 1, 13, 8))
    mean = v.mean(axis=-2)
    o = oracle.attention(np.zeros((1, 1, 3, 8)), k, v, 1.0)
    np.testing.assert_allclose(o, np.broadcast_to(mean[:, :, None], o.shape), atol=1e-14)
    keq = np.broadcast_to(k[:, :, :1], k.shape).copy()
    o2 = oracle.attention(r.standard_normal((1, 1, 3, 8)), keq, v, 1.0)
    np.testing.assert_allclose(o2, np.broadcast_to(mean[:, :, None], o2.shape), atol=1e-14)
    o3 = oracle.attention(r.standard_normal((1, 1, 3, 8)), k, v, 0.0)
    np.testing.assert_allclose(o3, np.broadcast_to(mean[:, :, None], o3.shape), atol=1e-14)


def test_single_key_returns_its_value():
    r = _rng(6)
    v = r.standard_normal((2, 2, 1, 8))
    o = oracle.attention(r.standard_normal((2, 2, 4, 8)), r.standard_normal((2, 2, 1, 8)), v, 0.125)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=0, atol=0)


def test_hard_attention_limit_picks_argmax_key():
    # A huge scale makes softmax a one-hot at the best-scoring key; a sign
    # error in the scores or the max shift would pick the worst key instead.
    r = _rng(7)
    q = r.standard_normal((1, 1, 6, 4))
    k = r.standard_normal((1, 1, 9, 4))
    v = r.standard_normal((1, 1, 9, 4))
    o = oracle.attention(q, k, v, 1e4)
    best = np.argmax(q[0, 0] @ k[0, 0].T, axis=-1)
    np.testing.assert_allclose(o[0, 0], v[0, 0, best], rtol=0, atol=1e-12)


def test_permuting_keys_with_values_changes_nothing():
    r = _rng(8)
    q = r.standard_normal((1, 2, 4, 8))
    k = r.standard_normal((1, 2, 21, 8))
    v = r.standard_normal((1, 2, 21, 8))
    perm = r.permutation(21)
    np.testing.assert_allclose(oracle.attention(q, k, v, 0.4),
                               oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.4),
                               rtol=0, atol=1e-14)


def test_effective_kv_rows():
    stale = np.arange(2 * 10 * 3, dtype=np.float64).reshape(2, 10, 3)
    fresh = -1.0 - np.arange(2 * 4 * 3, dtype=np.float64).reshape(2, 4, 3)
    eff = oracle.effective_kv(stale, fresh, 5)
    np.testing.assert_array_equal(eff[:, :5], stale[:, :5])
    np.testing.assert_array_equal(eff[:, 5:9], fresh)
    np.testing.assert_array_equal(eff[:, 9:], stale[:, 9:])
    with pytest.raises(ValueError):
        oracle.effective_kv(stale, fresh, 7)


def _small_level_inputs(P, n_text=0, seed=11):
    lv = inputs.AttnLevel(name="t", B=2, H=2, N_img=48, P=P, d=8, n_text=n_text,
                          dtype="f32", seed=seed)
    return lv, inputs.attention_inputs(lv)


def test_displaced_patch_uses_stale_outside_and_fresh_inside():
    lv, x = _small_level_inputs(P=4)
    p = 2
    r0, n = lv.row0(p), lv.n
    kf, vf = x.fresh_rows(p)
    o = oracle.patch_attention(x.q_patch(p), x.k_stale, x.v_stale, kf, vf, r0, 0.3)
    k_eff = np.concatenate([x.k_stale[:, :, :r0], kf, x.k_stale[:, :, r0 + n:]], axis=2)
    v_eff = np.concatenate([x.v_stale[:, :, :r0], vf, x.v_stale[:, :, r0 + n:]], axis=2)
    np.testing.assert_allclose(o, _numpy_attention(x.q_patch(p).astype(np.float64),
                                                   k_eff.astype(np.float64),
                                                   v_eff.astype(np.float64), 0.3),
                               rtol=0, atol=1e-13)
    # and the stale rows really matter: all-fresh attention is different
    full = oracle.attention(x.q_patch(p), x.k_fresh, x.v_fresh, 0.3)
    assert np.abs(full - o).max() > 1e-4


def test_single_patch_is_full_attention():
    lv, x = _small_level_inputs(P=1)
    kf, vf = x.fresh_rows(0)
    o = oracle.patch_attention(x.q_patch(0), x.k_stale, x.v_stale, kf, vf, 0, 0.35)
    np.testing.assert_allclose(o, oracle.attention(x.q, x.k_fresh, x.v_fresh, 0.35),
                               rtol=0, atol=0)


@pytest.mark.parametrize("n_text", [0, 5])
def test_stale_equal_fresh_tiles_full_attention(n_text):
    # The synchronous warm-up case: every region is fresh, so each patch's
    # output is its rows of full attention, and the patches tile it.
    lv, x = _small_level_inputs(P=3, n_text=n_text)
    full = oracle.attention(x.q, x.k_fresh, x.v_fresh, 0.3)
    outs = []
    for p in range(lv.P):
        kf, vf = x.fresh_rows(p)
        extra = [(x.text_rows()[0], x.text_rows()[1], 0)] if n_text else []
        outs.append(oracle.patch_attention(x.q_patch(p), x.k_fresh, x.v_fresh, kf, vf,
                                           lv.row0(p), 0.3, extra))
    np.testing.assert_allclose(np.concatenate(outs, axis=2), full, rtol=0, atol=1e-15)


def test_text_rows_are_fresh():
    lv, x = _small_level_inputs(P=3, n_text=5)
    p = 1
    kf, vf = x.fresh_rows(p)
    kt, vt = x.text_rows()
    o = oracle.patch_attention(x.q_patch(p), x.k_stale, x.v_stale, kf, vf, lv.row0(p), 0.3,
                               [(kt, vt, 0)])
    r0, n = lv.row0(p), lv.n
    k_eff = x.k_stale.astype(np.float64).copy()
    v_eff = x.v_stale.astype(np.float64).copy()
    k_eff[:, :, :5] = kt
    v_eff[:, :, :5] = vt
    k_eff[:, :, r0:r0 + n] = kf
    v_eff[:, :, r0:r0 + n] = vf
    np.testing.assert_allclose(o, _numpy_attention(x.q_patch(p).astype(np.float64), k_eff,
                                                   v_eff, 0.3), rtol=0, atol=1e-13)


def test_rows_subset_matches_full():
    r = _rng(12)
    q = r.standard_normal((2, 3, 10, 8))
    k = r.standard_normal((2, 3, 15, 8))
    v = r.standard_normal((2, 3, 15, 8))
    full = oracle.attention(q, k, v, 0.5).reshape(6, 10, 8)
    bh = np.array([0, 5, 3, 3])
    ii = np.array([9, 0, 4, 9])
    np.testing.assert_array_equal(oracle.attention_rows(q, k, v, 0.5, bh, ii), full[bh, ii])
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v, 0.5, [6], [0])


# ---------------------------------------------------------------- patch sweep
def _sweep_case(seed, B=1, H=2, N_img=48, P=4, d=8, n_text=0):
    rng = np.random.default_rng(seed)
    N = n_text + N_img
    q = rng.standard_normal((B, H, N_img, d))
    kf, vf = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    ks, vs = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    return q, kf, vf, ks, vs


@pytest.mark.parametrize("n_text", [0, 5])
def test_sweep_last_patch_is_full_fresh_attention(n_text):
    q, kf, vf, ks, vs = _sweep_case(11, n_text=n_text)
    outs = oracle.patch_sweep(q, ks, vs, kf, vf, 4, 0.3, n_text)
    full = oracle.attention(q, kf, vf, 0.3)
    np.testing.assert_allclose(outs[-1], full[..., 36:48, :], rtol=0, atol=1e-13)


def test_sweep_first_patch_is_displaced_patch_attention():
    q, kf, vf, ks, vs = _sweep_case(12)
    outs = oracle.patch_sweep(q, ks, vs, kf, vf, 4, 0.3)
    want = oracle.patch_attention(q[..., :12, :], ks, vs, kf[..., :12, :], vf[..., :12, :], 0, 0.3)
    np.testing.assert_array_equal(outs[0], want)


def test_sweep_reads_fresh_up_to_its_patch_and_stale_after():
    """Patch m's output ignores the stale rows of patches <= m and the fresh
    rows of patches > m (perturbing either changes nothing), and does move
    when a fresh row of patch m or a stale row after it changes."""
    q, kf, vf, ks, vs = _sweep_case(13)
    base = oracle.patch_sweep(q, ks, vs, kf, vf, 4, 0.3)
    m, n = 1, 12
    ks2, vs2 = ks.copy(), vs.copy()
    ks2[..., :(m + 1) * n, :] += 3.0
    vs2[..., :(m + 1) * n, :] -= 2.0
    kf2, vf2 = kf.copy(), vf.copy()
    kf2[..., (m + 1) * n:, :] += 3.0
    vf2[..., (m + 1) * n:, :] -= 2.0
    np.testing.assert_array_equal(oracle.patch_sweep(q, ks2, vs2, kf2, vf2, 4, 0.3)[m], base[m])
    vf3 = vf.copy()
    vf3[..., m * n, :] += 1.0
    assert np.abs(oracle.patch_sweep(q, ks, vs, kf, vf3, 4, 0.3)[m] - base[m]).max() > 1e-6
    vs3 = vs.copy()
    vs3[..., (m + 1) * n, :] += 1.0
    assert np.abs(oracle.patch_sweep(q, ks, vs3, kf, vf, 4, 0.3)[m] - base[m]).max() > 1e-6


def test_sweep_with_stale_equal_fresh_is_full_attention():
    q, kf, vf, _, _ = _sweep_case(14, n_text=3)
    outs = oracle.patch_sweep(q, kf, vf, kf, vf, 4, 0.3, 3)
    full = oracle.attention(q, kf, vf, 0.3)
    np.testing.assert_allclose(np.concatenate(outs, axis=-2), full, rtol=0, atol=1e-13)
