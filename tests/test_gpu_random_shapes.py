"""Seeded random shapes through every launch path of the bf16 attention:
head size 64/128, one or two key groups, split key ranges, zero to two
fresh ranges with and without landing, ragged queries and keys.  Every
element against the oracle over the effective K/V (bf16 bars), the fused
call bitwise equal to scatter + attention, the landed buffer exact, and the
workspace counters back at zero.  A second set forces every split count
from 2 to 8 at both head sizes over key ranges up to 5000 rows.  The draws
are fixed by the seed, so the cases are the same on every run."""
import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import dfp, inputs
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS = 2e-2


def _case(i):
    rng = np.random.Generator(np.random.PCG64(9000 + i))
    d = int(rng.choice([64, 64, 128]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    n_q = int(rng.integers(1, 400))
    N = int(rng.integers(64, 2200))
    ranges = _fresh_ranges(rng, N)
    ks = str(rng.choice(["auto", "1", "2"])) if d == 64 else "auto"
    splits = int(rng.choice([0, 0, 2, 3, 5]))
    land = bool(rng.integers(0, 2))
    return B, H, n_q, N, d, ranges, ks, splits, land


def _fresh_ranges(rng, N):
    """Zero to two disjoint fresh ranges of whole 64-row tiles."""
    ntiles_whole = N // 64
    ranges = []
    for _ in range(int(rng.integers(0, 3))):
        if ntiles_whole < 1:
            break
        t0 = int(rng.integers(0, ntiles_whole))
        nt = int(rng.integers(1, min(8, ntiles_whole - t0) + 1))
        if all(t0 + nt <= a // 64 or t0 >= (a + n) // 64 for a, n in ranges):
            ranges.append((t0 * 64, nt * 64))
    return ranges


def _split_case(i):
    """Every split count from 2 to 8 at both head sizes, longer key ranges."""
    rng = np.random.Generator(np.random.PCG64(31000 + i))
    d = int(rng.choice([64, 128]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    n_q = int(rng.integers(1, 700))
    N = int(rng.integers(64, 5000))
    ranges = _fresh_ranges(rng, N)
    splits = int(rng.integers(2, 9))
    land = bool(rng.integers(0, 2))
    return B, H, n_q, N, d, ranges, "auto", splits, land


@pytest.mark.parametrize("i", range(64))
def test_random_shape(monkeypatch, i):
    _run_case(monkeypatch, i, _case(i))


@pytest.mark.parametrize("i", range(96))
def test_random_split(monkeypatch, i):
    _run_case(monkeypatch, i, _split_case(i))


def _run_case(monkeypatch, i, case):
    B, H, n_q, N, d, ranges, ks, splits, land = case
    G.require_gpu()
    G.announce(f"random attention case {i}: B{B} H{H} nq{n_q} N{N} d{d} ranges={ranges} "
               f"ks={ks} splits={splits} land={land}")
    if ks != "auto":
        monkeypatch.setenv("DFP_ATTN_KS", ks)
    if splits:
        monkeypatch.setenv("DFP_ATTN_SPLITS", str(splits))
    torch = G.torch_mod()
    seed = 9100 + i
    q, k_st, v_st = inputs.random_attention_arrays(B, H, n_q, N, d, seed=seed)
    k_buf, v_buf = dfp.alloc_kv_buffer(B, H, N, d, torch.bfloat16)
    v_buf.fill_(float("nan"))   # padding columns past N must never reach a result
    dfp.kv_scatter(k_buf, v_buf, G.up(k_st, "bf16"), G.up(v_st, "bf16"), 0)
    k_eff, v_eff = k_st.copy(), v_st.copy()
    fresh = []
    for j, (row0, n) in enumerate(ranges):
        _, k_new, v_new = inputs.random_attention_arrays(B, H, 1, n, d, seed=seed + 50 + j)
        fresh.append((G.up(k_new, "bf16"), G.up(np.swapaxes(v_new, -1, -2), "bf16"), row0))
        k_eff[:, :, row0:row0 + n], v_eff[:, :, row0:row0 + n] = k_new, v_new
    qd = G.up(q, "bf16")
    ws = dfp.attention_workspace(B, H, n_q, N, d)
    want = oracle.attention(q, k_eff, v_eff, 1.0 / d ** 0.5)

    o = torch.empty_like(qd)
    if fresh:
        dfp.patch_attention_fresh(o, qd, k_buf, v_buf, fresh, land, None, ws)
    else:
        dfp.patch_attention(o, qd, k_buf, v_buf, None, ws)
    torch.cuda.synchronize()
    got = G.down(o).astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    err = np.abs(got - want).max()
    assert rel <= REL_L2 and err <= MAX_ABS, (rel, err)
    if ws is not None:
        G.assert_counters_zero(ws, B * H, n_q, d)
    if fresh:
        if land:
            np.testing.assert_array_equal(G.down(k_buf), k_eff)
            np.testing.assert_array_equal(G.v_buffer_to_rows(v_buf, N), v_eff)
        # scatter + plain attention over the landed buffer gives the same bits
        k2, v2 = dfp.alloc_kv_buffer(B, H, N, d, torch.bfloat16)
        dfp.kv_scatter(k2, v2, G.up(k_eff, "bf16"), G.up(v_eff, "bf16"), 0)
        o2 = torch.empty_like(qd)
        dfp.patch_attention(o2, qd, k2, v2, None, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.down(o2), G.down(o))
