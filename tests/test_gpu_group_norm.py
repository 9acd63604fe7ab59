"""GPU parity of dfp_displaced_group_norm (the corrected_async_gn mode) against
the fp64 oracle, through the C ABI.

Bars, derived from the kernel's arithmetic: the statistics are fp64, the
normalization fp32 -- y = (x - mean) * (rstd * gamma) + beta with mean and
rstd rounded to fp32 -- so each output carries a few fp32 roundings of an
O(1) value: max-abs error <= 1e-5 and relative L2 <= 1e-6.  The landed fresh
sums are fp64 sums in another order: relative 1e-10."""
import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import dfp, inputs
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-5
REL_L2 = 1e-6


def _run(B, C, G_, n, P, p, seed, affine=True, in_place=False, land=True, offset=0, ws=True):
    torch = G.torch_mod()
    a = inputs.group_norm_inputs(B, C, G_, n, P, p, seed)
    want_y, want_f = oracle.displaced_group_norm(a.x, a.stats, G_, p, 1e-5,
                                                 a.gamma if affine else None,
                                                 a.beta if affine else None)
    # offset > 0 places x (and y) off the 16-byte grid
    xs = torch.zeros(a.x.size + offset, dtype=torch.float32, device="cuda")
    xs[offset:] = torch.from_numpy(a.x.ravel()).cuda()
    x = xs[offset:].view(B, C, n)
    if in_place:
        y = x
    else:
        ys = torch.full((a.x.size + offset + 64,), float("nan"), device="cuda")
        y = ys[offset:offset + a.x.size].view(B, C, n)
    st = torch.from_numpy(a.stats).cuda()
    gamma = torch.from_numpy(a.gamma).cuda() if affine else None
    beta = torch.from_numpy(a.beta).cuda() if affine else None
    work = dfp.group_norm_workspace(B, C, G_, n) if ws else None
    if work is not None:
        work.fill_(0x7F)   # the chunked path needs no initial workspace contents
    dfp.displaced_group_norm(y, x, st, G_, p, 1e-5, gamma, beta, land, work)
    torch.cuda.synchronize()
    got = G.down(y).astype(np.float64)
    err = np.abs(got - want_y)
    rel = np.linalg.norm(got - want_y) / np.linalg.norm(want_y)
    assert err.max() <= MAX_ABS and rel <= REL_L2, (err.max(), rel)
    got_st = st.cpu().numpy()
    others = [q for q in range(P) if q != p]
    np.testing.assert_array_equal(got_st[:, :, others], a.stats[:, :, others])
    if land:
        np.testing.assert_allclose(got_st[:, :, p], want_f, rtol=1e-10, atol=1e-9)
    else:
        assert np.isnan(got_st[:, :, p]).all()
    if not in_place:
        assert torch.isnan(ys[offset + a.x.size:]).all()   # nothing past y written
    return got, got_st


@pytest.mark.parametrize("B,C,G_,n,P,p", [
    (2, 320, 32, 4096, 4, 1),     # SDXL-1024 first level: 128x128, 32-row patches
    (2, 640, 32, 1024, 4, 2),     # 64x64 level
    (2, 1280, 32, 256, 4, 3),     # 32x32 level
    (1, 64, 2, 4096, 8, 0),       # a group of 128 Ki floats: chunked, or streamed twice
    (2, 320, 32, 28800, 8, 3),    # SDXL-3840 first level: 480x480, 60-row patches
    (3, 12, 3, 1001, 5, 4),       # n not a multiple of 4: scalar path
    (3, 12, 3, 30001, 5, 4),      # ... with groups of 117 Ki floats
    (1, 8, 8, 4, 1, 0),           # one channel per group, one patch
    (1, 512, 1, 64, 2, 0),        # in registers, 512 channels: gamma/beta read from memory
    (1, 32768, 1, 4, 1, 0),       # chunks spanning 1024 channels each
    (1, 16, 1, 600001, 2, 1),     # x over 32 MiB, n odd: scalar chunks, launch 2 last chunk first
    (2, 64, 8, 256, 64, 63),      # 64 patches: every stale sum staged in LDS
    (2, 64, 8, 256, 65, 0),       # 65 patches: stale sums read after the reduction
    (1, 64, 2, 4096, 100, 57),    # chunked, 100 patches
])
@pytest.mark.parametrize("ws", [True, False])
def test_every_element(B, C, G_, n, P, p, ws):
    G.require_gpu()
    G.announce(f"group norm B{B} C{C} G{G_} n{n} P{P} p{p} workspace={ws}")
    _run(B, C, G_, n, P, p, seed=C + n + p, ws=ws)


@pytest.mark.parametrize("n", [1024, 16384])
def test_no_affine_in_place_no_landing(n):
    G.require_gpu()
    G.announce(f"group norm no affine, in place, no landing, n{n}")
    _run(2, 640, 32, n, 4, 0, seed=3, affine=False, in_place=True, land=False)


@pytest.mark.parametrize("n", [256, 8192])
def test_unaligned_takes_the_scalar_path(n):
    G.require_gpu()
    G.announce(f"group norm x and y off the 16-byte grid, n{n}")
    _run(2, 320, 32, n, 4, 1, seed=9, offset=1)


@pytest.mark.parametrize("n", [4096, 28800])
def test_bitwise_repeatable(n):
    G.require_gpu()
    G.announce(f"group norm bitwise repeatable n{n}")
    y1, s1 = _run(2, 320, 32, n, 4, 1, seed=21)
    y2, s2 = _run(2, 320, 32, n, 4, 1, seed=21)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(s1, s2)


def test_landed_sums_feed_the_next_step():
    """Two sweeps over the patches, each landing its sums, activations
    unchanged: in the second sweep every patch sees only current statistics,
    so the reassembled output is plain GroupNorm over the whole image (torch
    float64 on the CPU)."""
    import torch
    G.require_gpu()
    G.announce("group norm patch sweep")
    B, C, G_, n, P = 2, 64, 8, 512, 4
    a = inputs.group_norm_inputs(B, C, G_, P * n, 1, 0, seed=33)
    full = a.x
    st = torch.zeros((B, G_, P, 2), dtype=torch.float64, device="cuda")
    outs = []
    for sweep in range(2):
        outs = []
        for q in range(P):
            x = torch.from_numpy(np.ascontiguousarray(full[:, :, q * n:(q + 1) * n])).cuda()
            y = torch.empty_like(x)
            dfp.displaced_group_norm(y, x, st, G_, q, 1e-5, None, None, True,
                                     dfp.group_norm_workspace(B, C, G_, n))
            outs.append(G.down(y))
        torch.cuda.synchronize()
    want = torch.nn.functional.group_norm(torch.from_numpy(full.astype(np.float64)), G_,
                                          eps=1e-5).numpy()
    got = np.concatenate(outs, axis=-1)
    assert np.abs(got - want).max() <= MAX_ABS


def _random_case(i):
    rng = np.random.Generator(np.random.PCG64(7000 + i))
    G_ = int(rng.choice([1, 2, 4, 8, 32]))
    C = G_ * int(rng.integers(1, 9))
    n = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(1000, 40000))]))
    B = int(rng.integers(1, 4))
    P = int(rng.integers(1, 9))
    return dict(B=B, C=C, G_=G_, n=n, P=P, p=int(rng.integers(0, P)),
                affine=bool(rng.integers(0, 2)), in_place=bool(rng.integers(0, 4) == 0),
                land=bool(rng.integers(0, 4) != 0), offset=int(rng.choice([0, 0, 0, 1, 3])),
                ws=bool(rng.integers(0, 4) != 0))


@pytest.mark.parametrize("i", range(32))
def test_random_shape(i):
    """Seeded draws across the register, chunked and single-workgroup paths:
    group runs from a few floats to over 300 Ki, n with and without a
    multiple of 4, x and y on and off the 16-byte grid, in place, with and
    without gamma/beta, landing and workspace."""
    c = _random_case(i)
    G.require_gpu()
    G.announce(f"group norm random case {i}: {c}")
    kw = dict(c)
    B, C, G_, n, P, p = (kw.pop(k) for k in ("B", "C", "G_", "n", "P", "p"))
    _run(B, C, G_, n, P, p, seed=7100 + i, **kw)
