"""Shared plumbing for the GPU parity tests: upload seeded host arrays, land a
displaced buffer through the library's own scatter, read results back.
Nothing here computes any part of the method."""
from __future__ import annotations

import sys

import numpy as np

from patch_attention_cfg_amd import dfp


def torch_mod():
    import torch
    return torch


def require_gpu():
    import pytest
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    dfp.lib()  # raises loudly if libdfp.so is missing


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dtype_of(kind: str):
    torch = torch_mod()
    return torch.bfloat16 if kind == "bf16" else torch.float32


def up(a: np.ndarray, kind: str):
    """Host float32 (bf16-exact for bf16) -> device tensor of that dtype."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(dtype_of(kind)).contiguous()


def down(t) -> np.ndarray:
    return t.float().cpu().numpy()


def v_buffer_to_rows(v_buf_t, N: int) -> np.ndarray:
    """[B,H,d,ldv] device V buffer -> host [B,H,N,d] (layout only)."""
    return np.ascontiguousarray(np.swapaxes(down(v_buf_t)[..., :N], -1, -2))


def land_buffer(level, x, p: int, kind: str):
    """Device (k_buf, v_buf_t) holding the previous step's K/V everywhere,
    this step's K/V for patch p and for the text rows -- all landed with
    dfp_kv_scatter."""
    torch = torch_mod()
    B, H, N, d = level.B, level.H, level.N_kv, level.d
    k_buf, v_buf = dfp.alloc_kv_buffer(B, H, N, d, dtype_of(kind))
    dfp.kv_scatter(k_buf, v_buf, up(x.k_stale, kind), up(x.v_stale, kind), 0)
    kf, vf = x.fresh_rows(p)
    dfp.kv_scatter(k_buf, v_buf, up(kf, kind), up(vf, kind), level.row0(p))
    if level.n_text:
        kt, vt = x.text_rows()
        dfp.kv_scatter(k_buf, v_buf, up(kt, kind), up(vt, kind), 0)
    torch.cuda.synchronize()
    return k_buf, v_buf


def run_patch(level, x, p: int, kind: str | None = None, split_ok: bool = True):
    """Patch p's attention on the GPU.  With split_ok the call gets a
    workspace, so the library may split the key range (its default plan)."""
    kind = kind or level.dtype
    torch = torch_mod()
    k_buf, v_buf = land_buffer(level, x, p, kind)
    q = up(x.q_patch(p), kind)
    o = torch.empty_like(q)
    ws = (dfp.attention_workspace(level.B, level.H, level.n, level.N_kv, level.d)
          if split_ok else None)
    dfp.patch_attention(o, q, k_buf, v_buf, 1.0 / level.d ** 0.5, ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert_counters_zero(ws, level.B * level.H, level.n, level.d)
    return down(o)


def assert_counters_zero(ws, BH: int, n_q: int, d: int = 64) -> None:
    """The attention workspace starts with one uint32 arrival counter per
    query tile (128 rows at d=64, 256 at d=128); every call must leave them
    at zero."""
    block_m = 128 if d == 64 else 256
    n = BH * ((n_q + block_m - 1) // block_m) * 4
    assert int(ws[:n].sum().item()) == 0


def sample_rows(n: int, BH: int, block_m: int, total: int, seed: int):
    """(bh, row) pairs for every (batch, head): the first and last rows of
    the 32-, 64- and block_m-row tiles at both ends of the patch, every row
    of the last (possibly partial) block_m tile, plus seeded random rows
    spread over the (batch, head) slices until `total` random pairs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, block_m - 1, block_m,
             n - 1, n - 2, n - 33, n - 65, n - 129}
    tail0 = (n - 1) // block_m * block_m          # first row of the last tile
    fixed |= set(range(tail0, n))
    fixed |= {tail0 - 1, tail0 - 2}
    fixed = sorted(r for r in fixed if 0 <= r < n)
    extra_bh = rng.integers(0, BH, size=total)
    extra_row = rng.integers(0, n, size=total)
    pairs = {(bh, r) for bh in range(BH) for r in fixed}
    pairs |= {(int(b), int(r)) for b, r in zip(extra_bh, extra_row)}
    pairs = sorted(pairs)
    return (np.array([b for b, _ in pairs], dtype=np.int64),
            np.array([r for _, r in pairs], dtype=np.int64))


def block_m_of(level, with_workspace: bool = True) -> int:
    """Query rows per workgroup of the planner's launch for this level."""
    ks = dfp.attention_plan(level.B, level.H, level.n, level.N_kv, level.d, with_workspace)[0]
    return (128 if level.d == 64 else 256) // ks


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))
