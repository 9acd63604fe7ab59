"""The largest key range the bf16 attention takes: one (batch, head) whose K
is just under 2 GiB (the kernels address one head's K and V^T with 32-bit
byte offsets).  K and V are zero except a few planted rows spread up to the
last row, whose keys score far above the zero keys, so the expected output
has a closed form over the planted rows alone (the 16.7 M zero keys still
enter the denominator).  The first tile of every key range scores 0, so the
kernel also takes the path that raises its reference max mid-range."""
import numpy as np
import pytest

from patch_attention_cfg_amd import dfp
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS = 2e-2
N_Q = 64


def _bf16(a):
    """Round fp64/fp32 values to bf16 (nearest even) and back to fp64."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _case(d, N):
    rng = np.random.Generator(np.random.PCG64(4242 + d))
    q = _bf16(1.0 + 0.1 * rng.standard_normal((N_Q, d)))
    rows = [12345, N // 2 + 7, N - 64, N - 1]
    # exact in bf16; close enough that every planted row carries weight
    k_rows = np.stack([np.full(d, 4.0 + t / 32) for t in range(len(rows))])
    v_rows = rng.choice([-1.0, 1.0], size=(len(rows), d))
    return q, rows, k_rows, v_rows


def _expected(q, k_rows, v_rows, N, d):
    """softmax over the planted keys plus N - len(rows) keys of score 0."""
    z = (q @ k_rows.T) / np.sqrt(d)                          # [N_Q, rows]
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    den = w.sum(axis=1, keepdims=True) + (N - len(k_rows)) * np.exp(-m)
    return (w @ v_rows) / den


def _buffers(d, N, rows, k_rows, v_rows, torch):
    k_buf, v_buf = dfp.alloc_kv_buffer(1, 1, N, d, torch.bfloat16)
    k_buf.zero_()
    v_buf.zero_()
    for j, kr, vr in zip(rows, k_rows, v_rows):
        k_buf[0, 0, j, :] = torch.tensor(kr, dtype=torch.bfloat16)
        v_buf[0, 0, :, j] = torch.tensor(vr, dtype=torch.bfloat16)
    return k_buf, v_buf


def _check(got, want, what):
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    err = np.abs(got - want).max()
    assert np.isfinite(got).all(), what
    assert rel <= REL_L2 and err <= MAX_ABS, (what, rel, err)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("d,N", [(64, (1 << 24) - 64), (128, (1 << 23) - 64)])
def test_largest_key_range(d, N, split):
    G.require_gpu()
    torch = G.torch_mod()
    assert N * d * 2 < (1 << 31) and d * dfp.v_ld(N, dfp.BF16) * 2 < (1 << 31)
    G.announce(f"largest key range d{d} N{N} split={split}")
    q, rows, k_rows, v_rows = _case(d, N)
    k_buf, v_buf = _buffers(d, N, rows, k_rows, v_rows, torch)
    qd = torch.tensor(q.reshape(1, 1, N_Q, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(qd)
    ws = dfp.attention_workspace(1, 1, N_Q, N, d) if split else None
    dfp.patch_attention(o, qd, k_buf, v_buf, None, ws)
    torch.cuda.synchronize()
    got = G.down(o).reshape(N_Q, d).astype(np.float64)
    _check(got, _expected(q, k_rows, v_rows, N, d), f"d{d} split={split}")
    if ws is not None:
        G.assert_counters_zero(ws, 1, N_Q, d)


@pytest.mark.parametrize("d,N", [(64, (1 << 24) - 64), (128, (1 << 23) - 64)])
def test_largest_key_range_fresh_tail(d, N):
    """The last 64 rows (two planted keys among them) come from this step's
    tensors through the fused call and land at the top of the buffer."""
    G.require_gpu()
    torch = G.torch_mod()
    G.announce(f"largest key range d{d} N{N}, fresh last tile")
    q, rows, k_rows, v_rows = _case(d, N)
    k_buf, v_buf = _buffers(d, N, rows[:2], k_rows[:2], v_rows[:2], torch)
    k_new = np.zeros((64, d))
    v_new = np.zeros((64, d))
    for j, kr, vr in zip(rows[2:], k_rows[2:], v_rows[2:]):
        k_new[j - (N - 64)] = kr
        v_new[j - (N - 64)] = vr
    k_new_d = torch.tensor(k_new.reshape(1, 1, 64, d), dtype=torch.bfloat16, device="cuda")
    v_new_t = torch.tensor(v_new.T.reshape(1, 1, d, 64).copy(), dtype=torch.bfloat16,
                           device="cuda")
    qd = torch.tensor(q.reshape(1, 1, N_Q, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(qd)
    ws = dfp.attention_workspace(1, 1, N_Q, N, d)
    dfp.patch_attention_fresh(o, qd, k_buf, v_buf, [(k_new_d, v_new_t, N - 64)], True, None, ws)
    torch.cuda.synchronize()
    got = G.down(o).reshape(N_Q, d).astype(np.float64)
    _check(got, _expected(q, k_rows, v_rows, N, d), f"d{d} fresh")
    # the fresh rows landed bit for bit at the top of the buffer
    assert torch.equal(k_buf[0, 0, N - 64:, :], k_new_d[0, 0])
    assert torch.equal(v_buf[0, 0, :, N - 64:N], v_new_t[0, 0])
