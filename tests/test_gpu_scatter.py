"""GPU: dfp_kv_scatter must be a bit-exact landing of the fresh rows: after
the call the buffer equals the oracle's effective K/V (stale outside the
patch rows, fresh inside), bit for bit, in both dtypes, at aligned and
unaligned row offsets."""
import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import dfp, inputs
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _bits(a: np.ndarray, kind: str) -> np.ndarray:
    return inputs.bf16_bits(a) if kind == "bf16" else np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,N,d,row0,n", [
    (2, 2, 1024, 64, 512, 512),     # tiny fp32 workload shape
    (2, 3, 200, 64, 3, 37),          # unaligned offset, ragged n
    (1, 2, 130, 128, 64, 66),        # d=128, ragged tail
    (2, 2, 64, 64, 0, 64),           # whole buffer
    (1, 1, 13, 64, 12, 1),           # single row at the end, ragged N (padded ldv)
    (2, 2, 300, 8, 100, 150),        # small d
])
def test_scatter_bit_exact(kind, B, H, N, d, row0, n):
    G.require_gpu()
    G.announce(f"scatter {kind} B{B} H{H} N{N} d{d} row0={row0} n={n}")
    torch = G.torch_mod()
    q, stale_k, stale_v = inputs.random_attention_arrays(B, H, 1, N, d, seed=N + d, dtype=kind)
    _, fresh_k, fresh_v = inputs.random_attention_arrays(B, H, 1, n, d, seed=N + d + 1, dtype=kind)
    k_buf, v_buf = dfp.alloc_kv_buffer(B, H, N, d, G.dtype_of(kind))
    v_buf.fill_(float("nan"))   # padding columns must never matter
    dfp.kv_scatter(k_buf, v_buf, G.up(stale_k, kind), G.up(stale_v, kind), 0)
    dfp.kv_scatter(k_buf, v_buf, G.up(fresh_k, kind), G.up(fresh_v, kind), row0)
    torch.cuda.synchronize()
    want_k = oracle.effective_kv(stale_k, fresh_k, row0).astype(np.float32)
    want_v = oracle.effective_kv(stale_v, fresh_v, row0).astype(np.float32)
    got_k = G.down(k_buf)
    got_v = G.v_buffer_to_rows(v_buf, N)
    np.testing.assert_array_equal(_bits(got_k, kind), _bits(want_k, kind))
    np.testing.assert_array_equal(_bits(got_v, kind), _bits(want_v, kind))


def test_scatter_only_v_or_only_k_and_empty():
    G.require_gpu()
    G.announce("scatter partial pairs")
    torch = G.torch_mod()
    _, sk, sv = inputs.random_attention_arrays(1, 2, 1, 96, 64, seed=5)
    _, fk, fv = inputs.random_attention_arrays(1, 2, 1, 16, 64, seed=6)
    k_buf, v_buf = dfp.alloc_kv_buffer(1, 2, 96, 64, torch.bfloat16)
    dfp.kv_scatter(k_buf, v_buf, G.up(sk, "bf16"), G.up(sv, "bf16"), 0)
    dfp.kv_scatter(k_buf, None, G.up(fk, "bf16"), None, 40)   # K only
    dfp.kv_scatter(k_buf, v_buf, G.up(fk[:, :, :0], "bf16"), G.up(fv[:, :, :0], "bf16"), 96)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.down(k_buf), oracle.effective_kv(sk, fk, 40))
    np.testing.assert_array_equal(G.v_buffer_to_rows(v_buf, 96), sv)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,N,d,row0,n", [
    (2, 10, 57600, 64, 7200, 7200),  # an SDXL-3840 patch, from a [B, n, H, d] projection
    (2, 3, 200, 64, 3, 37),           # unaligned offset, ragged n
    (1, 2, 130, 128, 64, 66),         # d=128
    (2, 1, 96, 64, 5, 1),             # one row, one head
])
def test_strided_scatter_from_token_major_rows(kind, B, H, N, d, row0, n):
    """dfp_kv_scatter_strided lands fresh rows held token-major ([B, n, H, d],
    a projection's natural output, viewed as [B, H, n, d]) and rows of a
    wider tensor (a slice), bit for bit as dfp_kv_scatter of the dense rows."""
    G.require_gpu()
    G.announce(f"strided scatter {kind} B{B} H{H} N{N} d{d} row0={row0} n={n}")
    torch = G.torch_mod()
    _, sk, sv = inputs.random_attention_arrays(B, H, 1, N, d, seed=N + 3, dtype=kind)
    _, fk, fv = inputs.random_attention_arrays(B, H, 1, n, d, seed=N + 4, dtype=kind)
    dt = G.dtype_of(kind)
    want_k = oracle.effective_kv(sk, fk, row0).astype(np.float32)
    want_v = oracle.effective_kv(sv, fv, row0).astype(np.float32)
    # token-major storage [B, n, H, d], viewed as [B, H, n, d]
    tk = G.up(np.ascontiguousarray(np.swapaxes(fk, 1, 2)), kind).permute(0, 2, 1, 3)
    tv = G.up(np.ascontiguousarray(np.swapaxes(fv, 1, 2)), kind).permute(0, 2, 1, 3)
    # rows 8..8+n of a wider dense tensor
    wide_k = torch.zeros((B, H, n + 16, d), dtype=dt, device="cuda")
    wide_v = torch.zeros((B, H, n + 16, d), dtype=dt, device="cuda")
    wide_k[:, :, 8:8 + n] = G.up(fk, kind)
    wide_v[:, :, 8:8 + n] = G.up(fv, kind)
    for src_k, src_v in ((tk, tv), (wide_k[:, :, 8:8 + n], wide_v[:, :, 8:8 + n])):
        k_buf, v_buf = dfp.alloc_kv_buffer(B, H, N, d, dt)
        v_buf.fill_(float("nan"))
        dfp.kv_scatter(k_buf, v_buf, G.up(sk, kind), G.up(sv, kind), 0)
        dfp.kv_scatter_strided(k_buf, v_buf, src_k, src_v, row0)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(G.down(k_buf), kind), _bits(want_k, kind))
        np.testing.assert_array_equal(_bits(G.v_buffer_to_rows(v_buf, N), kind),
                                      _bits(want_v, kind))
