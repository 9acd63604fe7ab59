"""The Python binding rejects mismatched tensors before anything is
enqueued: the C ABI takes raw pointers, so a shorter g_u, a buffer of
another dtype or a wrong head size would otherwise make a kernel read past
an allocation.  Every case here raises ValueError in the binding."""
import pytest

from patch_attention_cfg_amd import dfp
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def test_latent_step_mismatches_rejected():
    G.require_gpu()
    G.announce("binding checks: latent step")
    torch = G.torch_mod()
    n = 4 * 32 * 32
    x = torch.zeros((1, n), device="cuda")
    g = torch.zeros((1, n), device="cuda")
    ws = dfp.cfg_workspace(n, 1)
    r = torch.zeros(1, device="cuda")
    bad = [
        lambda: dfp.cfg_step(x, g, g[:, :n - 4], 7.5, 1.0, -0.1, r, ws),           # short g_u
        lambda: dfp.cfg_step(x, g.double(), g, 7.5, 1.0, -0.1, r, ws),              # dtype
        lambda: dfp.cfg_step(x, g.cpu(), g, 7.5, 1.0, -0.1, r, ws),                 # host tensor
        lambda: dfp.cfg_step(x, g, g, 7.5, 1.0, -0.1, r.double(), ws),              # out dtype
        lambda: dfp.cfg_step_noise(x, g, g, g[:, :8], 7.5, 1.0, -0.1, 0.1, r, ws),  # short z
        lambda: dfp.cfg_step_philox(x, g, g.half(), 7.5, 1.0, -0.1, 0.1, 1, 0, r, ws),
        lambda: dfp.relmae(g, g[:, :16], r, ws),
        lambda: dfp.philox_normal(torch.zeros(8, 8, dtype=torch.float64, device="cuda"), 1, 0),
        lambda: dfp.philox4x64_10(torch.zeros(8, 3, dtype=torch.int64, device="cuda"), 0, 0, 0),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(ValueError):
            f()
    torch.cuda.synchronize()
    assert float(x.abs().sum().item()) == 0.0   # nothing ran


def test_attention_mismatches_rejected():
    G.require_gpu()
    G.announce("binding checks: attention and scatter")
    torch = G.torch_mod()
    B, H, N, d, nq = 1, 2, 256, 64, 64
    k_buf, v_buf = dfp.alloc_kv_buffer(B, H, N, d, torch.bfloat16)
    q = torch.zeros((B, H, nq, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    kf = torch.zeros((B, H, 64, d), dtype=torch.bfloat16, device="cuda")
    vft = torch.zeros((B, H, d, 64), dtype=torch.bfloat16, device="cuda")
    k128, v128 = dfp.alloc_kv_buffer(B, H, N, 128, torch.bfloat16)
    vbad = torch.zeros((B, H, 32, d), dtype=torch.bfloat16, device="cuda")
    bad = [
        lambda: dfp.patch_attention(o, q.float(), k_buf, v_buf),                 # q dtype
        lambda: dfp.patch_attention(o.float(), q, k_buf, v_buf),                 # o dtype
        lambda: dfp.patch_attention(o, q, k128, v_buf),                          # k head size
        lambda: dfp.patch_attention(o, q, k_buf, v128),                          # v head size
        lambda: dfp.patch_attention(o[:, :1], q, k_buf, v_buf),                  # o shape
        lambda: dfp.patch_attention_fresh(o, q, k_buf, v_buf, [(kf, vft.float(), 64)]),
        lambda: dfp.patch_attention_fresh(o, q, k_buf, v_buf, [(kf[:, :, :32], vft, 64)]),
        lambda: dfp.kv_scatter(k_buf, v_buf, kf, vbad, 0),                       # v rows != k rows
        lambda: dfp.kv_scatter(k_buf, v_buf, kf.float(), kf.float(), 0),         # dtype
        lambda: dfp.kv_scatter(k_buf, None, kf, kf, 0),                          # half a pair
    ]
    for f in bad:
        with pytest.raises(ValueError):
            f()
    torch.cuda.synchronize()
    assert bool((o.float() == 3.0).all())   # nothing ran
