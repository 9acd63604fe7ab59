"""dfp_cfg_step_static -- the fused step for callers that cannot allocate
device memory -- called through the C ABI against dfp_cfg_step on the same
inputs: two calls in a row on one GPU, the second with a smaller latent (the
static scratch keeps the first call's partials), both bit for bit equal to
dfp_cfg_step with a workspace and within the parity bars of the fp64 oracle
(step relative L2 <= 1e-5, rel-MAE relative <= 1e-5); sizes beyond the
static scratch are refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import dfp
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

STEP_REL_L2 = 1e-5
RELMAE_REL = 1e-5


def _run(torch, batch, n, seed, w, a_t, a_p):
    r = np.random.Generator(np.random.PCG64(seed))
    x0, g_c, g_u = (r.standard_normal((batch, n), dtype=np.float32) for _ in range(3))
    c_x, c_e = dfp.ddim_coeffs(a_t, a_p)
    dev = lambda a: torch.from_numpy(a).cuda()
    xa, xb = dev(x0), dev(x0)
    dc, du = dev(g_c), dev(g_u)
    ra = torch.full((batch,), float("nan"), device="cuda")
    rb = torch.full((batch,), float("nan"), device="cuda")
    L = dfp.lib()
    st = L.dfp_cfg_step_static(ctypes.c_void_p(xa.data_ptr()), ctypes.c_void_p(dc.data_ptr()),
                               ctypes.c_void_p(du.data_ptr()), n, batch, w, c_x, c_e,
                               ctypes.c_void_p(ra.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == dfp.OK, dfp.status_string(st)
    dfp.cfg_step(xb, dc, du, w, c_x, c_e, rb, dfp.cfg_workspace(n, batch))
    torch.cuda.synchronize()
    a, b = xa.cpu().numpy(), xb.cpu().numpy()
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    np.testing.assert_array_equal(ra.cpu().numpy(), rb.cpu().numpy())
    for i in range(batch):
        want = oracle.ddim_step(x0[i], oracle.cfg_combine(g_c[i], g_u[i], w), a_t, a_p, False)
        assert G.rel_l2(a[i], want) <= STEP_REL_L2
        rw = oracle.relmae(g_c[i], g_u[i])
        assert abs(float(ra[i].item()) - rw) / rw <= RELMAE_REL


def test_static_scratch_matches_workspace_call_twice():
    G.require_gpu()
    torch = G.torch_mod()
    G.announce("no-alloc cfg step: SDXL-3840 latent x2, then SDXL-1024 latent")
    _run(torch, 2, 4 * 480 * 480, 11, 7.5, 0.2, 0.4)
    _run(torch, 1, 4 * 128 * 128, 12, 5.0, 0.6, 0.8)


def test_static_scratch_refuses_oversize():
    G.require_gpu()
    torch = G.torch_mod()
    G.announce("no-alloc cfg step: oversize refused")
    L = dfp.lib()
    cap = int(L.dfp_cfg_static_scratch_bytes())
    n, batch = 4 * 480 * 480, 1
    while dfp.workspace_bytes(dfp.OP_CFG_STEP, n, batch) <= cap:
        batch += 1
    # real buffers of the refused size, so nothing could go out of bounds
    x = torch.zeros((batch, n), device="cuda")
    g = torch.ones((batch, n), device="cuda")
    r = torch.zeros(batch, device="cuda")
    st = L.dfp_cfg_step_static(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                               ctypes.c_void_p(g.data_ptr()), n, batch, 7.5, 1.0, -0.1,
                               ctypes.c_void_p(r.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == dfp.ERR_TOO_LARGE, dfp.status_string(st)
    torch.cuda.synchronize()
    assert float(x.abs().sum().item()) == 0.0 and float(r.abs().sum().item()) == 0.0
    # the largest size that fits runs
    st = L.dfp_cfg_step_static(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                               ctypes.c_void_p(g.data_ptr()), n, batch - 1, 7.5, 1.0, -0.1,
                               ctypes.c_void_p(r.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == dfp.OK
    torch.cuda.synchronize()
    assert bool((r[:batch - 1] == 0.0).all())   # g_c == g_u: rel-MAE 0 for every image
