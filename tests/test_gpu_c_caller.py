"""The hot path driven from a plain C program (tests/c/step_from_c.c, built
by build()): hipMalloc'd buffers, its own stream, and the C ABI's calls with
no Python in the path -- the fused guidance step (dfp_ddim_coeffs,
dfp_cfg_step) and the patch attention (dfp_kv_scatter of the stale buffer
and the fresh rows, dfp_patch_attention).  Outputs are checked against the
fp64 oracle at the step and bf16 attention bars."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import build, inputs
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,step", [("sdxl1024", 0), ("sdxl3840", 17)])
def test_step_from_c(tmp_path, name, step):
    G.require_gpu()
    assert os.path.exists(build.C_CALLER), "build() makes the C caller"
    wl = inputs.WORKLOADS[name]
    G.announce(f"fused step from C: {name} step {step}")
    st = inputs.sampler_stream(wl)
    x = st.x_T.reshape(-1)
    for _ in range(step):
        st.next_pair()
    g_c, g_u = (a.reshape(-1) for a in st.next_pair())
    sch = oracle.DDIMSchedule(wl.steps)
    a_t, a_prev, last = sch.step_args(step)
    for fname, arr in (("x.f32", x), ("g_c.f32", g_c), ("g_u.f32", g_u)):
        np.ascontiguousarray(arr, dtype=np.float32).tofile(tmp_path / fname)
    subprocess.run([build.C_CALLER, "step", str(tmp_path), str(x.size), repr(wl.w), repr(a_t),
                    repr(a_prev)], check=True, timeout=120)
    got = np.fromfile(tmp_path / "x_out.f32", dtype=np.float32).astype(np.float64)
    r = float(np.fromfile(tmp_path / "relmae.f32", dtype=np.float32)[0])
    want = oracle.ddim_step(x, oracle.cfg_combine(g_c, g_u, wl.w), a_t, a_prev, last)
    assert G.rel_l2(got, want) <= 1e-5
    rw = oracle.relmae(g_c, g_u)
    assert abs(r - rw) <= 1e-5 * abs(rw)


def _bf16_bits(a):
    """Bit patterns of values that are already bf16 (the inputs' rounding)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    assert not (u & 0xFFFF).any()
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("name,p", [("sdxl1024-64x64", 2), ("sdxl1024-32x32", 3)])
def test_attention_from_c(tmp_path, name, p):
    G.require_gpu()
    assert os.path.exists(build.C_CALLER), "build() makes the C caller"
    lv = inputs.LEVELS[name]
    G.announce(f"patch attention from C: {name} patch {p}")
    x = inputs.attention_inputs(lv)
    kf, vf = x.fresh_rows(p)
    q = x.q_patch(p)
    for fname, arr in (("q.bf16", q), ("k_stale.bf16", x.k_stale), ("v_stale.bf16", x.v_stale),
                       ("k_fresh.bf16", kf), ("v_fresh.bf16", vf)):
        _bf16_bits(arr).tofile(tmp_path / fname)
    subprocess.run([build.C_CALLER, "attn", str(tmp_path), str(lv.B), str(lv.H), str(lv.n),
                    str(lv.N_kv), str(lv.d), str(lv.row0(p)), str(lv.n)], check=True, timeout=120)
    o = np.fromfile(tmp_path / "o.bf16", dtype=np.uint16).astype(np.uint32) << 16
    got = o.view(np.float32).reshape(q.shape).astype(np.float64)
    want = oracle.patch_attention(q, x.k_stale, x.v_stale, kf, vf, lv.row0(p), 1.0 / lv.d ** 0.5)
    assert G.rel_l2(got, want) <= 1e-2
    assert np.abs(got - want).max() <= 2e-2
