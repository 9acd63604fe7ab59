"""The fused guidance step driven from a plain C program (tests/c/step_from_c.c,
built by build()): hipMalloc'd buffers, its own stream, dfp_ddim_coeffs and
dfp_cfg_step through the C ABI, no Python in the path.  Its output is
checked against the fp64 oracle at the latent-step and rel-MAE bars."""
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
    subprocess.run([build.C_CALLER, str(tmp_path), str(x.size), repr(wl.w), repr(a_t),
                    repr(a_prev)], check=True, timeout=120)
    got = np.fromfile(tmp_path / "x_out.f32", dtype=np.float32).astype(np.float64)
    r = float(np.fromfile(tmp_path / "relmae.f32", dtype=np.float32)[0])
    want = oracle.ddim_step(x, oracle.cfg_combine(g_c, g_u, wl.w), a_t, a_prev, last)
    assert G.rel_l2(got, want) <= 1e-5
    rw = oracle.relmae(g_c, g_u)
    assert abs(r - rw) <= 1e-5 * abs(rw)
