"""GPU parity of the fused guidance + sampler + rel-MAE step (dfp_cfg_step)
and of dfp_relmae against the fp64 oracle.

Bars: latent step relative L2 <= 1e-5, checked one step at a time (both
sides start each step from the same fp32 x_t); rel-MAE relative error
<= 1e-5 at every step.  Every workload runs its full sampler (10 / 50 / 28
steps)."""
import math

import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import dfp, inputs
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

STEP_REL_L2 = 1e-5
RELMAE_REL = 1e-5


def _schedule(wl):
    return oracle.DDIMSchedule(wl.steps) if wl.sampler == "ddim" else oracle.EulerSchedule(wl.steps)


def _gpu_coeffs(wl, i):
    """The GPU path's own coefficients from the library's host helpers."""
    if wl.sampler == "ddim":
        abar = dfp.scaled_linear_abar(1000, 0.00085, 0.012)
        ts = dfp.ddim_timesteps(1000, wl.steps)
        S = wl.steps
        t = ts[S - 1 - i]
        a_prev = 1.0 if i == S - 1 else abar[ts[S - 2 - i]]
        return dfp.ddim_coeffs(abar[t], a_prev)
    sig = [1.0 - k / wl.steps for k in range(wl.steps + 1)]
    return dfp.euler_coeffs(sig[i], sig[i + 1])


@pytest.mark.parametrize("name", ["tiny-f32", "sdxl1024", "sdxl2048", "sdxl3840", "dit1024"])
def test_sampler_run_step_by_step(name):
    G.require_gpu()
    wl = inputs.WORKLOADS[name]
    G.announce(f"cfg step {name}: {wl.steps} {wl.sampler} steps on {wl.latent}")
    torch = G.torch_mod()
    stream = inputs.sampler_stream(wl)
    sch = _schedule(wl)
    batch = wl.latent[0]
    n = wl.n_latent
    ws = dfp.cfg_workspace(n, batch).fill_(255)   # initial contents must not matter
    r_dev = torch.empty(batch, dtype=torch.float32, device="cuda")
    x_host = stream.x_T.astype(np.float32)
    x_ref_traj = x_host.astype(np.float64)
    worst_step, worst_r = 0.0, 0.0
    series = []
    for i in range(wl.steps):
        g_c, g_u = stream.next_pair()
        x = torch.from_numpy(x_host).cuda()
        c_x, c_e = _gpu_coeffs(wl, i)
        dfp.cfg_step(x, torch.from_numpy(g_c).cuda(), torch.from_numpy(g_u).cuda(), wl.w,
                     c_x, c_e, r_dev, ws)
        torch.cuda.synchronize()
        got = x.cpu().numpy()
        want, r_want = sch.step(x_host, g_c, g_u, wl.w, i)
        err = G.rel_l2(got, want)
        r_got = float(r_dev[0].item())
        series.append(r_got)
        rerr = abs(r_got - r_want) / abs(r_want)
        worst_step, worst_r = max(worst_step, err), max(worst_r, rerr)
        assert err <= STEP_REL_L2, f"{name} step {i}: rel L2 {err}"
        assert rerr <= RELMAE_REL, f"{name} step {i}: rel-MAE {r_got} vs {r_want}"
        x_ref_traj, _ = sch.step(x_ref_traj, g_c, g_u, wl.w, i)
        x_host = got
    traj = G.rel_l2(x_host, x_ref_traj)
    G.announce(f"{name}: worst step relL2 {worst_step:.2e}, worst rel-MAE err {worst_r:.2e}, "
               f"full-trajectory relL2 {traj:.2e}")
    assert np.isfinite(x_host).all()
    # the three-phase switch rule on the series this run produced
    for Lw, g in ((1, 0.01), (3, 0.005)):
        assert dfp.switch_points(series, Lw, g) == oracle.switch_points(series, Lw, g)


@pytest.mark.parametrize("name,eta", [("tiny-f32", 1.0), ("sdxl1024", 0.5), ("sdxl3840", 1.0)])
def test_ddim_eta_run_step_by_step(name, eta):
    """DDIM with eta > 0 through dfp_cfg_step_noise: every step against the
    oracle's literal eta step, on the same fp32 x_t, predictions and noise."""
    G.require_gpu()
    wl = inputs.WORKLOADS[name]
    G.announce(f"cfg step with noise {name}: eta {eta}, {wl.steps} steps on {wl.latent}")
    torch = G.torch_mod()
    stream = inputs.sampler_stream(wl)
    sch = oracle.DDIMSchedule(wl.steps)
    batch = wl.latent[0]
    ws = dfp.cfg_workspace(wl.n_latent, batch)
    r_dev = torch.empty(batch, dtype=torch.float32, device="cuda")
    x_host = stream.x_T.astype(np.float32)
    for i in range(wl.steps):
        g_c, g_u = stream.next_pair()
        z = stream.next_noise()
        at, ap, last = sch.step_args(i)
        c_x, c_e, c_z = dfp.ddim_eta_coeffs(at, ap, eta)
        x = torch.from_numpy(x_host).cuda()
        dfp.cfg_step_noise(x, torch.from_numpy(g_c).cuda(), torch.from_numpy(g_u).cuda(),
                           torch.from_numpy(z).cuda(), wl.w, c_x, c_e, c_z, r_dev, ws)
        torch.cuda.synchronize()
        got = x.cpu().numpy()
        want, r_want = sch.step_eta(x_host, g_c, g_u, wl.w, i, eta, z)
        err = G.rel_l2(got, want)
        rerr = abs(float(r_dev[0].item()) - r_want) / abs(r_want)
        assert err <= STEP_REL_L2, f"{name} step {i}: rel L2 {err}"
        assert rerr <= RELMAE_REL, f"{name} step {i}: rel-MAE error {rerr}"
        x_host = got
    assert np.isfinite(x_host).all()


def test_relmae_alone_batch_and_determinism():
    G.require_gpu()
    G.announce("relmae batch=3, determinism")
    torch = G.torch_mod()
    r = np.random.Generator(np.random.PCG64(77))
    n = 4 * 96 * 96
    g_c = r.standard_normal((3, n), dtype=np.float32)
    g_u = r.standard_normal((3, n), dtype=np.float32)
    g_c[1] = 1.5 * g_u[1]                      # rel-MAE exactly 0.5
    ws = dfp.cfg_workspace(n, 3)
    out = torch.empty(3, dtype=torch.float32, device="cuda")
    dc, du = torch.from_numpy(g_c).cuda(), torch.from_numpy(g_u).cuda()
    dfp.relmae(dc, du, out, ws)
    torch.cuda.synchronize()
    a = out.cpu().numpy().copy()
    for b in range(3):
        want = oracle.relmae(g_c[b], g_u[b])
        assert abs(a[b] - want) / want <= RELMAE_REL
    assert abs(a[1] - 0.5) < 1e-6
    dfp.relmae(dc, du, out, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), a)


def test_relmae_many_images_one_call():
    """Batch 70 in one call (one merge workgroup per image): every image's
    ratio against the oracle."""
    G.require_gpu()
    G.announce("relmae batch=70")
    torch = G.torch_mod()
    r = np.random.Generator(np.random.PCG64(78))
    batch, n = 70, 4 * 64 * 64
    g_c = r.standard_normal((batch, n), dtype=np.float32)
    g_u = r.standard_normal((batch, n), dtype=np.float32) * np.linspace(0.5, 2.0, batch,
                                                                         dtype=np.float32)[:, None]
    ws = dfp.cfg_workspace(n, batch)
    out = torch.empty(batch, dtype=torch.float32, device="cuda")
    dfp.relmae(torch.from_numpy(g_c).cuda(), torch.from_numpy(g_u).cuda(), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(batch):
        want = oracle.relmae(g_c[b], g_u[b])
        assert abs(got[b] - want) / want <= RELMAE_REL, f"image {b}"


@pytest.mark.parametrize("n,offset", [(1001, 0), (4096, 1), (3, 0), (1, 0)])
def test_scalar_path_ragged_or_misaligned(n, offset):
    G.require_gpu()
    G.announce(f"cfg step scalar path n={n} offset={offset}")
    torch = G.torch_mod()
    r = np.random.Generator(np.random.PCG64(n + offset))
    x0 = r.standard_normal(n, dtype=np.float32)
    g_c = r.standard_normal(n, dtype=np.float32)
    g_u = r.standard_normal(n, dtype=np.float32)

    def dev(a):
        t = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
        t[offset:] = torch.from_numpy(a).cuda()
        return t[offset:].view(1, n)

    x = dev(x0)
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = dfp.cfg_workspace(n, 1)
    c_x, c_e = dfp.ddim_coeffs(0.3, 0.6)
    dfp.cfg_step(x, dev(g_c), dev(g_u), 7.5, c_x, c_e, out, ws)
    torch.cuda.synchronize()
    want = oracle.ddim_step(x0, oracle.cfg_combine(g_c, g_u, 7.5), 0.3, 0.6, False)
    assert G.rel_l2(x.cpu().numpy().ravel(), want) <= STEP_REL_L2
    rw = oracle.relmae(g_c, g_u)
    assert abs(out.item() - rw) / rw <= RELMAE_REL


def test_no_reduction_and_degenerate_ratios():
    G.require_gpu()
    G.announce("cfg step without rel-MAE; degenerate rel-MAE")
    torch = G.torch_mod()
    n = 4 * 32 * 32
    r = np.random.Generator(np.random.PCG64(3))
    x0 = r.standard_normal((1, n), dtype=np.float32)
    g = r.standard_normal((1, n), dtype=np.float32)
    x = torch.from_numpy(x0).cuda()
    dg = torch.from_numpy(g).cuda()
    c_x, c_e = dfp.euler_coeffs(1.0, 0.5)
    dfp.cfg_step(x, dg, dg, 3.5, c_x, c_e, None, None)
    torch.cuda.synchronize()
    want = oracle.euler_step(x0, g, 1.0, 0.5)
    assert G.rel_l2(x.cpu().numpy(), want) <= STEP_REL_L2
    ws = dfp.cfg_workspace(n, 2)
    out = torch.empty(2, dtype=torch.float32, device="cuda")
    zeros = torch.zeros((2, n), dtype=torch.float32, device="cuda")
    ones = torch.ones((2, n), dtype=torch.float32, device="cuda")
    dfp.relmae(zeros, zeros, out, ws)
    torch.cuda.synchronize()
    assert math.isnan(out[0].item()) and math.isnan(out[1].item())
    dfp.relmae(ones, zeros, out, ws)
    torch.cuda.synchronize()
    assert math.isinf(out[0].item()) and out[0].item() > 0


def _random_case(i):
    rng = np.random.Generator(np.random.PCG64(8000 + i))
    n = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 70000)),
                        int(rng.integers(70000, 600000))]))
    a_t = float(rng.uniform(0.01, 0.9))
    s0 = float(rng.uniform(0.05, 1.0))
    return dict(batch=int(rng.integers(1, 6)), n=n,
                kind=str(rng.choice(["ddim", "ddim_last", "euler", "eta"])),
                w=float(rng.uniform(0.0, 10.0)), offset=int(rng.choice([0, 0, 1, 2, 3])),
                with_relmae=bool(rng.integers(0, 4) != 0), a_t=a_t,
                a_prev=float(rng.uniform(a_t, 0.999)), eta=float(rng.uniform(0.0, 1.0)),
                s0=s0, s1=float(rng.uniform(0.0, s0)))


@pytest.mark.parametrize("i", range(24))
def test_random_shape(i):
    """Seeded draws over latent sizes (a few floats to over half a million
    per image, 1-5 images per call), x and the predictions on and off the
    16-byte grid, DDIM (also its last step and eta > 0) and Euler updates,
    any guidance weight, with and without the rel-MAE output: every image's
    step and rel-MAE against the oracle, from a workspace of arbitrary bytes."""
    c = _random_case(i)
    G.require_gpu()
    G.announce(f"cfg step random case {i}: {c}")
    torch = G.torch_mod()
    B, n, off = c["batch"], c["n"], c["offset"]
    r = np.random.Generator(np.random.PCG64(8100 + i))
    x0, g_c, g_u, z = (r.standard_normal((B, n), dtype=np.float32) for _ in range(4))

    def dev(a):
        t = torch.full((B * n + off + 16,), float("nan"), dtype=torch.float32, device="cuda")
        t[off:off + B * n] = torch.from_numpy(a.ravel()).cuda()
        return t, t[off:off + B * n].view(B, n)

    xs, x = dev(x0)
    out = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda") \
        if c["with_relmae"] else None
    ws = dfp.cfg_workspace(n, B).fill_(0xA5) if c["with_relmae"] else None
    args = (dev(g_c)[1], dev(g_u)[1])
    kind = c["kind"]
    if kind == "eta":
        c_x, c_e, c_z = dfp.ddim_eta_coeffs(c["a_t"], c["a_prev"], c["eta"])
        dfp.cfg_step_noise(x, *args, dev(z)[1], c["w"], c_x, c_e, c_z, out, ws)
    else:
        if kind == "euler":
            c_x, c_e = dfp.euler_coeffs(c["s0"], c["s1"])
        else:
            c_x, c_e = dfp.ddim_coeffs(c["a_t"], 1.0 if kind == "ddim_last" else c["a_prev"])
        dfp.cfg_step(x, *args, c["w"], c_x, c_e, out, ws)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    for b in range(B):
        g = oracle.cfg_combine(g_c[b], g_u[b], c["w"])
        if kind == "eta":
            want = oracle.ddim_step_eta(x0[b], g, z[b], c["a_t"], c["a_prev"], c["eta"], False)
        elif kind == "euler":
            want = oracle.euler_step(x0[b], g, c["s0"], c["s1"])
        else:
            want = oracle.ddim_step(x0[b], g, c["a_t"], c["a_prev"], kind == "ddim_last")
        assert G.rel_l2(got[b], want) <= STEP_REL_L2, f"image {b}"
        if out is not None:
            rw = oracle.relmae(g_c[b], g_u[b])
            assert abs(out[b].item() - rw) / rw <= RELMAE_REL, f"image {b}"
    assert torch.isnan(xs[off + B * n:]).all() and torch.isnan(xs[:off]).all()
