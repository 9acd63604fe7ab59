"""The library's calls captured in a HIP graph, as bench.py times them:
fused attention with landing (split plan, so the workspace counters are
used) followed by the fused guidance step, replayed several times with eager
library calls between the replays.  Every replay must match the same calls
run eagerly, bit for bit (both are deterministic), and leave the counters at
zero."""
import numpy as np
import pytest

from patch_attention_cfg_amd import dfp, inputs
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(monkeypatch):
    G.require_gpu()
    G.announce("graph replay: fused attention (3-way split) + fused cfg step, 4 replays")
    monkeypatch.setenv("DFP_ATTN_SPLITS", "3")
    torch = G.torch_mod()
    B, H, nq, N, d, row0, n = 2, 2, 256, 1024, 64, 256, 256
    q, k_st, v_st = inputs.random_attention_arrays(B, H, nq, N, d, seed=41)
    _, k_new, v_new = inputs.random_attention_arrays(B, H, 1, n, d, seed=42)
    k_buf, v_buf = dfp.alloc_kv_buffer(B, H, N, d, torch.bfloat16)
    dfp.kv_scatter(k_buf, v_buf, G.up(k_st, "bf16"), G.up(v_st, "bf16"), 0)
    fresh = [(G.up(k_new, "bf16"), G.up(np.swapaxes(v_new, -1, -2), "bf16"), row0)]
    qd = G.up(q, "bf16")
    ws = dfp.attention_workspace(B, H, nq, N, d)
    assert ws is not None

    rng = np.random.Generator(np.random.PCG64(43))
    nl = 4 * 32 * 32
    x0 = rng.standard_normal((1, nl), dtype=np.float32)
    g_c = torch.from_numpy(rng.standard_normal((1, nl), dtype=np.float32)).cuda()
    g_u = torch.from_numpy(rng.standard_normal((1, nl), dtype=np.float32)).cuda()
    c_x, c_e = dfp.ddim_coeffs(0.5, 0.6)
    cws = dfp.cfg_workspace(nl, 1)

    def step(o, x, r):
        dfp.patch_attention_fresh(o, qd, k_buf, v_buf, fresh, True, None, ws)
        dfp.cfg_step(x, g_c, g_u, 7.5, c_x, c_e, r, cws)

    # eager reference: the attention output and the latent after 1..4 steps
    o_e = torch.empty_like(qd)
    x_e = torch.from_numpy(x0.copy()).cuda()
    r_e = torch.empty(1, dtype=torch.float32, device="cuda")
    want_x, want_r = [], []
    for _ in range(4):
        step(o_e, x_e, r_e)
        torch.cuda.synchronize()
        want_x.append(x_e.cpu().numpy().copy())
        want_r.append(r_e.cpu().numpy().copy())
    want_o = G.down(o_e)

    o_g = torch.empty_like(qd)
    x_g = torch.from_numpy(x0.copy()).cuda()
    r_g = torch.empty(1, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # warm-up outside capture, then restore x
        step(o_g, x_g, r_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    x_g.copy_(torch.from_numpy(x0))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(o_g, x_g, r_g)
    torch.cuda.synchronize()
    x_g.copy_(torch.from_numpy(x0))
    torch.cuda.synchronize()

    other = torch.empty_like(qd)
    for i in range(4):
        o_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.down(o_g), want_o, err_msg=f"replay {i} attention")
        np.testing.assert_array_equal(x_g.cpu().numpy(), want_x[i], err_msg=f"replay {i} latent")
        np.testing.assert_array_equal(r_g.cpu().numpy(), want_r[i], err_msg=f"replay {i} rel-MAE")
        G.assert_counters_zero(ws, B * H, nq, d)
        # eager work on the same workspace between replays
        dfp.patch_attention(other, qd, k_buf, v_buf, None, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.down(other), want_o)


def test_group_norm_graph_replays_match_eager():
    """The chunked displaced GroupNorm (two launches: chunk sums, then
    statistics and normalization) captured in a HIP graph: every replay
    gives the eager call's bits and lands the same sums, with an eager call
    on the same workspace between replays."""
    G.require_gpu()
    G.announce("graph replay: chunked displaced GroupNorm, 4 replays")
    torch = G.torch_mod()
    B, C, G_, n, P, p = 2, 64, 4, 8192, 4, 2        # groups of 128 Ki floats: chunked
    a = inputs.group_norm_inputs(B, C, G_, n, P, p, seed=44)
    x = torch.from_numpy(a.x).cuda()
    ga, be = torch.from_numpy(a.gamma).cuda(), torch.from_numpy(a.beta).cuda()
    ws = dfp.group_norm_workspace(B, C, G_, n)
    assert ws is not None

    st_e = torch.from_numpy(a.stats).cuda()
    y_e = torch.empty_like(x)
    dfp.displaced_group_norm(y_e, x, st_e, G_, p, 1e-5, ga, be, True, ws)
    torch.cuda.synchronize()
    want_y, want_st = G.down(y_e), st_e.cpu().numpy()

    st_g = torch.from_numpy(a.stats).cuda()
    y_g = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # warm-up outside capture
        dfp.displaced_group_norm(y_g, x, st_g, G_, p, 1e-5, ga, be, True, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dfp.displaced_group_norm(y_g, x, st_g, G_, p, 1e-5, ga, be, True, ws)
    torch.cuda.synchronize()

    other = torch.empty_like(x)
    for i in range(4):
        y_g.zero_()
        st_g.copy_(torch.from_numpy(a.stats))
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.down(y_g), want_y, err_msg=f"replay {i} output")
        np.testing.assert_array_equal(st_g.cpu().numpy(), want_st, err_msg=f"replay {i} sums")
        dfp.displaced_group_norm(other, x, st_e, G_, p, 1e-5, ga, be, True, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.down(other), want_y)


def test_fused_step_entries_in_graph():
    """The fused step's other entry points under capture: the in-kernel noise
    draw (dfp_cfg_step_philox) and the no-allocation step
    (dfp_cfg_step_static, partials in the library's static scratch), two
    launches each, captured in one graph and replayed four times with eager
    calls of both entries (other sizes, the same scratch) between the
    replays; every replay matches the eager sequence bit for bit."""
    G.require_gpu()
    G.announce("graph replay: cfg_step_philox + cfg_step_static, 4 replays")
    torch = G.torch_mod()
    rng = np.random.Generator(np.random.PCG64(47))
    n, batch = 4 * 96 * 96, 2
    x0 = rng.standard_normal((batch, n), dtype=np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    g_c, g_u = dev(rng.standard_normal((batch, n), dtype=np.float32)), \
        dev(rng.standard_normal((batch, n), dtype=np.float32))
    c_x, c_e, c_z = dfp.ddim_eta_coeffs(0.3, 0.5, 0.7)
    ws = dfp.cfg_workspace(n, batch)

    def step(x, r1, r2):
        dfp.cfg_step_philox(x, g_c, g_u, 6.0, c_x, c_e, c_z, 2024, 11, r1, ws)
        dfp.cfg_step_static(x, g_u, g_c, 4.0, 0.99, -0.02, r2)

    x_e = dev(x0.copy())
    r1_e = torch.empty(batch, device="cuda")
    r2_e = torch.empty(batch, device="cuda")
    want = []
    for _ in range(4):
        step(x_e, r1_e, r2_e)
        torch.cuda.synchronize()
        want.append((x_e.cpu().numpy().copy(), r1_e.cpu().numpy().copy(),
                     r2_e.cpu().numpy().copy()))

    x_g = dev(x0.copy())
    r1_g = torch.empty(batch, device="cuda")
    r2_g = torch.empty(batch, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # warm-up outside capture, then restore x
        step(x_g, r1_g, r2_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    x_g.copy_(dev(x0))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(x_g, r1_g, r2_g)
    torch.cuda.synchronize()
    x_g.copy_(dev(x0))
    torch.cuda.synchronize()

    small = dev(rng.standard_normal((1, 4 * 32 * 32), dtype=np.float32))
    r_small = torch.empty(1, device="cuda")
    for i in range(4):
        graph.replay()
        torch.cuda.synchronize()
        wx, wr1, wr2 = want[i]
        np.testing.assert_array_equal(x_g.cpu().numpy(), wx, err_msg=f"replay {i} latent")
        np.testing.assert_array_equal(r1_g.cpu().numpy(), wr1, err_msg=f"replay {i} rel-MAE 1")
        np.testing.assert_array_equal(r2_g.cpu().numpy(), wr2, err_msg=f"replay {i} rel-MAE 2")
        # eager calls of both entries between replays, on other sizes
        xs = small.clone()
        dfp.cfg_step_static(xs, small, small * 0.5, 2.0, 1.0, -0.1, r_small)
        dfp.cfg_step_philox(xs, small, small, 1.0, 1.0, 0.0, 0.1, 5, i, r_small,
                            dfp.cfg_workspace(small.numel(), 1))
        torch.cuda.synchronize()
