"""GPU parity of the one-device patch sweep ("xDiT: an Inference Engine for
Diffusion Transformers (DiTs) with Massive Parallelism", 三.2 PipeFusion):
every patch of a layer lands its fresh K/V with dfp_kv_scatter and then
attends with dfp_patch_attention, in patch order, so patch m sees fresh rows
for patches 0..m and stale rows after.  Checked against the oracle's
patch_sweep on every patch.

The stale rows here differ from the fresh ones by unit-variance noise (not
the workloads' 0.05), so reading a wrong fresh/stale row range moves the
output far outside the bf16 bounds.  Large levels compare every query row of
the first (batch, head) slices while the GPU runs the full shape."""
import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import dfp, inputs
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 2e-2
F32_MAX_ABS = 1e-4


@pytest.mark.parametrize("name,heads,fresh", [("tiny-f32", None, False),
                                              ("sdxl1024-64x64", None, False),
                                              ("sdxl1024-32x32", None, False),
                                              ("dit1024", 2, False), ("sdxl2048", 1, False),
                                              ("sdxl1024-64x64", None, True),
                                              ("sdxl1024-32x32", None, True),
                                              ("dit1024", 2, True), ("sdxl2048", 1, True)])
def test_patch_sweep_every_patch(name, heads, fresh):
    """With `fresh` each patch runs dfp_patch_attention_fresh (reading its own
    rows, and a DiT's text rows, from the fresh tensors and landing them)
    instead of scatter + dfp_patch_attention."""
    G.require_gpu()
    torch = G.torch_mod()
    level = inputs.LEVELS[name]
    G.announce(f"patch sweep {name} (P={level.P}) fresh={fresh}")
    kind = level.dtype
    x = inputs.attention_inputs(level, stale_std=1.0)
    B, H, N, d, n = level.B, level.H, level.N_kv, level.d, level.n
    k_buf, v_buf = dfp.alloc_kv_buffer(B, H, N, d, G.dtype_of(kind))
    dfp.kv_scatter(k_buf, v_buf, G.up(x.k_stale, kind), G.up(x.v_stale, kind), 0)
    if level.n_text:
        kt, vt = x.text_rows()
        dfp.kv_scatter(k_buf, v_buf, G.up(kt, kind), G.up(vt, kind), 0)
    sl = (slice(None), slice(None)) if heads is None else (slice(0, 1), slice(0, heads))
    want = oracle.patch_sweep(x.q[sl], x.k_stale[sl], x.v_stale[sl], x.k_fresh[sl],
                              x.v_fresh[sl], level.P, 1.0 / d ** 0.5, level.n_text)
    ws = dfp.attention_workspace(B, H, n, N, d)
    text = None
    if fresh and level.n_text:   # the text rows are fresh in every call
        kt, vt = x.text_rows()
        text = (G.up(kt, kind), G.up(np.swapaxes(vt, -1, -2), kind), 0)
    for m in range(level.P):
        kf, vf = x.fresh_rows(m)
        q = G.up(x.q_patch(m), kind)
        o = torch.empty_like(q)
        if fresh:
            ranges = [(G.up(kf, kind), G.up(np.swapaxes(vf, -1, -2), kind), level.row0(m))]
            dfp.patch_attention_fresh(o, q, k_buf, v_buf, ([text] if text else []) + ranges,
                                      True, 1.0 / d ** 0.5, ws)
        else:
            dfp.kv_scatter(k_buf, v_buf, G.up(kf, kind), G.up(vf, kind), level.row0(m))
            dfp.patch_attention(o, q, k_buf, v_buf, 1.0 / d ** 0.5, ws)
        torch.cuda.synchronize()
        got = G.down(o)[sl]
        err = np.abs(got - want[m]).max()
        if kind == "f32":
            assert err <= F32_MAX_ABS, f"{name} patch {m}: max-abs {err}"
        else:
            rl = G.rel_l2(got, want[m])
            assert rl <= BF16_REL_L2 and err <= BF16_MAX_ABS, \
                f"{name} patch {m}: relL2 {rl} max-abs {err}"
