"""Host-side checks of libdfp.so (no GPU work): the library loads, exports
every function include/dfp.h declares, validates arguments before launching
anything, and its host helpers (schedule, timesteps, folded sampler
coefficients) agree with the oracle."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from patch_attention_cfg_amd import dfp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "dfp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dfp_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dfp.LIB_PATH):
        from patch_attention_cfg_amd import build
        build.build_library()
    return dfp.lib()


def test_exports_every_declared_symbol(L):
    names = _header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(dfp.SIGNATURES)


def test_status_strings(L):
    for code in (0, 1, 2, 3):
        assert dfp.status_string(code).startswith("DFP_")
    assert "unknown" in dfp.status_string(99)


def test_v_ld(L):
    assert dfp.v_ld(4096, dfp.BF16) == 4096
    assert dfp.v_ld(13, dfp.BF16) == 16
    assert dfp.v_ld(13, dfp.F32) == 16
    assert dfp.v_ld(1, dfp.F32) == 4
    assert dfp.v_ld(0, dfp.BF16) == 0
    assert dfp.v_ld(10, 7) == 0


# ---------------------------------------------------- validation, no launch
NULL = None
S0 = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("args,expect", [
    # k pair half null
    ((FAKE, NULL, NULL, NULL, 2, 2, 64, 64, 0, 8, dfp.BF16), dfp.ERR_INVALID_ARG),
    # row0 + n > N_buf
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 60, 8, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, -1, 8, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 0, 2, 64, 64, 0, 8, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 0, -1, dfp.BF16), dfp.ERR_INVALID_ARG),
    # d not a multiple of 16 bytes
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 12, 0, 8, dfp.BF16), dfp.ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 0, 8, 5), dfp.ERR_UNSUPPORTED),
    # misaligned pointer
    ((ctypes.c_void_p(0x100002), FAKE, FAKE, FAKE, 2, 2, 64, 64, 0, 8, dfp.BF16),
     dfp.ERR_INVALID_ARG),
    # n == 0 is a no-op
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 64, 3, 0, dfp.BF16), dfp.OK),
    ((FAKE, FAKE, NULL, NULL, 2, 2, 64, 64, 64, 0, dfp.BF16), dfp.OK),
])
def test_scatter_validation(L, args, expect):
    assert L.dfp_kv_scatter(*args, S0) == expect


@pytest.mark.parametrize("strides,expect", [
    ((2 * 64 * 16, 64, 2 * 64), dfp.ERR_INVALID_ARG),   # nothing wrong but a NULL v_new below
    ((4, 64, 128), dfp.ERR_INVALID_ARG),                # batch stride not 16-byte rows (bf16: x8)
    ((2048, 60, 128), dfp.ERR_INVALID_ARG),             # head stride not a multiple of 8
    ((2048, 64, 32), dfp.ERR_INVALID_ARG),              # rows overlap (stride_n < d)
    ((-2048, 64, 128), dfp.ERR_INVALID_ARG),            # negative
])
def test_strided_scatter_validation(L, strides, expect):
    v_new = NULL if strides == (2 * 64 * 16, 64, 2 * 64) else FAKE
    assert L.dfp_kv_scatter_strided(FAKE, FAKE, FAKE, v_new, 2, 2, 64, 64, 0, 16, *strides,
                                    dfp.BF16, S0) == expect
    # empty landings are no-ops whatever the strides
    assert L.dfp_kv_scatter_strided(NULL, NULL, NULL, NULL, 2, 2, 64, 64, 0, 0, 1, 1, 1,
                                    dfp.BF16, S0) == dfp.OK


@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, FAKE, 2, 2, 16, 64, 64, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, NULL, 2, 2, 16, 64, 64, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 16, 0, 64, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, -1, 64, 64, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 16, 64, 64, 0.0, dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 16, 64, 64, float("nan"), dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 16, 64, 64, float("inf"), dfp.BF16), dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 16, 64, 96, 0.125, dfp.BF16), dfp.ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 16, 64, 64, 0.125, 4), dfp.ERR_UNSUPPORTED),
    ((FAKE, FAKE, ctypes.c_void_p(0x100008), FAKE, 2, 2, 16, 64, 64, 0.125, dfp.BF16),
     dfp.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, 2, 2, 0, 64, 64, 0.125, dfp.BF16), dfp.OK),
    ((NULL, NULL, NULL, NULL, 2, 2, 0, 64, 64, 0.125, dfp.BF16), dfp.OK),
])
def test_attention_validation(L, args, expect):
    assert L.dfp_patch_attention(*args, NULL, 0, S0) == expect


# Sizes past the 32-bit offsets and grid sizes the kernels use are refused
# before anything is enqueued (so these run without a GPU).
@pytest.mark.parametrize("dt", [dfp.BF16, dfp.F32])
@pytest.mark.parametrize("B,H,n_q,N_kv,d,bf16_only", [
    (1, 1, 64, 1 << 24, 64, True),          # one head's K is 2 GiB of bf16
    (1, 1, 64, 1 << 23, 128, True),
    (1 << 16, 1 << 15, 64, 64, 64, False),  # 2^31 (batch, head) pairs
    (1 << 15, 1 << 15, 256, 64, 64, False),  # 2^31 workgroups
])
def test_attention_refuses_sizes_past_its_limits(L, dt, B, H, n_q, N_kv, d, bf16_only):
    if bf16_only and dt != dfp.BF16:
        pytest.skip("the fp32 path addresses K and V with 64-bit offsets")
    assert L.dfp_patch_attention(FAKE, FAKE, FAKE, FAKE, B, H, n_q, N_kv, d, 0.125, dt,
                                 NULL, 0, S0) == dfp.ERR_UNSUPPORTED


def test_fresh_attention_refuses_sizes_past_its_limits(L):
    big = dfp.FreshRows(FAKE, FAKE, 0, 64)
    arr = (dfp.FreshRows * 1)(big)
    assert L.dfp_patch_attention_fresh(FAKE, FAKE, FAKE, FAKE, arr, 1, 1, 1, 64, 1 << 24, 64, 1,
                                       0.125, dfp.BF16, NULL, 0, S0) == dfp.ERR_UNSUPPORTED
    assert L.dfp_patch_attention_fresh(FAKE, FAKE, FAKE, FAKE, arr, 1, 1 << 16, 1 << 15, 64, 64,
                                       64, 1, 0.125, dfp.BF16, NULL, 0, S0) == dfp.ERR_UNSUPPORTED


def test_scatter_refuses_grids_past_its_limits(L):
    # 2^30 (batch, head) pairs of two 64-row V^T tiles: 2^31 workgroups
    assert L.dfp_kv_scatter(FAKE, FAKE, FAKE, FAKE, 1 << 15, 1 << 15, 128, 64, 0, 128, dfp.BF16,
                            S0) == dfp.ERR_UNSUPPORTED


MIS = ctypes.c_void_p(0x100008)   # 8-byte aligned only


def _ranges(*spec):
    """A host dfp_fresh_rows array; spec items are (k, v_t, row0, n)."""
    arr = (dfp.FreshRows * max(len(spec), 1))()
    for i, (k, vt, row0, n) in enumerate(spec):
        arr[i] = dfp.FreshRows(k.value if k else None, vt.value if vt else None, row0, n)
    return ctypes.cast(arr, ctypes.c_void_p), arr


R_OK = (FAKE, FAKE, 64, 128)


# (ranges, n_fresh, B, H, n_q, N_kv, d, land, scale, dt, buffers/outputs present)
@pytest.mark.parametrize("ranges,n_fresh,shape,expect", [
    # a range outside the buffer, empty or negative
    ([(FAKE, FAKE, 192, 128)], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ([(FAKE, FAKE, -64, 128)], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ([(FAKE, FAKE, 0, 0)], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    # not whole 64-key tiles
    ([(FAKE, FAKE, 32, 128)], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_UNSUPPORTED),
    ([(FAKE, FAKE, 64, 100)], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_UNSUPPORTED),
    # bf16 only; d 64 or 128
    ([R_OK], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.F32), dfp.ERR_UNSUPPORTED),
    ([R_OK], 1, (2, 2, 16, 256, 96, 1, 0.125, dfp.BF16), dfp.ERR_UNSUPPORTED),
    # range count: none, more than two; overlapping ranges
    ([], 0, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ([R_OK, (FAKE, FAKE, 0, 64), (FAKE, FAKE, 192, 64)], 3, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16),
     dfp.ERR_UNSUPPORTED),
    ([R_OK, (FAKE, FAKE, 128, 128)], 2, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16),
     dfp.ERR_INVALID_ARG),
    ([(FAKE, FAKE, 128, 128), (FAKE, FAKE, 0, 192)], 2, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16),
     dfp.ERR_INVALID_ARG),
    # null or misaligned fresh pointers, bad scale, bad sizes
    ([(NULL, FAKE, 64, 128)], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ([(FAKE, MIS, 64, 128)], 1, (2, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ([R_OK], 1, (2, 2, 16, 256, 64, 1, float("nan"), dfp.BF16), dfp.ERR_INVALID_ARG),
    ([R_OK], 1, (0, 2, 16, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    ([R_OK], 1, (2, 2, -1, 256, 64, 1, 0.125, dfp.BF16), dfp.ERR_INVALID_ARG),
    # no queries and no landing: nothing to do
    ([R_OK], 1, (2, 2, 0, 256, 64, 0, 0.125, dfp.BF16), dfp.OK),
])
def test_fresh_attention_validation(L, ranges, n_fresh, shape, expect):
    ptr, keep = _ranges(*ranges)
    B, H, n_q, N_kv, d, land, scale, dt = shape
    out = (FAKE, FAKE, FAKE, FAKE) if n_q else (NULL, NULL, FAKE, FAKE)
    assert L.dfp_patch_attention_fresh(*out, ptr, n_fresh, B, H, n_q, N_kv, d, land, scale, dt,
                                       NULL, 0, S0) == expect


def test_fresh_attention_null_range_array(L):
    assert L.dfp_patch_attention_fresh(FAKE, FAKE, FAKE, FAKE, NULL, 1, 2, 2, 16, 256, 64, 1,
                                       0.125, dfp.BF16, NULL, 0, S0) == dfp.ERR_INVALID_ARG


def test_cfg_step_validation(L):
    ws_need = dfp.workspace_bytes(dfp.OP_CFG_STEP, 4096, 1)
    assert ws_need >= 16   # one fp64 pair per workgroup
    cases = [
        ((NULL, FAKE, FAKE, 4096, 1, 7.5, 1.0, -0.5, NULL, NULL, 0), dfp.ERR_INVALID_ARG),
        ((FAKE, NULL, FAKE, 4096, 1, 7.5, 1.0, -0.5, NULL, NULL, 0), dfp.ERR_INVALID_ARG),
        ((FAKE, FAKE, FAKE, 0, 1, 7.5, 1.0, -0.5, NULL, NULL, 0), dfp.ERR_INVALID_ARG),
        ((FAKE, FAKE, FAKE, 4096, 0, 7.5, 1.0, -0.5, NULL, NULL, 0), dfp.ERR_INVALID_ARG),
        ((FAKE, FAKE, FAKE, 4096, 1, float("nan"), 1.0, -0.5, NULL, NULL, 0),
         dfp.ERR_INVALID_ARG),
        ((FAKE, FAKE, FAKE, 4096, 1, 7.5, float("inf"), -0.5, NULL, NULL, 0),
         dfp.ERR_INVALID_ARG),
        # reduction requested without (enough) workspace
        ((FAKE, FAKE, FAKE, 4096, 1, 7.5, 1.0, -0.5, FAKE, NULL, 0), dfp.ERR_INVALID_ARG),
        ((FAKE, FAKE, FAKE, 4096, 1, 7.5, 1.0, -0.5, FAKE, FAKE, ws_need - 1),
         dfp.ERR_INVALID_ARG),
    ]
    for args, expect in cases:
        assert L.dfp_cfg_step(*args, S0) == expect, args
    assert L.dfp_relmae(FAKE, FAKE, 4096, 1, NULL, FAKE, ws_need, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_relmae(FAKE, FAKE, 4096, 1, FAKE, NULL, 0, S0) == dfp.ERR_INVALID_ARG


def test_philox_entry_validation(L):
    ws_need = dfp.workspace_bytes(dfp.OP_CFG_STEP, 4096, 1)
    base = (FAKE, FAKE, FAKE, 4096, 1, 7.5, 1.0, -0.5, 0.1, 5, 3)
    assert L.dfp_cfg_step_philox(*base, FAKE, NULL, 0, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_cfg_step_philox(*base[:8], float("nan"), 5, 3, NULL, NULL, 0,
                                 S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_cfg_step_philox(NULL, *base[1:], NULL, NULL, 0, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_cfg_step_philox(*base, FAKE, FAKE, ws_need - 1, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_philox_normal(NULL, 16, 1, 0, 0, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_philox_normal(FAKE, 0, 1, 0, 0, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_philox_normal(FAKE, 16, 0, 0, 0, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_philox4x64_10(NULL, 4, 0, 0, 0, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_philox4x64_10(FAKE, -1, 0, 0, 0, S0) == dfp.ERR_INVALID_ARG
    assert L.dfp_philox4x64_10(NULL, 0, 0, 0, 0, S0) == dfp.OK   # nothing to do


def test_workspace_sizes_grow_with_batch(L):
    a = dfp.workspace_bytes(dfp.OP_CFG_STEP, 921600, 1)
    b = dfp.workspace_bytes(dfp.OP_CFG_STEP, 921600, 2)
    assert b == 2 * a and a > 256
    assert dfp.workspace_bytes(dfp.OP_RELMAE, 921600, 1) == a
    assert dfp.workspace_bytes(99) == 0


def test_group_norm_validation(L):
    """dfp_displaced_group_norm rejects bad arguments before any launch."""
    X = ctypes.c_void_p(0x200000)
    Y = ctypes.c_void_p(0x400000)
    ST = ctypes.c_void_p(0x600000)
    f = L.dfp_displaced_group_norm

    def call(y=Y, x=X, st=ST, B=2, C=8, G=4, n=16, P=3, p=1, eps=1e-5):
        return f(y, x, st, NULL, NULL, B, C, G, n, P, p, eps, 1, NULL, 0, S0)

    E = dfp.ERR_INVALID_ARG
    assert call(y=NULL) == E
    assert call(x=NULL) == E
    assert call(st=NULL) == E
    assert call(st=ctypes.c_void_p(0x600004)) == E     # stats not 8-byte aligned
    assert call(y=ctypes.c_void_p(0x200004)) == E      # y partly overlaps x
    assert call(C=10) == E                             # C not a multiple of G
    assert call(G=0) == E
    assert call(B=0) == E
    assert call(n=0) == E
    assert call(P=0) == E
    assert call(p=3) == E
    assert call(p=-1) == E
    assert call(eps=-1.0) == E
    assert call(eps=float("nan")) == E
    assert call(eps=float("inf")) == E
    assert call(B=65536) == dfp.ERR_UNSUPPORTED
    # groups of up to 64 Ki floats (n % 4 == 0) need none; longer ones one
    # fp64 pair per 4 Ki-float chunk of every group
    ws = L.dfp_group_norm_workspace_bytes
    assert ws(2, 320, 32, 4096) == 0                 # 40 Ki floats per group
    assert ws(2, 320, 32, 4097) == 64 * 11 * 16      # n % 4 != 0: chunked
    assert ws(2, 320, 32, 28800) == 64 * 71 * 16     # 281.25 Ki floats: 71 chunks
    assert ws(2, 320, 30, 28800) == 0              # C not a multiple of G
    assert ws(0, 320, 32, 28800) == 0


def test_attention_plan(L, monkeypatch):
    """The bf16 launch plan: two key groups only for d=64 grids far too small
    to fill the GPU, a key-range split only with a workspace, and the
    environment overrides honoured."""
    monkeypatch.delenv("DFP_ATTN_KS", raising=False)
    monkeypatch.delenv("DFP_ATTN_SPLITS", raising=False)
    # SDXL-1024 32x32 level: 40 (batch, head) pairs x 256 queries
    assert dfp.attention_plan(2, 20, 256, 1024, 64) == (2, 1, 160)
    # two key groups need no workspace
    assert dfp.attention_plan(2, 20, 256, 1024, 64, with_workspace=False) == (2, 1, 160)
    # SDXL-1024 64x64 level: one key group, key range split across workgroups
    ks, sp, wg = dfp.attention_plan(2, 10, 1024, 4096, 64)
    assert ks == 1 and sp > 1 and wg == 160 * sp
    assert dfp.attention_plan(2, 10, 1024, 4096, 64, with_workspace=False) == (1, 1, 160)
    # grids that fill the GPU, d=128, a single key tile: one key group
    assert dfp.attention_plan(2, 10, 2048, 16384, 64)[0] == 1
    assert dfp.attention_plan(2, 20, 256, 1024, 128)[0] == 1
    assert dfp.attention_plan(1, 1, 64, 64, 64) == (1, 1, 1)
    monkeypatch.setenv("DFP_ATTN_KS", "1")
    assert dfp.attention_plan(2, 20, 256, 1024, 64)[0] == 1
    monkeypatch.setenv("DFP_ATTN_KS", "2")
    assert dfp.attention_plan(2, 10, 2048, 16384, 64) == (2, 1, 20 * 32)
    monkeypatch.delenv("DFP_ATTN_KS")
    monkeypatch.setenv("DFP_ATTN_SPLITS", "4")
    assert dfp.attention_plan(2, 20, 256, 1024, 64) == (1, 4, 320)
    out = ctypes.c_int(7)
    assert L.dfp_attention_plan(0, 1, 1, 1, 64, 1, ctypes.byref(out), None, None) == \
        dfp.ERR_INVALID_ARG
    assert L.dfp_attention_plan(1, 1, 0, 1, 64, 1, None, None, None) == dfp.ERR_INVALID_ARG
    assert L.dfp_attention_plan(1, 1, 1, 1, 96, 1, None, None, None) == dfp.ERR_UNSUPPORTED
    assert out.value == 7


# ------------------------------------------------- host helpers vs oracle
def test_schedule_matches_oracle(L):
    ours = dfp.scaled_linear_abar(1000, 0.00085, 0.012)
    ref = oracle.alphas_cumprod(oracle.scaled_linear_betas(1000, 0.00085, 0.012))
    np.testing.assert_allclose(ours, ref, rtol=1e-14, atol=0)


@pytest.mark.parametrize("S", [1, 10, 28, 50, 100, 999])
def test_timesteps_match_oracle(L, S):
    np.testing.assert_array_equal(dfp.ddim_timesteps(1000, S), oracle.ddim_timesteps(1000, S))


@pytest.mark.parametrize("steps", [10, 50])
def test_folded_ddim_coefficients_reproduce_two_stage_step(L, steps):
    # x' = c_x x + c_e g must equal the oracle's x0-estimate form at every step
    sch = oracle.DDIMSchedule(steps)
    r = np.random.Generator(np.random.PCG64(steps))
    x = r.standard_normal(256)
    g = r.standard_normal(256)
    for i in range(steps):
        at, ap, last = sch.step_args(i)
        cx, ce = dfp.ddim_coeffs(at, ap)
        want = oracle.ddim_step(x, g, at, ap, last)
        np.testing.assert_allclose(cx * x + ce * g, want, rtol=1e-12, atol=1e-12)


def test_coefficient_edge_cases(L):
    cx, ce = dfp.ddim_coeffs(0.5, 0.5)
    assert abs(cx - 1) < 1e-15 and abs(ce) < 1e-15
    cx, ce = dfp.euler_coeffs(1.0, 27 / 28)
    assert cx == 1.0 and abs(ce + 1 / 28) < 1e-16
    with pytest.raises(dfp.DFPError):
        dfp.ddim_coeffs(0.0, 0.5)
    with pytest.raises(dfp.DFPError):
        dfp.ddim_coeffs(0.5, 1.5)
    with pytest.raises(dfp.DFPError):
        dfp.euler_coeffs(math.nan, 0.0)
    with pytest.raises(dfp.DFPError):
        dfp.scaled_linear_abar(1, 0.1, 0.2)


@pytest.mark.parametrize("eta", [0.0, 0.5, 1.0])
def test_folded_eta_coefficients_reproduce_two_stage_step(L, eta):
    # x' = c_x x + c_e g + c_z z must equal the oracle's literal eta step
    sch = oracle.DDIMSchedule(50)
    r = np.random.Generator(np.random.PCG64(77))
    x, g, z = (r.standard_normal(256) for _ in range(3))
    for i in range(50):
        at, ap, last = sch.step_args(i)
        cx, ce, cz = dfp.ddim_eta_coeffs(at, ap, eta)
        want = oracle.ddim_step_eta(x, g, z, at, ap, eta, last)
        np.testing.assert_allclose(cx * x + ce * g + cz * z, want, rtol=1e-12, atol=1e-12)


def test_eta_coefficient_edges(L):
    assert dfp.ddim_eta_coeffs(0.3, 0.6, 0.0) == pytest.approx(dfp.ddim_coeffs(0.3, 0.6) + (0.0,),
                                                               abs=1e-15)
    assert dfp.ddim_eta_coeffs(0.3, 1.0, 1.0)[2] == 0.0          # last step: no noise
    with pytest.raises(dfp.DFPError):
        dfp.ddim_eta_coeffs(0.3, 0.6, 3.0)                       # sigma^2 > 1 - abar_prev
    with pytest.raises(dfp.DFPError):
        dfp.ddim_eta_coeffs(0.6, 0.3, 0.5)                       # abar_t > abar_prev
    with pytest.raises(dfp.DFPError):
        dfp.ddim_eta_coeffs(0.3, 0.6, -0.1)


def test_switch_points_match_oracle(L):
    """The library's switch rule against the oracle's on fp32 series: clean
    U curves, plateaus, noisy curves and strictly monotone ones."""
    rng = np.random.Generator(np.random.PCG64(31))
    series = []
    t = np.arange(50)
    series.append(((t - 23) ** 2 / 50 + 0.1))
    series.append(np.concatenate([np.linspace(1, 0.1, 11), np.full(20, 0.1),
                                  [0.08, 0.06, 0.05, 0.07, 0.1, 0.2]]))
    series.append(np.linspace(1, 0, 28))
    for _ in range(100):
        S = int(rng.integers(1, 60))
        base = np.abs(np.linspace(-1, 1, S)) + 0.3
        series.append(base + 0.05 * rng.standard_normal(S))
    for M in series:
        M = np.asarray(M, dtype=np.float32)
        for Lw, g, k in ((1, 0.01, 5), (3, 0.02, 5), (5, 0.005, 10)):
            assert dfp.switch_points(M, Lw, g, k) == oracle.switch_points(M, Lw, g, k)


def test_switch_points_validation(L):
    with pytest.raises(dfp.DFPError):
        dfp.switch_points([], 1, 0.1)
    with pytest.raises(dfp.DFPError):
        dfp.switch_points([0.3, 0.2], 0, 0.1)
    with pytest.raises(dfp.DFPError):
        dfp.switch_points([0.3, float("nan")], 1, 0.1)
