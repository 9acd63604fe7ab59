"""fp64 CPU oracle: the definition of what the patch-attention and guided
sampler step compute, used to check the HIP library.

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
``patch_attention_cfg_amd``; neither imports the other.  The arithmetic lives
in ``dfp_oracle.c`` (plain C, double precision); this module only marshals
numpy arrays into it and strings the per-step functions into a sampler run in
the pages' order.

Citations use the page titles (see the header of ``dfp_oracle.c``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dfp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdfp_oracle.so")

_lib = None


def build_oracle() -> str:
    """Compile the C oracle with gcc (-O2, OpenMP) into oracle/libdfp_oracle.so."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build_oracle()
    lib = ctypes.CDLL(_LIB_PATH)
    D = ctypes.POINTER(ctypes.c_double)
    I = ctypes.POINTER(ctypes.c_int64)
    U = ctypes.POINTER(ctypes.c_uint64)
    u64 = ctypes.c_uint64
    i64, dbl, cint = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    sigs = {
        "oracle_effective_kv": (None, [D, D, i64, i64, i64, i64, i64]),
        "oracle_attention": (cint, [D, D, D, i64, i64, i64, i64, dbl, D]),
        "oracle_attention_rows": (cint, [D, D, D, i64, i64, i64, i64, dbl, I, I, i64, D]),
        "oracle_attention_probs": (None, [D, D, i64, i64, i64, i64, dbl, D]),
        "oracle_scaled_linear_betas": (None, [i64, dbl, dbl, D]),
        "oracle_alphas_cumprod": (None, [i64, D, D]),
        "oracle_ddim_timesteps": (None, [i64, i64, I]),
        "oracle_cfg_combine": (None, [D, D, i64, dbl, D]),
        "oracle_ddim_sigma": (dbl, [dbl, dbl, dbl]),
        "oracle_ddim_update": (None, [D, D, D, i64, dbl, dbl, dbl]),
        "oracle_philox4x64_10": (None, [U, U, U]),
        "oracle_philox_normals": (None, [D, i64, u64, u64, u64]),
        "oracle_set_threads": (None, [cint]),
        "oracle_switch_points": (cint, [D, i64, i64, dbl, i64, I, I]),
        "oracle_flow_sigmas": (None, [i64, D]),
        "oracle_euler_step": (None, [D, D, i64, dbl, dbl]),
        "oracle_relmae": (dbl, [D, D, i64]),
        "oracle_num_threads": (cint, []),
        "oracle_displaced_group_norm": (None, [D, D, D, D, i64, i64, i64, i64, i64, i64, dbl,
                                               D, D]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _pd(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _pi(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def num_threads() -> int:
    """Threads the oracle's parallel loops use (OpenMP)."""
    return int(_load().oracle_num_threads())


# --------------------------------------------------------------------------
# Displaced patch attention
# --------------------------------------------------------------------------
def effective_kv(stale, fresh, row0: int) -> np.ndarray:
    """The K (or V) the patch attends over: the stale buffer [..., N, d] with
    rows [row0, row0+n) replaced by the fresh patch rows [..., n, d]."""
    stale = _f64(stale)
    fresh = _f64(fresh)
    *lead, N, d = stale.shape
    n = fresh.shape[-2]
    if tuple(fresh.shape[:-2]) != tuple(lead) or fresh.shape[-1] != d:
        raise ValueError("fresh and stale disagree in leading dims or d")
    if row0 < 0 or row0 + n > N:
        raise ValueError("patch rows fall outside the buffer")
    out = stale.copy()
    BH = int(np.prod(lead)) if lead else 1
    _load().oracle_effective_kv(_pd(out), _pd(fresh), BH, N, d, row0, n)
    return out


def attention(q, k, v, scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v per (batch, head); q [..., nq, d], k/v [..., N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, nq, d = q.shape
    Nkv = k.shape[-2]
    if k.shape != v.shape or k.shape[-1] != d or tuple(k.shape[:-2]) != tuple(lead):
        raise ValueError("q/k/v shapes disagree")
    BH = int(np.prod(lead)) if lead else 1
    o = np.empty_like(q)
    rc = _load().oracle_attention(_pd(q), _pd(k), _pd(v), BH, nq, Nkv, d, float(scale), _pd(o))
    if rc != 0:
        raise MemoryError("oracle_attention could not allocate its score row")
    return o


def attention_rows(q, k, v, scale: float, rows_bh, rows_i) -> np.ndarray:
    """Attention output for selected rows only: row r is (flattened batch*head
    rows_bh[r], query rows_i[r]).  Returns [nrows, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, nq, d = q.shape
    Nkv = k.shape[-2]
    BH = int(np.prod(lead)) if lead else 1
    rb = np.ascontiguousarray(np.asarray(rows_bh, dtype=np.int64))
    ri = np.ascontiguousarray(np.asarray(rows_i, dtype=np.int64))
    if rb.shape != ri.shape or rb.ndim != 1:
        raise ValueError("row index arrays must be 1-D and equal length")
    if rb.size and (rb.min() < 0 or rb.max() >= BH or ri.min() < 0 or ri.max() >= nq):
        raise ValueError("row index out of range")
    o = np.empty((rb.size, d), dtype=np.float64)
    rc = _load().oracle_attention_rows(_pd(q), _pd(k), _pd(v), BH, nq, Nkv, d,
                                       float(scale), _pi(rb), _pi(ri), rb.size, _pd(o))
    if rc != 0:
        raise MemoryError("oracle_attention_rows could not allocate its score row")
    return o


def attention_probs(q, k, scale: float) -> np.ndarray:
    """The softmax probability matrix [..., nq, Nkv] (tiny inputs only)."""
    q, k = _f64(q), _f64(k)
    *lead, nq, d = q.shape
    Nkv = k.shape[-2]
    BH = int(np.prod(lead)) if lead else 1
    p = np.empty(tuple(lead) + (nq, Nkv), dtype=np.float64)
    _load().oracle_attention_probs(_pd(q), _pd(k), BH, nq, Nkv, d, float(scale), _pd(p))
    return p


def patch_attention(q_patch, k_stale, v_stale, k_fresh_rows, v_fresh_rows,
                    row0: int, scale: float, extra_fresh=()):
    """One patch's attention over the displaced buffer.  The fresh patch rows
    land at row0; ``extra_fresh`` is a sequence of (k_rows, v_rows, row) for
    other always-fresh ranges (a DiT's text tokens)."""
    k_eff = effective_kv(k_stale, k_fresh_rows, row0)
    v_eff = effective_kv(v_stale, v_fresh_rows, row0)
    for kr, vr, r0 in extra_fresh:
        k_eff = effective_kv(k_eff, kr, r0)
        v_eff = effective_kv(v_eff, vr, r0)
    return attention(q_patch, k_eff, v_eff, scale)


def patch_sweep(q, k_stale, v_stale, k_fresh, v_fresh, P: int, scale: float, n_text: int = 0):
    """One device running every patch of a layer in order ("xDiT: an
    Inference Engine for Diffusion Transformers (DiTs) with Massive
    Parallelism", 三.2 PipeFusion: M non-overlapping patches processed one
    after another, each reusing the previous step's activations for the
    patches it has not reached): patch m lands its fresh K/V, then attends
    over fresh rows for patches 0..m and the previous step's rows for patches
    m+1..P-1; always-fresh text rows [0, n_text) land first.

    q [..., N_img, d] holds every image token's query; k/v fresh and stale
    [..., n_text + N_img, d].  Returns the P patch outputs [..., N_img/P, d]."""
    N_img = q.shape[-2]
    if P <= 0 or N_img % P:
        raise ValueError("P must divide the image tokens")
    n = N_img // P
    k_eff, v_eff = _f64(k_stale), _f64(v_stale)
    if n_text:
        k_eff = effective_kv(k_eff, _f64(k_fresh)[..., :n_text, :], 0)
        v_eff = effective_kv(v_eff, _f64(v_fresh)[..., :n_text, :], 0)
    outs = []
    for m in range(P):
        r0 = n_text + m * n
        k_eff = effective_kv(k_eff, _f64(k_fresh)[..., r0:r0 + n, :], r0)
        v_eff = effective_kv(v_eff, _f64(v_fresh)[..., r0:r0 + n, :], r0)
        outs.append(attention(_f64(q)[..., m * n:(m + 1) * n, :], k_eff, v_eff, scale))
    return outs


# --------------------------------------------------------------------------
# Schedules, guidance, samplers, rel-MAE
# --------------------------------------------------------------------------
def scaled_linear_betas(T: int = 1000, beta_start: float = 0.00085,
                        beta_end: float = 0.012) -> np.ndarray:
    b = np.empty(T, dtype=np.float64)
    _load().oracle_scaled_linear_betas(T, beta_start, beta_end, _pd(b))
    return b


def alphas_cumprod(betas) -> np.ndarray:
    betas = _f64(betas)
    a = np.empty_like(betas)
    _load().oracle_alphas_cumprod(betas.size, _pd(betas), _pd(a))
    return a


def ddim_timesteps(T: int, S: int) -> np.ndarray:
    ts = np.empty(S, dtype=np.int64)
    _load().oracle_ddim_timesteps(T, S, _pi(ts))
    return ts


def flow_sigmas(S: int) -> np.ndarray:
    s = np.empty(S + 1, dtype=np.float64)
    _load().oracle_flow_sigmas(S, _pd(s))
    return s


def cfg_combine(g_c, g_u, w: float) -> np.ndarray:
    g_c, g_u = _f64(g_c), _f64(g_u)
    if g_c.shape != g_u.shape:
        raise ValueError("g_c and g_u shapes differ")
    g = np.empty_like(g_c)
    _load().oracle_cfg_combine(_pd(g_c), _pd(g_u), g_c.size, float(w), _pd(g))
    return g


def ddim_sigma(abar_t: float, abar_prev: float, eta: float) -> float:
    """Noise scale of a DDIM step with parameter eta."""
    return float(_load().oracle_ddim_sigma(float(abar_t), float(abar_prev), float(eta)))


def _ddim(x, eps, z, abar_t, abar_prev, eta, last):
    x = _f64(x).copy()
    eps = _f64(eps)
    if eps.shape != x.shape or (z is not None and z.shape != x.shape):
        raise ValueError("x, eps and z shapes differ")
    a_prev = 1.0 if last else float(abar_prev)   # the last step returns the x0 estimate
    sigma = ddim_sigma(abar_t, a_prev, eta) if eta else 0.0
    _load().oracle_ddim_update(_pd(x), _pd(eps), None if z is None else _pd(_f64(z)), x.size,
                               float(abar_t), a_prev, sigma)
    return x


def ddim_step(x, eps, abar_t: float, abar_prev: float, last: bool) -> np.ndarray:
    """DDIM with eta = 0: x_t -> the previous sampled timestep (abar_prev),
    or -> the x0 estimate on the last step."""
    return _ddim(x, eps, None, abar_t, abar_prev, 0.0, last)


def ddim_step_eta(x, eps, z, abar_t: float, abar_prev: float, eta: float,
                  last: bool) -> np.ndarray:
    """DDIM with noise scale eta and the standard-normal draw z."""
    return _ddim(x, eps, _f64(z), abar_t, abar_prev, eta, last)


def philox4x64_10(counter, key) -> np.ndarray:
    """One Philox4x64-10 block: counter (4 uint64), key (2 uint64) -> 4 uint64."""
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint64))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64))
    if c.shape != (4,) or k.shape != (2,):
        raise ValueError("counter must hold 4 words and key 2")
    out = np.empty(4, dtype=np.uint64)
    P = ctypes.POINTER(ctypes.c_uint64)
    _load().oracle_philox4x64_10(c.ctypes.data_as(P), k.ctypes.data_as(P), out.ctypes.data_as(P))
    return out


def philox_normals(n: int, seed: int, step: int, image: int = 0) -> np.ndarray:
    """The standard-normal draw z[0..n) of one image at one sampler step
    (Philox4x64-10 + Box-Muller; mapping in dfp_oracle.c)."""
    z = np.empty(int(n), dtype=np.float64)
    _load().oracle_philox_normals(_pd(z), int(n), int(seed) & (2**64 - 1),
                                  int(step) & (2**64 - 1), int(image) & (2**64 - 1))
    return z


def set_threads(threads: int) -> None:
    """Threads the oracle's parallel loops use from now on (timing only)."""
    _load().oracle_set_threads(int(threads))


def euler_step(x, v, sigma: float, sigma_next: float) -> np.ndarray:
    x = _f64(x).copy()
    v = _f64(v)
    _load().oracle_euler_step(_pd(x), _pd(v), x.size, float(sigma), float(sigma_next))
    return x


def relmae(g_c, g_u) -> float:
    g_c, g_u = _f64(g_c), _f64(g_u)
    if g_c.shape != g_u.shape:
        raise ValueError("g_c and g_u shapes differ")
    return float(_load().oracle_relmae(_pd(g_c), _pd(g_u), g_c.size))


class DDIMSchedule:
    """DDIM (eta = 0) over a 1000-step scaled-linear schedule, walked as the
    DDIM listing of the AIGC speed-up page's section 3 walks it: reversed
    timesteps; on every step but the last the target is the previous sampled
    timestep, on the last the x0 estimate is returned."""

    def __init__(self, steps: int, T: int = 1000, beta_start: float = 0.00085,
                 beta_end: float = 0.012):
        self.abar = alphas_cumprod(scaled_linear_betas(T, beta_start, beta_end))
        self.ts = ddim_timesteps(T, steps)
        self.steps = steps

    def step_args(self, i: int):
        """(abar_t, abar_prev, last) for the i-th step (i = 0 is the noisiest)."""
        S = self.steps
        t = int(self.ts[S - 1 - i])
        last = i == S - 1
        abar_prev = 1.0 if last else float(self.abar[int(self.ts[S - 2 - i])])
        return float(self.abar[t]), abar_prev, last

    def step(self, x, g_c, g_u, w: float, i: int):
        """One guided step: returns (x_next, rel-MAE of this step's pair)."""
        r = relmae(g_c, g_u)
        g = cfg_combine(g_c, g_u, w)
        abar_t, abar_prev, last = self.step_args(i)
        return ddim_step(x, g, abar_t, abar_prev, last), r

    def step_eta(self, x, g_c, g_u, w: float, i: int, eta: float, z):
        """One guided step of DDIM with noise scale eta and standard-normal
        draw z: returns (x_next, rel-MAE of this step's pair)."""
        r = relmae(g_c, g_u)
        g = cfg_combine(g_c, g_u, w)
        abar_t, abar_prev, last = self.step_args(i)
        return ddim_step_eta(x, g, z, abar_t, abar_prev, eta, last), r


class EulerSchedule:
    """Flow-matching Euler over sigma_i = 1 - i/S (S steps from 1 to 0)."""

    def __init__(self, steps: int):
        self.sigmas = flow_sigmas(steps)
        self.steps = steps

    def step(self, x, v_c, v_u, w: float, i: int):
        r = relmae(v_c, v_u)
        g = cfg_combine(v_c, v_u, w)
        return euler_step(x, g, float(self.sigmas[i]), float(self.sigmas[i + 1])), r


def switch_points(relmae_series, L: int, g_slope: float, k: int = 5):
    """(tau1, tau2) of the three-phase schedule from a rel-MAE series
    ("Accelerating Diffusion via Hybrid Data-Pipeline Parallelism Based on
    Conditional Guidance Scheduling", 关键设计 3); steps are indices into the
    series, 0 = the first denoising step."""
    M = _f64(relmae_series).ravel()
    t1 = np.zeros(1, dtype=np.int64)
    t2 = np.zeros(1, dtype=np.int64)
    if _load().oracle_switch_points(_pd(M), M.size, int(L), float(g_slope), int(k), _pi(t1),
                                    _pi(t2)) != 0:
        raise ValueError("need a non-empty series and L >= 1")
    return int(t1[0]), int(t2[0])


# --------------------------------------------------------------------------
# Displaced GroupNorm ([DT] corrected_async_gn; reading in dfp_oracle.c)
# --------------------------------------------------------------------------
def displaced_group_norm(x, stats, G: int, p: int, eps: float, gamma=None, beta=None):
    """GroupNorm of one patch x [B, C, n] whose statistics combine the other
    patches' previous-step sums stats [B, G, P, 2] with this patch's fresh
    ones.  Returns (y [B, C, n], fresh sums [B, G, 2])."""
    x = _f64(x)
    stats = _f64(stats)
    B, C, n = x.shape
    if C % G != 0:
        raise ValueError("C must be a multiple of G")
    if stats.shape[:2] != (B, G) or stats.shape[3] != 2:
        raise ValueError("stats must be [B, G, P, 2]")
    P = stats.shape[2]
    if not 0 <= p < P:
        raise ValueError("patch index out of range")
    ga = None if gamma is None else _f64(gamma)
    be = None if beta is None else _f64(beta)
    for a in (ga, be):
        if a is not None and a.shape != (C,):
            raise ValueError("gamma and beta must be [C]")
    y = np.empty_like(x)
    fresh = np.empty((B, G, 2), dtype=np.float64)
    _load().oracle_displaced_group_norm(_pd(x), _pd(stats), None if ga is None else _pd(ga),
                                        None if be is None else _pd(be), B, C, G, n, P, p,
                                        float(eps), _pd(y), _pd(fresh))
    return y, fresh
