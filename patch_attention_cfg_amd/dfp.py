"""Python binding of libdfp.so (ctypes).  Argument marshalling only: every
step of the computation runs in the library's HIP kernels.  PyTorch supplies
device memory and the current stream.

The names mirror include/dfp.h without the ``dfp_`` prefix.  A non-OK status
raises DFPError.  There is no fallback: if libdfp.so is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdfp.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_TOO_LARGE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
OP_CFG_STEP, OP_RELMAE, OP_PATCH_ATTENTION = 0, 1, 2
_M64 = 2**64 - 1

# Every function include/dfp.h declares, with its ctypes signature.
_P, _I, _I64, _F, _D, _SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_double, ctypes.c_size_t)
_U64 = ctypes.c_uint64
SIGNATURES = {
    "dfp_v_ld": (_I64, [_I64, _I]),
    "dfp_kv_scatter": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "dfp_kv_scatter_strided": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _I64, _I64, _I,
                                    _P]),
    "dfp_patch_attention": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "dfp_patch_attention_fresh": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                       _P, _SZ, _P]),
    "dfp_cfg_step": (_I, [_P, _P, _P, _I64, _I, _F, _D, _D, _P, _P, _SZ, _P]),
    "dfp_cfg_step_noise": (_I, [_P, _P, _P, _P, _I64, _I, _F, _D, _D, _D, _P, _P, _SZ, _P]),
    "dfp_cfg_step_philox": (_I, [_P, _P, _P, _I64, _I, _F, _D, _D, _D, _U64, _U64, _P, _P,
                                 _SZ, _P]),
    "dfp_philox_normal": (_I, [_P, _I64, _I, _U64, _U64, _P]),
    "dfp_philox4x64_10": (_I, [_P, _I64, _U64, _U64, _U64, _P]),
    "dfp_cfg_step_static": (_I, [_P, _P, _P, _I64, _I, _F, _D, _D, _P, _P]),
    "dfp_cfg_static_scratch_bytes": (_SZ, []),
    "dfp_relmae": (_I, [_P, _P, _I64, _I, _P, _P, _SZ, _P]),
    "dfp_workspace_bytes": (_SZ, [_I, _I64, _I, _I, _I, _I, _I, _I]),
    "dfp_attention_plan": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "dfp_displaced_group_norm": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I64, _I, _I, _F, _I,
                                      _P, _SZ, _P]),
    "dfp_group_norm_workspace_bytes": (_SZ, [_I, _I, _I, _I64]),
    "dfp_ddim_coeffs": (_I, [_D, _D, _P, _P]),
    "dfp_ddim_eta_coeffs": (_I, [_D, _D, _D, _P, _P, _P]),
    "dfp_euler_coeffs": (_I, [_D, _D, _P, _P]),
    "dfp_switch_points": (_I, [_P, _I, _I, _D, _I, _P, _P]),
    "dfp_scaled_linear_abar": (_I, [_I, _D, _D, _P]),
    "dfp_ddim_timesteps": (_I, [_I, _I, _P]),
    "dfp_status_string": (ctypes.c_char_p, [_I]),
}



class FreshRows(ctypes.Structure):
    """dfp_fresh_rows: one range of fresh rows (device pointers)."""
    _fields_ = [("k", ctypes.c_void_p), ("v_t", ctypes.c_void_p), ("row0", ctypes.c_int),
                ("n", ctypes.c_int)]


_lib = None


class DFPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded libdfp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m patch_attention_cfg_amd.build`"
                " (there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().dfp_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise DFPError(status, where)


# ----------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(cond: bool, msg: str) -> None:
    """Argument check of the binding: the C ABI takes raw pointers, so
    shapes, dtypes and devices are checked here, before anything is
    enqueued."""
    if not cond:
        raise ValueError(msg)


def _on_one_device(*ts) -> None:
    ts = [t for t in ts if t is not None]
    for t in ts:
        _need(t.is_cuda, "every tensor must live on the GPU")
        _need(t.is_contiguous(), "every tensor must be contiguous")
    _need(len({t.device for t in ts}) <= 1, "tensors live on different devices")


def _f32_like(ref, *ts) -> None:
    torch = _torch()
    for t in ts:
        if t is None:
            continue
        _need(t.dtype == torch.float32, "latent tensors must be float32")
        _need(t.numel() == ref.numel(), "latent tensors must have as many elements as x")


def _ws_bytes(workspace) -> int:
    return workspace.numel() * workspace.element_size() if workspace is not None else 0


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------- helpers
def v_ld(N_buf: int, dtype_code: int) -> int:
    return int(lib().dfp_v_ld(int(N_buf), int(dtype_code)))


def workspace_bytes(op: int, n_per_image: int = 0, batch: int = 0, B: int = 0, H: int = 0,
                    n_q: int = 0, N_kv: int = 0, d: int = 0) -> int:
    return int(lib().dfp_workspace_bytes(op, n_per_image, batch, B, H, n_q, N_kv, d))


def attention_plan(B: int, H: int, n_q: int, N_kv: int, d: int, with_workspace: bool = True):
    """(key_groups, splits, workgroups) of a bf16 attention call of these
    sizes (dfp_attention_plan; host only)."""
    ks, sp, wg = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    _check(lib().dfp_attention_plan(B, H, n_q, N_kv, d, 1 if with_workspace else 0,
                                    ctypes.byref(ks), ctypes.byref(sp), ctypes.byref(wg)),
           "dfp_attention_plan")
    return ks.value, sp.value, wg.value


def ddim_coeffs(abar_t: float, abar_prev: float):
    cx, ce = ctypes.c_double(), ctypes.c_double()
    _check(lib().dfp_ddim_coeffs(abar_t, abar_prev, ctypes.byref(cx), ctypes.byref(ce)),
           "dfp_ddim_coeffs")
    return cx.value, ce.value


def ddim_eta_coeffs(abar_t: float, abar_prev: float, eta: float):
    cx, ce, cz = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().dfp_ddim_eta_coeffs(abar_t, abar_prev, eta, ctypes.byref(cx), ctypes.byref(ce),
                                     ctypes.byref(cz)), "dfp_ddim_eta_coeffs")
    return cx.value, ce.value, cz.value


def euler_coeffs(sigma: float, sigma_next: float):
    cx, ce = ctypes.c_double(), ctypes.c_double()
    _check(lib().dfp_euler_coeffs(sigma, sigma_next, ctypes.byref(cx), ctypes.byref(ce)),
           "dfp_euler_coeffs")
    return cx.value, ce.value


def scaled_linear_abar(T: int = 1000, beta_start: float = 0.00085,
                       beta_end: float = 0.012) -> np.ndarray:
    out = np.empty(T, dtype=np.float64)
    _check(lib().dfp_scaled_linear_abar(T, beta_start, beta_end, out.ctypes.data),
           "dfp_scaled_linear_abar")
    return out


def switch_points(relmae_series, L: int, g_slope: float, k: int = 5):
    """(tau1, tau2) from a host rel-MAE series (see dfp_switch_points)."""
    m = np.ascontiguousarray(np.asarray(relmae_series, dtype=np.float32).ravel())
    t1, t2 = ctypes.c_int(), ctypes.c_int()
    _check(lib().dfp_switch_points(m.ctypes.data, m.size, int(L), float(g_slope), int(k),
                                   ctypes.byref(t1), ctypes.byref(t2)), "dfp_switch_points")
    return t1.value, t2.value


def ddim_timesteps(T: int, S: int) -> np.ndarray:
    out = np.empty(S, dtype=np.int32)
    _check(lib().dfp_ddim_timesteps(T, S, out.ctypes.data), "dfp_ddim_timesteps")
    return out


# ----------------------------------------------------------------- GPU calls
def alloc_kv_buffer(B: int, H: int, N_buf: int, d: int, dtype, device="cuda"):
    """Allocate (k_buf [B,H,N_buf,d], v_buf_t [B,H,d,ldv]) uninitialised."""
    torch = _torch()
    code = BF16 if dtype == torch.bfloat16 else F32
    ld = v_ld(N_buf, code)
    k = torch.empty((B, H, N_buf, d), dtype=dtype, device=device)
    v = torch.empty((B, H, d, ld), dtype=dtype, device=device)
    return k, v


def kv_scatter(k_buf, v_buf_t, k_new, v_new, row0: int, stream=None) -> None:
    ref = k_buf if k_buf is not None else v_buf_t
    new = k_new if k_new is not None else v_new
    _need(ref is not None and new is not None, "nothing to land")
    _need((k_buf is None) == (k_new is None) and (v_buf_t is None) == (v_new is None),
          "pass both tensors of the K pair and of the V pair, or neither")
    _on_one_device(k_buf, v_buf_t, k_new, v_new)
    _need(new.dim() == 4, "fresh rows must be [B,H,n,d]")
    B, H = new.shape[0], new.shape[1]
    n, d = new.shape[2], new.shape[3]
    for t in (k_new, v_new):
        _need(t is None or tuple(t.shape) == (B, H, n, d), "k_new and v_new must be [B,H,n,d]")
    for t in (k_buf, v_buf_t, k_new, v_new):
        _need(t is None or t.dtype == ref.dtype, "buffer and fresh rows must share a dtype")
    N_buf = k_buf.shape[2] if k_buf is not None else None
    if k_buf is not None:
        _need(k_buf.dim() == 4 and tuple(k_buf.shape[:2]) == (B, H) and k_buf.shape[3] == d,
              "k_buf must be [B,H,N_buf,d]")
    if v_buf_t is not None:
        _need(v_buf_t.dim() == 4 and tuple(v_buf_t.shape[:3]) == (B, H, d),
              "v_buf_t must be [B,H,d,ldv]")
        _need(N_buf is not None, "landing V alone needs N_buf; pass k_buf as well")
        _need(v_buf_t.shape[3] == v_ld(N_buf, _dtype_code(v_buf_t)),
              "v_buf_t row stride does not match dfp_v_ld(N_buf)")
    st = lib().dfp_kv_scatter(_ptr(k_buf), _ptr(v_buf_t), _ptr(k_new), _ptr(v_new), B, H,
                              N_buf, d, int(row0), n, _dtype_code(ref), _stream(stream))
    _check(st, "dfp_kv_scatter")


def kv_scatter_strided(k_buf, v_buf_t, k_new, v_new, row0: int, stream=None) -> None:
    """dfp_kv_scatter_strided: k_new / v_new are [B,H,n,d] views of any layout
    with contiguous rows (stride 1 along d) and equal strides, e.g.
    x.permute(0, 2, 1, 3) of a projection's [B,n,H,d] output."""
    _need(k_new is not None and v_new is not None and k_buf is not None and v_buf_t is not None,
          "the strided landing takes both K and V")
    for t in (k_buf, v_buf_t):
        _need(t.is_cuda and t.is_contiguous(), "the buffers must be contiguous GPU tensors")
    for t in (k_new, v_new):
        _need(t.is_cuda and t.dim() == 4 and t.stride(3) == 1,
              "fresh rows must be [B,H,n,d] GPU views with contiguous rows")
    _need(len({t.device for t in (k_buf, v_buf_t, k_new, v_new)}) == 1,
          "tensors live on different devices")
    _need(tuple(k_new.shape) == tuple(v_new.shape) and k_new.stride() == v_new.stride(),
          "k_new and v_new must share shape and strides")
    B, H, n, d = k_new.shape
    _need(len({t.dtype for t in (k_buf, v_buf_t, k_new, v_new)}) == 1,
          "buffer and fresh rows must share a dtype")
    _need(k_buf.dim() == 4 and tuple(k_buf.shape[:2]) == (B, H) and k_buf.shape[3] == d,
          "k_buf must be [B,H,N_buf,d]")
    N_buf = k_buf.shape[2]
    _need(tuple(v_buf_t.shape[:3]) == (B, H, d) and
          v_buf_t.shape[3] == v_ld(N_buf, _dtype_code(v_buf_t)), "v_buf_t must be [B,H,d,ldv]")
    sb, sh, sn = k_new.stride(0), k_new.stride(1), k_new.stride(2)
    # a size-1 dimension's stride is never used
    sb, sh, sn = (0 if B == 1 else sb), (0 if H == 1 else sh), (d if n == 1 else sn)
    st = lib().dfp_kv_scatter_strided(_ptr(k_buf), _ptr(v_buf_t),
                                      ctypes.c_void_p(k_new.data_ptr()),
                                      ctypes.c_void_p(v_new.data_ptr()), B, H, N_buf, d, int(row0),
                                      n, sb, sh, sn, _dtype_code(k_buf), _stream(stream))
    _check(st, "dfp_kv_scatter_strided")


def _check_attention(o, q, k_buf, v_buf_t, workspace):
    _on_one_device(o, q, k_buf, v_buf_t, workspace)
    _need(q.dim() == 4 and k_buf.dim() == 4 and v_buf_t.dim() == 4, "tensors must be 4-D")
    B, H, n_q, d = q.shape
    N_kv = k_buf.shape[2]
    _need(tuple(o.shape) == tuple(q.shape), "o must be shaped like q")
    _need(tuple(k_buf.shape) == (B, H, N_kv, d), "k_buf must be [B,H,N_kv,d]")
    _need(o.dtype == q.dtype == k_buf.dtype == v_buf_t.dtype,
          "o, q, k_buf and v_buf_t must share a dtype")
    _need(tuple(v_buf_t.shape[:3]) == (B, H, d) and
          v_buf_t.shape[3] == v_ld(N_kv, _dtype_code(q)), "v_buf_t must be [B,H,d,dfp_v_ld(N_kv)]")
    return B, H, n_q, N_kv, d


def patch_attention(o, q, k_buf, v_buf_t, scale: float | None = None, workspace=None,
                    stream=None) -> None:
    B, H, n_q, N_kv, d = _check_attention(o, q, k_buf, v_buf_t, workspace)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    st = lib().dfp_patch_attention(_ptr(o), _ptr(q), _ptr(k_buf), _ptr(v_buf_t), B, H, n_q, N_kv,
                                   d, float(scale), _dtype_code(q), _ptr(workspace),
                                   _ws_bytes(workspace), _stream(stream))
    _check(st, "dfp_patch_attention")


def patch_attention_fresh(o, q, k_buf, v_buf_t, fresh, land: bool = True,
                          scale: float | None = None, workspace=None, stream=None) -> None:
    """Attention with the rows of each fresh range read from this step's
    tensors, landing them in the buffer in the same launch when `land`.
    `fresh` is a list of one or two (k_new [B,H,n,d], v_new_t [B,H,d,n]
    channel-major, row0) tuples."""
    B, H, n_q, N_kv, d = _check_attention(o, q, k_buf, v_buf_t, workspace)
    ranges = (FreshRows * max(len(fresh), 1))()
    for i, (k_new, v_new_t, row0) in enumerate(fresh):
        _on_one_device(q, k_new, v_new_t)
        n = k_new.shape[2]
        _need(tuple(k_new.shape) == (B, H, n, d) and tuple(v_new_t.shape) == (B, H, d, n),
              "fresh k must be [B,H,n,d] and v_t [B,H,d,n]")
        _need(k_new.dtype == v_new_t.dtype == q.dtype, "fresh rows must share q's dtype")
        ranges[i] = FreshRows(_ptr(k_new).value, _ptr(v_new_t).value, int(row0), n)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    st = lib().dfp_patch_attention_fresh(_ptr(o), _ptr(q), _ptr(k_buf), _ptr(v_buf_t),
                                         ctypes.cast(ranges, ctypes.c_void_p), len(fresh), B, H,
                                         n_q, N_kv, d, 1 if land else 0, float(scale),
                                         _dtype_code(q), _ptr(workspace), _ws_bytes(workspace),
                                         _stream(stream))
    _check(st, "dfp_patch_attention_fresh")


def displaced_group_norm(y, x, stats, G: int, p: int, eps: float = 1e-5, gamma=None,
                         beta=None, land: bool = True, workspace=None, stream=None) -> None:
    """dfp_displaced_group_norm: y [B,C,n] = GroupNorm of the patch x [B,C,n]
    with statistics from the other patches' previous-step sums in stats
    [B,G,P,2] (float64) and this patch's fresh sums, which land in slot p."""
    torch = _torch()
    _on_one_device(y, x, stats, gamma, beta, workspace)
    _need(x.dim() == 3 and tuple(y.shape) == tuple(x.shape), "x and y must be [B,C,n]")
    B, C, n = x.shape
    _need(x.dtype == y.dtype == torch.float32, "x and y must be float32")
    _need(stats.dim() == 4 and tuple(stats.shape[:2]) == (B, G) and stats.shape[3] == 2 and
          stats.dtype == torch.float64, "stats must be float64 [B,G,P,2]")
    for t in (gamma, beta):
        _need(t is None or (t.dtype == torch.float32 and t.numel() == C),
              "gamma and beta must be float32 [C]")
    P = stats.shape[2]
    st = lib().dfp_displaced_group_norm(_ptr(y), _ptr(x), _ptr(stats), _ptr(gamma), _ptr(beta),
                                        B, C, G, n, P, p, float(eps), 1 if land else 0,
                                        _ptr(workspace), _ws_bytes(workspace), _stream(stream))
    _check(st, "dfp_displaced_group_norm")


def group_norm_workspace(B: int, C: int, G: int, n: int, device="cuda"):
    """A zero-filled workspace for dfp_displaced_group_norm (None when the
    sizes need none)."""
    torch = _torch()
    nbytes = int(lib().dfp_group_norm_workspace_bytes(B, C, G, n))
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def attention_workspace(B: int, H: int, n_q: int, N_kv: int, d: int, device="cuda"):
    """A zero-filled workspace that lets dfp_patch_attention split the key
    range (None when the chosen plan does not split)."""
    torch = _torch()
    nbytes = workspace_bytes(OP_PATCH_ATTENTION, 0, 0, B, H, n_q, N_kv, d)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def cfg_workspace(n_per_image: int, batch: int, device="cuda"):
    """A zero-filled workspace for dfp_cfg_step / dfp_relmae."""
    torch = _torch()
    nbytes = workspace_bytes(OP_CFG_STEP, n_per_image, batch)
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def _check_latent(x, g_c, g_u, z, relmae_out, workspace):
    """x [batch, ...] float32 and the arrays that go with it."""
    torch = _torch()
    _on_one_device(x, g_c, g_u, z, relmae_out, workspace)
    _need(x.dim() >= 1 and x.shape[0] >= 1, "x must be [batch, ...]")
    _f32_like(x, x, g_c, g_u, z)
    batch = x.shape[0]
    if relmae_out is not None:
        _need(relmae_out.dtype == torch.float32 and relmae_out.numel() >= batch,
              "relmae_out must hold one float32 per image")
    return batch, x.numel() // batch


def cfg_step(x, g_c, g_u, w: float, c_x: float, c_e: float, relmae_out=None, workspace=None,
             stream=None) -> None:
    batch, n = _check_latent(x, g_c, g_u, None, relmae_out, workspace)
    st = lib().dfp_cfg_step(_ptr(x), _ptr(g_c), _ptr(g_u), n, batch, float(w), float(c_x),
                            float(c_e), _ptr(relmae_out), _ptr(workspace), _ws_bytes(workspace),
                            _stream(stream))
    _check(st, "dfp_cfg_step")


def cfg_step_static(x, g_c, g_u, w: float, c_x: float, c_e: float, relmae_out=None,
                    stream=None) -> None:
    """dfp_cfg_step without a workspace: the partials use the library's
    static scratch (for callers that cannot allocate)."""
    batch, n = _check_latent(x, g_c, g_u, None, relmae_out, None)
    st = lib().dfp_cfg_step_static(_ptr(x), _ptr(g_c), _ptr(g_u), n, batch, float(w),
                                   float(c_x), float(c_e), _ptr(relmae_out), _stream(stream))
    _check(st, "dfp_cfg_step_static")


def cfg_step_noise(x, g_c, g_u, z, w: float, c_x: float, c_e: float, c_z: float,
                   relmae_out=None, workspace=None, stream=None) -> None:
    _need(z is not None, "z is required")
    batch, n = _check_latent(x, g_c, g_u, z, relmae_out, workspace)
    st = lib().dfp_cfg_step_noise(_ptr(x), _ptr(g_c), _ptr(g_u), _ptr(z), n, batch, float(w),
                                  float(c_x), float(c_e), float(c_z), _ptr(relmae_out),
                                  _ptr(workspace), _ws_bytes(workspace), _stream(stream))
    _check(st, "dfp_cfg_step_noise")


def cfg_step_philox(x, g_c, g_u, w: float, c_x: float, c_e: float, c_z: float, seed: int,
                    step: int, relmae_out=None, workspace=None, stream=None) -> None:
    """Fused step with the sampler noise drawn in the kernel (Philox4x64-10 +
    Box-Muller keyed by (seed, step), counter (block, image))."""
    batch, n = _check_latent(x, g_c, g_u, None, relmae_out, workspace)
    st = lib().dfp_cfg_step_philox(_ptr(x), _ptr(g_c), _ptr(g_u), n, batch, float(w),
                                   float(c_x), float(c_e), float(c_z), int(seed) & _M64,
                                   int(step) & _M64, _ptr(relmae_out), _ptr(workspace),
                                   _ws_bytes(workspace), _stream(stream))
    _check(st, "dfp_cfg_step_philox")


def philox_normal(z, seed: int, step: int, stream=None) -> None:
    """Write into z [batch, ...] the draw dfp_cfg_step_philox adds."""
    _on_one_device(z)
    _need(z.dtype == _torch().float32 and z.dim() >= 1, "z must be float32 [batch, ...]")
    batch = z.shape[0]
    st = lib().dfp_philox_normal(_ptr(z), z.numel() // batch, batch, int(seed) & _M64,
                                 int(step) & _M64, _stream(stream))
    _check(st, "dfp_philox_normal")


def philox4x64_10(out, counter1: int, key0: int, key1: int, stream=None) -> None:
    """Raw Philox4x64-10 blocks into out [blocks, 4] (64-bit integer storage)."""
    _on_one_device(out)
    _need(out.dim() == 2 and out.shape[1] == 4 and out.element_size() == 8,
          "out must be [blocks, 4] of 64-bit integers")
    st = lib().dfp_philox4x64_10(_ptr(out), out.shape[0], int(counter1) & _M64, int(key0) & _M64,
                                 int(key1) & _M64, _stream(stream))
    _check(st, "dfp_philox4x64_10")


def relmae(g_c, g_u, out, workspace, stream=None) -> None:
    _need(out is not None and workspace is not None, "out and workspace are required")
    batch, n = _check_latent(g_c, g_c, g_u, None, out, workspace)
    st = lib().dfp_relmae(_ptr(g_c), _ptr(g_u), n, batch, _ptr(out), _ptr(workspace),
                          _ws_bytes(workspace), _stream(stream))
    _check(st, "dfp_relmae")
