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

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
F32, BF16 = 0, 1
OP_CFG_STEP, OP_RELMAE, OP_PATCH_ATTENTION = 0, 1, 2

# Every function include/dfp.h declares, with its ctypes signature.
_P, _I, _I64, _F, _D, _SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_double, ctypes.c_size_t)
SIGNATURES = {
    "dfp_v_ld": (_I64, [_I64, _I]),
    "dfp_kv_scatter": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "dfp_patch_attention": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "dfp_patch_attention_fresh": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                       _P, _SZ, _P]),
    "dfp_cfg_step": (_I, [_P, _P, _P, _I64, _I, _F, _D, _D, _P, _P, _SZ, _P]),
    "dfp_cfg_step_noise": (_I, [_P, _P, _P, _P, _I64, _I, _F, _D, _D, _D, _P, _P, _SZ, _P]),
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
    B, H = new.shape[0], new.shape[1]
    n, d = new.shape[2], new.shape[3]
    N_buf = k_buf.shape[2] if k_buf is not None else None
    if v_buf_t is not None:
        if v_buf_t.shape[2] != d:
            raise ValueError("v_buf_t must be [B,H,d,ldv]")
        if N_buf is None:
            raise ValueError("landing V alone needs N_buf; pass k_buf as well")
        if v_buf_t.shape[3] != v_ld(N_buf, _dtype_code(v_buf_t)):
            raise ValueError("v_buf_t row stride does not match dfp_v_ld(N_buf)")
    st = lib().dfp_kv_scatter(_ptr(k_buf), _ptr(v_buf_t), _ptr(k_new), _ptr(v_new), B, H,
                              N_buf, d, int(row0), n, _dtype_code(ref), _stream(stream))
    _check(st, "dfp_kv_scatter")


def patch_attention(o, q, k_buf, v_buf_t, scale: float | None = None, workspace=None,
                    stream=None) -> None:
    B, H, n_q, d = q.shape
    N_kv = k_buf.shape[2]
    if tuple(o.shape) != tuple(q.shape) or k_buf.shape[:2] != q.shape[:2]:
        raise ValueError("o/q/k_buf shapes disagree")
    if tuple(v_buf_t.shape[:3]) != (B, H, d) or v_buf_t.shape[3] != v_ld(N_kv, _dtype_code(q)):
        raise ValueError("v_buf_t must be [B,H,d,dfp_v_ld(N_kv)]")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().dfp_patch_attention(_ptr(o), _ptr(q), _ptr(k_buf), _ptr(v_buf_t), B, H, n_q, N_kv,
                                   d, float(scale), _dtype_code(q), ws_ptr, ws_bytes,
                                   _stream(stream))
    _check(st, "dfp_patch_attention")


def patch_attention_fresh(o, q, k_buf, v_buf_t, fresh, land: bool = True,
                          scale: float | None = None, workspace=None, stream=None) -> None:
    """Attention with the rows of each fresh range read from this step's
    tensors, landing them in the buffer in the same launch when `land`.
    `fresh` is a list of one or two (k_new [B,H,n,d], v_new_t [B,H,d,n]
    channel-major, row0) tuples."""
    B, H, n_q, d = q.shape
    N_kv = k_buf.shape[2]
    if tuple(o.shape) != tuple(q.shape) or k_buf.shape[:2] != q.shape[:2]:
        raise ValueError("o/q/k_buf shapes disagree")
    if tuple(v_buf_t.shape[:3]) != (B, H, d) or v_buf_t.shape[3] != v_ld(N_kv, _dtype_code(q)):
        raise ValueError("v_buf_t must be [B,H,d,dfp_v_ld(N_kv)]")
    ranges = (FreshRows * max(len(fresh), 1))()
    for i, (k_new, v_new_t, row0) in enumerate(fresh):
        n = k_new.shape[2]
        if tuple(k_new.shape) != (B, H, n, d) or tuple(v_new_t.shape) != (B, H, d, n):
            raise ValueError("fresh k must be [B,H,n,d] and v_t [B,H,d,n]")
        ranges[i] = FreshRows(_ptr(k_new).value, _ptr(v_new_t).value, int(row0), n)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().dfp_patch_attention_fresh(_ptr(o), _ptr(q), _ptr(k_buf), _ptr(v_buf_t),
                                         ctypes.cast(ranges, ctypes.c_void_p), len(fresh), B, H,
                                         n_q, N_kv, d, 1 if land else 0, float(scale),
                                         _dtype_code(q), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "dfp_patch_attention_fresh")


def displaced_group_norm(y, x, stats, G: int, p: int, eps: float = 1e-5, gamma=None,
                         beta=None, land: bool = True, workspace=None, stream=None) -> None:
    """dfp_displaced_group_norm: y [B,C,n] = GroupNorm of the patch x [B,C,n]
    with statistics from the other patches' previous-step sums in stats
    [B,G,P,2] (float64) and this patch's fresh sums, which land in slot p."""
    B, C, n = x.shape
    P = stats.shape[2]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().dfp_displaced_group_norm(_ptr(y), _ptr(x), _ptr(stats),
                                        _ptr(gamma) if gamma is not None else None,
                                        _ptr(beta) if beta is not None else None, B, C, G, n,
                                        P, p, float(eps), 1 if land else 0,
                                        _ptr(workspace) if workspace is not None else None,
                                        ws_bytes, _stream(stream))
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


def cfg_step(x, g_c, g_u, w: float, c_x: float, c_e: float, relmae_out=None, workspace=None,
             stream=None) -> None:
    batch = x.shape[0]
    n = x.numel() // batch
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().dfp_cfg_step(_ptr(x), _ptr(g_c), _ptr(g_u), n, batch, float(w), float(c_x),
                            float(c_e), _ptr(relmae_out), _ptr(workspace), ws_bytes,
                            _stream(stream))
    _check(st, "dfp_cfg_step")


def cfg_step_noise(x, g_c, g_u, z, w: float, c_x: float, c_e: float, c_z: float,
                   relmae_out=None, workspace=None, stream=None) -> None:
    batch = x.shape[0]
    n = x.numel() // batch
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().dfp_cfg_step_noise(_ptr(x), _ptr(g_c), _ptr(g_u), _ptr(z), n, batch, float(w),
                                  float(c_x), float(c_e), float(c_z), _ptr(relmae_out),
                                  _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "dfp_cfg_step_noise")


def relmae(g_c, g_u, out, workspace, stream=None) -> None:
    batch = g_c.shape[0]
    n = g_c.numel() // batch
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().dfp_relmae(_ptr(g_c), _ptr(g_u), n, batch, _ptr(out), _ptr(workspace), ws_bytes,
                          _stream(stream))
    _check(st, "dfp_relmae")
