"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds data only: workload shapes and random draws.  It contains
none of the method's arithmetic (no attention, schedule, guidance, sampler or
rel-MAE); both sides receive the same arrays from here and compute everything
else on their own.

Workloads (all iid Gaussian; the pages measure quality on real prompts and
weights, which these synthetic draws stand in for):
  tiny-f32  fp32 check case: N=1024 (32x32 grid), P=2, 2 heads x 64, batch 2;
            latent 4x32x32, 10 DDIM steps, w=7.5.
  sdxl1024  SDXL-1024 shaped, bf16: 64x64 level N=4096, 10 heads, P=4 and
            32x32 level N=1024, 20 heads, P=4; latent 4x128x128, 50 DDIM
            steps, w=7.5.
  sdxl2048  SDXL-2048 shaped: N=16384, 10 heads, P=8; latent 4x256x256, 50
            steps.
  sdxl3840  SDXL-3840 shaped: N=57600, 10 heads, P=8; latent 4x480x480, 50
            steps.
  dit1024   DiT/flow shaped: 4096 image tokens + 256 always-fresh text
            tokens, 24 heads x 128, P=4; latent 16x128x128, 28 Euler steps,
            w=3.5.
Batch 2 on the attention side is the (cond, uncond) pair of classifier-free
guidance.  Head dim is 64 except dit1024 (128).

Draw recipe (numpy PCG64, standard_normal in float32), per attention level:
  q      [B,H,N_img,d]   queries of every image token (a patch uses its rows)
  k, v   [B,H,N_kv,d]    this step's ("fresh") keys / values, text rows first
  nk, nv [B,H,N_kv,d]    noise;  stale = fresh + 0.05 * noise
then every array is rounded to bf16 (nearest-even) for the bf16 workloads.
Sampler stream (seed + 200): x_T [1,C,H,W], then per step g_c and g_u;
sampler noise z for DDIM with eta > 0 comes from its own stream (seed + 300)
when the caller draws it, or from the counter-based generator keyed by
(seed + 300, step index) when the step draws it (noise_seed).
Seeds: per workload (1001 ... 1005 in the order above); a workload's second
attention level adds 100.

Displaced GroupNorm (the corrected_async_gn mode), one patch of a U-Net
feature map [B, C, H, W] cut into P row bands, n = (H/P) * W:
  x      [B,C,n]    per-channel N(mu_c, sigma_c), mu_c ~ N(0, 0.5),
                    sigma_c ~ U(0.5, 2) (activations differ per channel)
  stats  [B,G,P,2]  each other patch's (sum, sum of squares) of the previous
                    step, from drawn per-(image, group, patch) moments
                    m ~ N(0, 0.5), s ~ U(0.5, 2): (cnt m, cnt (s^2 + m^2)),
                    cnt = (C/G) n; the patch's own slot holds NaN (unused)
  gamma  [C] 1 + 0.1 N(0,1);  beta [C] 0.1 N(0,1)
SDXL-1024's first U-Net level stands in for the workload: C=320, G=32,
128x128, P=4, B=2.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

STALE_NOISE_STD = 0.05


@dataclass(frozen=True)
class AttnLevel:
    name: str
    B: int          # CFG batch (cond, uncond)
    H: int          # heads
    N_img: int      # image tokens in the full-image buffer
    P: int          # row-band patches (one patch = one GPU's share)
    d: int          # head dim
    n_text: int = 0  # always-fresh text tokens at rows [0, n_text)
    dtype: str = "bf16"
    seed: int = 0

    @property
    def n(self) -> int:
        """Query rows (and fresh K/V rows) of one patch."""
        return self.N_img // self.P

    @property
    def N_kv(self) -> int:
        return self.n_text + self.N_img

    def row0(self, p: int) -> int:
        """First buffer row of patch p (row-band patches, row-major grid)."""
        if not 0 <= p < self.P:
            raise ValueError("patch index out of range")
        return self.n_text + p * self.n

    def flops(self) -> float:
        """Algorithmic FLOP of one patch's attention: Q K^T and P V."""
        return 4.0 * self.B * self.H * self.n * self.N_kv * self.d


@dataclass(frozen=True)
class Workload:
    name: str
    levels: Tuple[AttnLevel, ...]
    latent: Tuple[int, int, int, int]  # (batch, C, H, W) of x
    steps: int
    sampler: str    # "ddim" or "euler"
    w: float
    seed: int

    @property
    def n_latent(self) -> int:
        b, c, h, w = self.latent
        return c * h * w


def _mk(name: str, seed: int, levels: List[dict], latent, steps, sampler, w) -> Workload:
    lv = tuple(AttnLevel(seed=seed + 100 * i, **kw) for i, kw in enumerate(levels))
    return Workload(name, lv, latent, steps, sampler, w, seed)


WORKLOADS = {
    "tiny-f32": _mk("tiny-f32", 1001,
                    [dict(name="tiny-f32", B=2, H=2, N_img=1024, P=2, d=64, dtype="f32")],
                    (1, 4, 32, 32), 10, "ddim", 7.5),
    "sdxl1024": _mk("sdxl1024", 1002,
                    [dict(name="sdxl1024-64x64", B=2, H=10, N_img=4096, P=4, d=64),
                     dict(name="sdxl1024-32x32", B=2, H=20, N_img=1024, P=4, d=64)],
                    (1, 4, 128, 128), 50, "ddim", 7.5),
    "sdxl2048": _mk("sdxl2048", 1003,
                    [dict(name="sdxl2048", B=2, H=10, N_img=16384, P=8, d=64)],
                    (1, 4, 256, 256), 50, "ddim", 7.5),
    "sdxl3840": _mk("sdxl3840", 1004,
                    [dict(name="sdxl3840", B=2, H=10, N_img=57600, P=8, d=64)],
                    (1, 4, 480, 480), 50, "ddim", 7.5),
    "dit1024": _mk("dit1024", 1005,
                   [dict(name="dit1024", B=2, H=24, N_img=4096, P=4, d=128, n_text=256)],
                   (1, 16, 128, 128), 28, "euler", 3.5),
}

LEVELS = {lv.name: lv for wl in WORKLOADS.values() for lv in wl.levels}


# --------------------------------------------------------------------------
# bf16 storage helpers (round to nearest even)
# --------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, nearest-even; NaN stays NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values that bf16 represents exactly (nearest-even rounding)."""
    return bf16_to_f32(bf16_bits(a))


# --------------------------------------------------------------------------
# Attention inputs
# --------------------------------------------------------------------------
@dataclass
class AttnInputs:
    level: AttnLevel
    q: np.ndarray        # [B,H,N_img,d] float32 (bf16-exact for bf16 levels)
    k_fresh: np.ndarray  # [B,H,N_kv,d]
    v_fresh: np.ndarray
    k_stale: np.ndarray
    v_stale: np.ndarray

    def q_patch(self, p: int) -> np.ndarray:
        n = self.level.n
        return self.q[:, :, p * n:(p + 1) * n, :]

    def fresh_rows(self, p: int):
        r0, n = self.level.row0(p), self.level.n
        return (self.k_fresh[:, :, r0:r0 + n, :], self.v_fresh[:, :, r0:r0 + n, :])

    def text_rows(self):
        t = self.level.n_text
        return (self.k_fresh[:, :, :t, :], self.v_fresh[:, :, :t, :])


def attention_inputs(level: AttnLevel, seed: int | None = None,
                     stale_std: float = STALE_NOISE_STD) -> AttnInputs:
    rng = np.random.Generator(np.random.PCG64(level.seed if seed is None else seed))
    B, H, d = level.B, level.H, level.d
    q = rng.standard_normal((B, H, level.N_img, d), dtype=np.float32)
    k = rng.standard_normal((B, H, level.N_kv, d), dtype=np.float32)
    v = rng.standard_normal((B, H, level.N_kv, d), dtype=np.float32)
    nk = rng.standard_normal((B, H, level.N_kv, d), dtype=np.float32)
    ks = k + np.float32(stale_std) * nk
    del nk
    nv = rng.standard_normal((B, H, level.N_kv, d), dtype=np.float32)
    vs = v + np.float32(stale_std) * nv
    del nv
    if level.dtype == "bf16":
        q, k, v, ks, vs = (round_bf16(a) for a in (q, k, v, ks, vs))
    return AttnInputs(level, q, k, v, ks, vs)


def random_attention_arrays(B: int, H: int, nq: int, N: int, d: int, seed: int,
                            dtype: str = "bf16"):
    """Free-form (q, k, v) for edge-case shapes; same distribution."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, nq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


# --------------------------------------------------------------------------
# Sampler inputs
# --------------------------------------------------------------------------
@dataclass
class SamplerStream:
    workload: Workload
    rng: np.random.Generator = field(repr=False)
    x_T: np.ndarray = None
    noise_rng: np.random.Generator = field(default=None, repr=False)

    def next_pair(self):
        """This step's (g_c, g_u), each shaped like x, float32 N(0,1)."""
        shape = self.workload.latent
        g_c = self.rng.standard_normal(shape, dtype=np.float32)
        g_u = self.rng.standard_normal(shape, dtype=np.float32)
        return g_c, g_u

    def next_noise(self):
        """This step's sampler noise z (DDIM with eta > 0), shaped like x,
        float32 N(0,1), from its own stream so the prediction draws do not
        depend on whether noise is drawn."""
        return self.noise_rng.standard_normal(self.workload.latent, dtype=np.float32)


def noise_seed(workload: Workload) -> int:
    """Seed of the sampler noise the fused step draws itself (the generator's
    key is (noise_seed, step index))."""
    return workload.seed + 300


def sampler_stream(workload: Workload, seed: int | None = None) -> SamplerStream:
    s = workload.seed + 200 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(s))
    x_T = rng.standard_normal(workload.latent, dtype=np.float32)
    return SamplerStream(workload, rng, x_T, np.random.Generator(np.random.PCG64(s + 100)))


@dataclass(frozen=True)
class GroupNormInputs:
    x: np.ndarray       # [B, C, n] float32
    stats: np.ndarray   # [B, G, P, 2] float64
    gamma: np.ndarray   # [C] float32
    beta: np.ndarray    # [C] float32


def group_norm_inputs(B: int, C: int, G: int, n: int, P: int, p: int,
                      seed: int) -> GroupNormInputs:
    """Seeded inputs of one displaced GroupNorm call (recipe in the module
    docstring)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    mu = rng.normal(0.0, 0.5, size=(B, C, 1)).astype(np.float32)
    sd = rng.uniform(0.5, 2.0, size=(B, C, 1)).astype(np.float32)
    x = (rng.standard_normal((B, C, n), dtype=np.float32) * sd + mu).astype(np.float32)
    cnt = float((C // G) * n)
    m = rng.normal(0.0, 0.5, size=(B, G, P))
    s = rng.uniform(0.5, 2.0, size=(B, G, P))
    stats = np.stack([cnt * m, cnt * (s * s + m * m)], axis=-1)
    stats[:, :, p, :] = np.nan
    gamma = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return GroupNormInputs(x, stats, gamma, beta)
