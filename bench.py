#!/usr/bin/env python3
"""Benchmark of one GPU's share of a patch-parallel diffusion step on MI355X.

The headline workload is the largest one that fits one GPU, SDXL-3840-shaped:
the 240x240 attention level (57600 tokens, 10 heads x 64, P=8, so one patch
is 7200 query rows against the 57600-row displaced K/V buffer; batch 2 =
cond/uncond) and the fused CFG + DDIM-50 + rel-MAE step on the 1x4x480x480
latent (w=7.5).  One timed "step" is the whole hot path once:
  landing of the patch's fresh K/V in the persistent buffer
      (dfp_kv_scatter: the patch's 7200 rows are not whole 64-key tiles) or,
      where the rows are whole tiles, inside the attention launch
      (dfp_patch_attention_fresh; a DiT passes its text rows as a second
      fresh range)
  patch attention over the buffer
  fused CFG + sampler update + rel-MAE on the latent.
All inputs are seeded synthetic arrays resident in HBM before timing starts.
The timed steps replay one HIP graph of the step (eager launches if capture
is refused).  Per-kernel durations come from HIP events on the launch stream
around batches of back-to-back launches.

The same run also times the other configurations' kernels (SDXL-1024's two
levels, SDXL-2048, DiT-1024) and reports them under "configs", and times
the fp64 oracle on the host on a bounded, seeded sample of the headline
workload ("cpu_baseline").

Prints ONE JSON line.  `--gpus N` with N > 1 is refused: this library is the
single-GPU share of the work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("patch-attn TFLOP/s (% bf16 MFMA peak); CFG+sampler step GB/s (% HBM peak)")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (vendor figure, 2.4 GHz)
PEAK_CLOCK_GHZ = 2.4
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
NAMES = {"sdxl1024": "SDXL-1024-shaped", "sdxl2048": "SDXL-2048-shaped",
         "sdxl3840": "SDXL-3840-shaped", "dit1024": "DiT/flow-shaped"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sdxl3840", choices=sorted(NAMES),
                    help="headline workload (default: the largest single-GPU one)")
    ap.add_argument("--configs", default="sdxl1024,sdxl2048,dit1024",
                    help="other workloads whose kernels are timed in the same run "
                         "(comma list; empty for none)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="host time budget of the oracle on all cores (the 1-core run "
                         "gets half of it)")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--sweep", action="store_true",
                    help="time the one-device patch sweep: every patch of each level in order "
                         "(each landing its fresh K/V for the patches after it), instead of one "
                         "patch")
    ap.add_argument("--no-fresh", action="store_true",
                    help="land fresh K/V with dfp_kv_scatter before dfp_patch_attention instead "
                         "of the fused dfp_patch_attention_fresh")
    ap.add_argument("--eta", type=float, default=0.0,
                    help="DDIM noise scale (DDIM workloads): > 0 runs the fused step with the "
                         "sampler-noise term drawn in the kernel (dfp_cfg_step_philox)")
    ap.add_argument("--noise-array", action="store_true",
                    help="with --eta: read the noise from a caller array (dfp_cfg_step_noise) "
                         "instead of drawing it in the kernel")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB, the "
                         "reference kernel that scales FETCH_SIZE/WRITE_SIZE counter runs")
    return ap.parse_args()


def profile_fields(path: str, section: str | None = None) -> dict:
    """key: value lines of a committed rocprofv3 summary (of one [section]
    when given)."""
    fields, cur = {}, None
    if not os.path.exists(path):
        return fields
    with open(path) as fh:
        for line in fh:
            s = line.strip()
            if s.startswith("[") and s.endswith("]"):
                cur = s[1:-1]
                continue
            if ":" in s and not s.startswith("#") and (section is None or cur == section
                                                       or cur is None):
                k, v = s.split(":", 1)
                fields[k.strip()] = v.strip()
    return fields


def source_sha(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def counted(path: str, source: str, key: str, section: str | None = None):
    """A figure from a committed counter summary, only while the kernel
    source still hashes to the one the counters were taken on (else None)."""
    f = profile_fields(path, section)
    if f.get("source_sha256") != source_sha(source) or key not in f:
        return None
    return float(f[key])


class Level:
    """Device buffers of one attention level, all resident in HBM.  By
    default the step covers one patch (one GPU's share); with `sweep` it
    covers every patch of the level in order (the one-device patch sweep)."""

    def __init__(self, level, dfp, torch, inputs, sweep=False, fresh=True):
        x = inputs.attention_inputs(level)
        self.level = level
        self.patches = list(range(level.P)) if sweep else [1 if level.P > 1 else 0]
        bf = torch.bfloat16

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a)).cuda().to(bf).contiguous()

        self.k_buf, self.v_buf = dfp.alloc_kv_buffer(level.B, level.H, level.N_kv, level.d, bf)
        dfp.kv_scatter(self.k_buf, self.v_buf, up(x.k_stale), up(x.v_stale), 0)
        # fused path: every fresh range (the patch, a DiT's text rows) whole 64-key tiles
        self.fused = (fresh and level.n % 64 == 0 and level.n_text % 64 == 0 and
                      all(level.row0(p) % 64 == 0 for p in self.patches))
        self.fresh, self.q, self.o = [], [], []
        for p in self.patches:
            kf, vf = x.fresh_rows(p)
            # the fused call takes V channel-major ([B,H,d,n]), as a projection can emit it
            v_in = np.swapaxes(vf, -1, -2) if self.fused else vf
            self.fresh.append((up(kf), up(v_in), level.row0(p)))
            self.q.append(up(x.q_patch(p)))
            self.o.append(torch.empty_like(self.q[-1]))
        self.text = None
        if level.n_text:
            kt, vt = x.text_rows()
            self.text = (up(kt), up(np.swapaxes(vt, -1, -2) if self.fused else vt))
        del x
        self.ws = dfp.attention_workspace(level.B, level.H, level.n, level.N_kv, level.d)
        self.scale = 1.0 / level.d ** 0.5
        self.flops = level.flops() * len(self.patches)
        self.fresh_bytes = 2 * 2 * self.fresh[0][0].numel() * 2   # K and V, read + write
        if self.text:
            self.fresh_bytes += 2 * 2 * self.text[0].numel() * 2
        self.plan = dfp.attention_plan(level.B, level.H, level.n, level.N_kv, level.d,
                                       self.ws is not None)

    def scatter(self, dfp, i=0):
        if self.text and i == 0:
            dfp.kv_scatter(self.k_buf, self.v_buf, self.text[0], self.text[1], 0)
        k, v, row0 = self.fresh[i]
        dfp.kv_scatter(self.k_buf, self.v_buf, k, v, row0)

    def attend(self, dfp, i=0):
        dfp.patch_attention(self.o[i], self.q[i], self.k_buf, self.v_buf, self.scale, self.ws)

    def attend_fresh(self, dfp, i=0):
        ranges = ([(self.text[0], self.text[1], 0)] if self.text else []) + [self.fresh[i]]
        dfp.patch_attention_fresh(self.o[i], self.q[i], self.k_buf, self.v_buf, ranges, True,
                                  self.scale, self.ws)

    def run(self, dfp):
        for i in range(len(self.patches)):
            if self.fused:
                self.attend_fresh(dfp, i)
            else:
                self.scatter(dfp, i)
                self.attend(dfp, i)

    def kernel_name(self):
        ks = self.plan[0]
        nf = (2 if self.text else 1) if self.fused else 0   # fresh ranges the launch reads
        return f"attn_fwd_bf16<{self.level.d}, {ks}, {nf}>"


class Sampler:
    """Latent, per-step prediction pairs (and caller noise when eta > 0 with
    --noise-array) and coefficients, all in HBM.  The pairs of every step
    stay resident, so consecutive timed steps read different predictions."""

    def __init__(self, wl, dfp, torch, inputs, eta=0.0, noise_array=False):
        st = inputs.sampler_stream(wl)
        self.wl = wl
        self.eta = eta if wl.sampler == "ddim" else 0.0
        self.noise_array = noise_array and self.eta > 0
        self.seed = inputs.noise_seed(wl)
        self.x = torch.from_numpy(st.x_T).cuda()
        pairs = [st.next_pair() for _ in range(wl.steps)]
        self.g_c = [torch.from_numpy(a).cuda() for a, _ in pairs]
        self.g_u = [torch.from_numpy(b).cuda() for _, b in pairs]
        self.z = ([torch.from_numpy(st.next_noise()).cuda() for _ in range(wl.steps)]
                  if self.noise_array else None)
        self.coeffs = []
        if wl.sampler == "ddim":
            abar = dfp.scaled_linear_abar(1000, 0.00085, 0.012)
            ts = dfp.ddim_timesteps(1000, wl.steps)
            S = wl.steps
            for i in range(S):
                a_prev = 1.0 if i == S - 1 else abar[ts[S - 2 - i]]
                self.coeffs.append(dfp.ddim_eta_coeffs(abar[ts[S - 1 - i]], a_prev, self.eta))
        else:
            for i in range(wl.steps):
                self.coeffs.append(dfp.euler_coeffs(1 - i / wl.steps, 1 - (i + 1) / wl.steps)
                                   + (0.0,))
        batch = wl.latent[0]
        self.ws = dfp.cfg_workspace(wl.n_latent, batch)
        self.r = torch.empty((wl.steps, batch), dtype=torch.float32, device="cuda")
        self.bytes = (20 if self.noise_array else 16) * self.x.numel()
        self.entry = ("dfp_cfg_step_noise" if self.noise_array else
                      "dfp_cfg_step_philox" if self.eta > 0 else "dfp_cfg_step")

    def step(self, dfp, i):
        k = i % self.wl.steps
        c_x, c_e, c_z = self.coeffs[k]
        if self.noise_array:
            dfp.cfg_step_noise(self.x, self.g_c[k], self.g_u[k], self.z[k], self.wl.w, c_x, c_e,
                               c_z, self.r[k], self.ws)
        elif self.eta > 0:
            dfp.cfg_step_philox(self.x, self.g_c[k], self.g_u[k], self.wl.w, c_x, c_e, c_z,
                                self.seed, k, self.r[k], self.ws)
        else:
            dfp.cfg_step(self.x, self.g_c[k], self.g_u[k], self.wl.w, c_x, c_e, self.r[k],
                         self.ws)


def time_kernel(torch, fn, reps, batches=3):
    """Average launch duration (us) of `fn`: HIP events on the launch stream
    around `reps` back-to-back launches, divided by `reps`, for each of
    `batches` batches.  A GPU spin queued first lets every launch reach the
    queue before any of them runs, so host launch latency does not land
    between the events; one event pair per batch (not per launch) keeps the
    events' own packets out of the kernel times.  Returns (mean over batches,
    min over batches)."""
    fn()
    torch.cuda.synchronize()
    per = []
    for _ in range(batches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(2e6 + reps * 1e5))
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / reps)
    return float(np.mean(per)), float(np.min(per))


def attn_reps(flops: float, reps: int) -> int:
    """Fewer back-to-back launches for long kernels (about 50 ms per batch)."""
    per = flops / 1e15   # seconds at ~1 PFLOP/s
    return max(3, min(reps, int(0.05 / max(per, 1e-9))))


def attention_bytes(level, landing: bool) -> float:
    """Algorithmic HBM bytes of one patch's attention launch (bf16): Q read
    and O written once, every K and V row read once (the patch's own rows
    from this step's tensors), and, when the launch lands the fresh rows
    (the patch's and a DiT's text rows), their write into the buffer."""
    e = 2
    bytes_ = 2 * level.B * level.H * level.n * level.d * e          # Q, O
    bytes_ += 2 * level.B * level.H * level.N_kv * level.d * e      # K, V
    if landing:
        bytes_ += 2 * level.B * level.H * (level.n + level.n_text) * level.d * e
    return float(bytes_)


def time_levels(levels, sampler, dfp, torch, reps):
    kern = {}
    for L in levels:
        # the attention launch the step runs: fused with the landing, or plain
        fn = (lambda L=L: L.attend_fresh(dfp)) if L.fused else (lambda L=L: L.attend(dfp))
        mean, mn = time_kernel(torch, fn, attn_reps(L.level.flops(), reps))
        tf = L.level.flops() / (mean * 1e-6) / 1e12
        # roofline of this launch: min(dense bf16 peak, arithmetic intensity x HBM)
        nbytes = attention_bytes(L.level, L.fused)
        ai = L.level.flops() / nbytes
        attain = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBPS / 1e3)
        kern[f"attn_{L.level.name}"] = {
            "us_mean": mean, "us_min": mn, "tflops": tf,
            "frac_bf16_peak": tf / PEAK_BF16_TFLOPS, "flop": L.level.flops(),
            "algorithmic_bytes": nbytes, "flop_per_byte": ai,
            "bound": "mfma" if attain >= PEAK_BF16_TFLOPS else "hbm",
            "attainable_tflops": attain, "frac_attainable": tf / attain,
            "kernel": L.kernel_name(),
            "plan": {"key_groups": L.plan[0], "splits": L.plan[1], "workgroups": L.plan[2]},
            "launch": "dfp_patch_attention_fresh (attention + landing of the fresh K/V)"
                      if L.fused else "dfp_patch_attention"}
        if not L.fused:
            mean, mn = time_kernel(torch, lambda L=L: L.scatter(dfp), reps)
            kern[f"scatter_{L.level.name}"] = {
                "us_mean": mean, "us_min": mn,
                "gbps": L.fresh_bytes / (mean * 1e-6) / 1e9,
                "frac_hbm_peak": L.fresh_bytes / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                "bytes": L.fresh_bytes}
    ctr = [0]

    def cfg():
        sampler.step(dfp, ctr[0])
        ctr[0] += 1
    mean, mn = time_kernel(torch, cfg, max(reps, 50))
    kern["cfg_step"] = {"us_mean": mean, "us_min": mn,
                        "gbps": sampler.bytes / (mean * 1e-6) / 1e9,
                        "frac_hbm_peak": sampler.bytes / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                        "bytes": sampler.bytes, "entry": sampler.entry}
    return kern


def time_sampler_graph(sampler, dfp, torch, replays=5):
    """The whole sampler trajectory -- every step's fused CFG step (both
    launches), in order -- captured as one HIP graph and replayed: per-step
    time with launch gaps as small as the runtime makes them, to set beside
    the per-launch figure.  x drifts over the replays; only time is read."""
    S = sampler.wl.steps
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(S):
                sampler.step(dfp, i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(S):
                sampler.step(dfp, i)
        g.replay()
        torch.cuda.synchronize()
    except Exception as e:  # capture refused: report nothing
        print(f"[bench] sampler graph unavailable ({e})", file=sys.stderr)
        return None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / replays
    del g
    return {"steps": S, "us_per_trajectory": us, "us_per_step": us / S,
            "gbps": sampler.bytes / (us / S * 1e-6) / 1e9,
            "launch": "one HIP graph of the whole trajectory"}


def rocminfo_max_clock_ghz():
    """The gfx950 agent's maximum engine clock as rocminfo reports it, or None."""
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    found = False
    for line in out.splitlines():
        t = line.strip()
        if t.startswith("Name:") and "gfx950" in t:
            found = True
        elif found and t.startswith("Max Clock Freq. (MHz):"):
            try:
                return float(t.split(":", 1)[1]) / 1e3
            except ValueError:
                return None
    return None


def time_group_norm(wl, dfp, torch, inputs, reps):
    """Displaced GroupNorm (the corrected_async_gn mode) on the workload's
    first U-Net level: 320 channels in 32 groups over the latent grid, one
    patch's row band, batch 2, with a workspace (the whole-GPU path).  A DiT
    has no GroupNorm.  8 algorithmic bytes per element (x read, y written);
    the per-group sums are a few KB."""
    if not wl.name.startswith("sdxl"):
        return None
    _, _, hl, wdl = wl.latent
    pg = wl.levels[0].P
    n = (hl // pg) * wdl
    gi = inputs.group_norm_inputs(2, 320, 32, n, pg, 1, wl.seed + 300)
    gx = torch.from_numpy(gi.x).cuda()
    gy = torch.empty_like(gx)
    gst = torch.from_numpy(gi.stats).cuda()
    gga, gbe = torch.from_numpy(gi.gamma).cuda(), torch.from_numpy(gi.beta).cuda()
    gws = dfp.group_norm_workspace(2, 320, 32, n)
    mean, mn = time_kernel(torch, lambda: dfp.displaced_group_norm(
        gy, gx, gst, 32, 1, 1e-5, gga, gbe, True, gws), reps)
    gb = 8 * gx.numel()
    return {"us_mean": mean, "us_min": mn, "gbps": gb / (mean * 1e-6) / 1e9,
            "frac_hbm_peak": gb / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS, "bytes": gb,
            "shape": f"x [2, 320, {n}] (patch 1 of {pg}), 32 groups"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inputs, budget_s: float):
    """The fp64 oracle, as it stands, on the headline workload: the patch
    attention of seeded random (batch*head, query row) pairs of patch 1 of
    every level over its displaced buffer, in rounds of 256 rows until the
    time budget is spent -- once on every host core the oracle's OpenMP
    loops use, once on one core.  Reported like `value` (attention FLOP of
    the rows timed / host time)."""
    import oracle
    levels = []
    for lv in wl.levels:
        x = inputs.attention_inputs(lv)
        p = 1 if lv.P > 1 else 0
        k_eff = oracle.effective_kv(x.k_stale, x.fresh_rows(p)[0], lv.row0(p))
        v_eff = oracle.effective_kv(x.v_stale, x.fresh_rows(p)[1], lv.row0(p))
        if lv.n_text:
            k_eff = oracle.effective_kv(k_eff, x.text_rows()[0], 0)
            v_eff = oracle.effective_kv(v_eff, x.text_rows()[1], 0)
        q = np.ascontiguousarray(x.q_patch(p), dtype=np.float64)
        del x
        levels.append((lv, q, k_eff, v_eff))
    rng = np.random.Generator(np.random.PCG64(wl.seed + 900))

    def run(seconds):
        rows, flop, t0 = 0, 0.0, time.perf_counter()
        while True:
            for lv, q, k, v in levels:
                bh = rng.integers(0, lv.B * lv.H, size=256)
                ri = rng.integers(0, lv.n, size=256)
                oracle.attention_rows(q, k, v, 1.0 / lv.d ** 0.5, bh, ri)
                rows += 256
                flop += 256 * 4.0 * lv.N_kv * lv.d
            dt = time.perf_counter() - t0
            if dt >= seconds:
                return rows, flop, dt

    cores = oracle.num_threads()
    rows, flop, dt = run(budget_s)
    oracle.set_threads(1)
    rows1, flop1, dt1 = run(budget_s / 2)
    oracle.set_threads(cores)
    lv_desc = ", ".join(f"{lv.name} (N_kv {lv.N_kv}, d {lv.d})" for lv, *_ in levels)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} seeded random (batch*head, query row) pairs of patch 1 of "
                      f"{lv_desc}, fp64 two-pass attention over the displaced buffer, "
                      f"{flop / 1e9:.1f} GFLOP in {dt:.1f} s on {cores} threads",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "value_1core": flop1 / dt1 / 1e12,
            "sample_1core": f"{rows1} pairs, {flop1 / 1e9:.1f} GFLOP in {dt1:.1f} s on 1 thread"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU's share of the work; "
                                   "run it with --gpus 1 (multi-GPU runs are not supported)"}))
        sys.exit(2)

    import torch
    from patch_attention_cfg_amd import dfp, inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    dfp.lib()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = inputs.WORKLOADS[args.workload]
    levels = [Level(lv, dfp, torch, inputs, args.sweep, not args.no_fresh) for lv in wl.levels]
    sampler = Sampler(wl, dfp, torch, inputs, args.eta, args.noise_array)
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: inputs resident", file=sys.stderr, flush=True)

    def one_step(i):
        for L in levels:
            L.run(dfp)
        sampler.step(dfp, i)

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()

    launch = "eager"
    graph = None
    if not args.no_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                one_step(0)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                one_step(0)
            torch.cuda.synchronize()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            launch = "hip-graph"
        except Exception as e:  # capture refused: time eager launches instead
            print(f"graph capture unavailable ({e}); timing eager launches", file=sys.stderr)
            graph = None

    # ---- timed region: exactly K steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            one_step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = max(ev0.elapsed_time(ev1), 1e-9) / args.steps
    attn_flops = sum(L.flops for L in levels)
    print(f"[bench] {wl.name}: {args.steps} steps timed, {ms_per_step:.3f} ms/step",
          file=sys.stderr, flush=True)

    # ---- per-kernel durations (HIP events on the launch stream)
    kern = time_levels(levels, sampler, dfp, torch, args.kernel_reps)
    kern["cfg_step"]["trajectory_graph"] = time_sampler_graph(sampler, dfp, torch)
    gn = time_group_norm(wl, dfp, torch, inputs, max(args.kernel_reps, 50))
    if gn:
        kern["displaced_group_norm"] = gn

    dom = max(levels, key=lambda L: L.level.flops())
    dk = kern[f"attn_{dom.level.name}"]
    attn_src = "patch_attention_cfg_amd/csrc/attention_bf16.hip"
    prof = os.path.join(ROOT, "profiles")
    traffic = counted(os.path.join(prof, f"attn_bf16_{dom.level.name}_hbm_traffic.txt"),
                      attn_src, "traffic_bytes")
    clock = counted(os.path.join(prof, f"attn_bf16_{dom.level.name}_sq_counters.txt"),
                    attn_src, "clock_ghz")
    roofline = {"bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dk["tflops"] / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": f"{dom.kernel_name()} ({dom.level.name}, "
                          f"{dom.level.flops() / 1e9:.2f} GFLOP per launch)"}
    if clock:
        pc = PEAK_BF16_TFLOPS * clock / PEAK_CLOCK_GHZ
        roofline.update({"clock_ghz_measured": clock, "peak_at_measured_clock": pc,
                         "frac_at_measured_clock": dk["tflops"] / pc})
    roofline["clock_ghz_rocminfo_max"] = rocminfo_max_clock_ghz()
    ck = kern["cfg_step"]
    cfg_src = "patch_attention_cfg_amd/csrc/cfg_step.hip"
    cfg_prof = os.path.join(prof, f"cfg_step_{wl.name}_hbm_traffic.txt")
    rd = counted(cfg_prof, cfg_src, "read_bytes")
    wr = counted(cfg_prof, cfg_src, "write_bytes")
    cfg_roofline = {"bound": "hbm", "achieved": ck["gbps"], "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": ck["frac_hbm_peak"],
                    "traffic": (rd + wr) if rd is not None and wr is not None else None,
                    "kernel": f"cfg_step_kernel ({sampler.entry}, latent "
                              f"{'x'.join(map(str, wl.latent))}, {sampler.bytes} B per launch)"}
    del graph
    keep = {"attn": [(L.level.name, L.kernel_name()) for L in levels]}
    del levels, sampler
    torch.cuda.empty_cache()

    # ---- the other configurations' kernels, same run
    configs = {}
    for name in [c for c in args.configs.split(",") if c and c != wl.name]:
        cw = inputs.WORKLOADS[name]
        clv = [Level(lv, dfp, torch, inputs, False, not args.no_fresh) for lv in cw.levels]
        csm = Sampler(cw, dfp, torch, inputs, args.eta, args.noise_array)
        torch.cuda.synchronize()
        for _ in range(2):
            for L in clv:
                L.run(dfp)
            csm.step(dfp, 0)
        ckern = time_levels(clv, csm, dfp, torch, args.kernel_reps)
        ckern["cfg_step"]["trajectory_graph"] = time_sampler_graph(csm, dfp, torch)
        cgn = time_group_norm(cw, dfp, torch, inputs, max(args.kernel_reps, 50))
        if cgn:
            ckern["displaced_group_norm"] = cgn
        configs[name] = {"workload": NAMES[name], "kernels": ckern}
        print(f"[bench] {name}: kernels timed", file=sys.stderr, flush=True)
        del clv, csm
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inputs, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": attn_flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": NAMES[wl.name]
                        + (" one-device patch sweep: every patch of each attention level in order"
                           " + fused CFG step" if args.sweep else
                           " patch-parallel step: one patch per attention level + fused CFG step"),
            "attention": [f"{lv.name}: B{lv.B} H{lv.H} n_q{lv.n} N_kv{lv.N_kv} d{lv.d} bf16"
                          for lv in wl.levels],
            "attention_kernels": dict(keep["attn"]),
            "latent": list(wl.latent), "sampler": f"{wl.sampler}{wl.steps} fp32"
            + (f" eta={args.eta}" if args.eta > 0 and wl.sampler == "ddim" else ""),
            "w": wl.w, "launch": launch},
        "cfg_step_gbps": ck["gbps"],
        "cfg_step_frac_hbm_peak": ck["frac_hbm_peak"],
        "wall_s_timed": wall,
        "kernels": kern,
        "roofline": roofline,
        "cfg_step_roofline": cfg_roofline,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
