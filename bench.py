#!/usr/bin/env python3
"""Benchmark of one GPU's share of a patch-parallel diffusion step on MI355X.

One timed "step" is the whole hot path once, at the SDXL-1024-shaped workload
(64x64 level: 4096 tokens, 10 heads x 64, P=4; 32x32 level: 1024 tokens,
20 heads x 64, P=4; batch 2 = cond/uncond; latent 1x4x128x128, DDIM-50,
w=7.5):
  patch attention (64x64 level), reading the patch's fresh K/V from this
      step's tensors and landing them in the persistent buffer in the same
      launch (dfp_patch_attention_fresh)
  the same for the 32x32 level
  fused CFG + DDIM update + rel-MAE on the latent.
A DiT level passes its always-fresh text rows as a second fresh range.  A
level whose patch rows are not whole 64-key tiles (SDXL-3840) lands its K/V
with dfp_kv_scatter and then runs dfp_patch_attention; `--no-fresh` times
that path everywhere.
All inputs are seeded synthetic arrays resident in HBM before timing starts.
The timed steps replay one HIP graph of the step (falls back to eager
launches if capture is refused).  Per-kernel durations for the roofline come
from HIP events on the launch stream around batches of back-to-back launches.

Prints ONE JSON line.  `--gpus N` with N > 1 is refused: this library is the
single-GPU share of the work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("patch-attn TFLOP/s (% bf16 MFMA peak); CFG+sampler step GB/s (% HBM peak)")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sdxl1024",
                    choices=["sdxl1024", "sdxl2048", "sdxl3840", "dit1024"],
                    help="sdxl1024 is the reported workload; the others are for exploration")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--sweep", action="store_true",
                    help="time the one-device patch sweep: every patch of each level in order "
                         "(each landing its fresh K/V for the patches after it), instead of one "
                         "patch")
    ap.add_argument("--no-fresh", action="store_true",
                    help="land fresh K/V with dfp_kv_scatter before dfp_patch_attention instead "
                         "of the fused dfp_patch_attention_fresh")
    ap.add_argument("--eta", type=float, default=0.0,
                    help="DDIM noise scale (DDIM workloads): > 0 runs the fused step with the "
                         "sampler-noise term (dfp_cfg_step_noise)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB, the "
                         "reference kernel that scales FETCH_SIZE/WRITE_SIZE counter runs")
    return ap.parse_args()


def measured_traffic(kernel_source: str, level_name: str):
    """HBM bytes per launch of the attention kernel on `level_name`, from the
    committed rocprofv3 counter summary -- only while the kernel source still
    hashes to the one the counters were taken on (else None)."""
    path = os.path.join(ROOT, "profiles", f"attn_bf16_{level_name}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(kernel_source, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    if fields.get("source_sha256") != sha or "traffic_bytes" not in fields:
        return None
    return float(fields["traffic_bytes"])


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
        self.ws = dfp.attention_workspace(level.B, level.H, level.n, level.N_kv, level.d)
        self.scale = 1.0 / level.d ** 0.5
        self.flops = level.flops() * len(self.patches)
        self.fresh_bytes = 2 * 2 * self.fresh[0][0].numel() * 2   # K and V, read + write
        if self.text:
            self.fresh_bytes += 2 * 2 * self.text[0].numel() * 2

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


class Sampler:
    """Latent, per-step prediction pairs (and sampler noise when eta > 0) and
    coefficients, all in HBM."""

    def __init__(self, wl, dfp, torch, inputs, eta=0.0):
        st = inputs.sampler_stream(wl)
        self.wl = wl
        self.eta = eta if wl.sampler == "ddim" else 0.0
        self.x = torch.from_numpy(st.x_T).cuda()
        pairs = [st.next_pair() for _ in range(wl.steps)]
        self.g_c = [torch.from_numpy(a).cuda() for a, _ in pairs]
        self.g_u = [torch.from_numpy(b).cuda() for _, b in pairs]
        self.z = ([torch.from_numpy(st.next_noise()).cuda() for _ in range(wl.steps)]
                  if self.eta > 0 else None)
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
        self.bytes = (20 if self.z else 16) * self.x.numel()

    def step(self, dfp, i):
        k = i % self.wl.steps
        c_x, c_e, c_z = self.coeffs[k]
        if self.z:
            dfp.cfg_step_noise(self.x, self.g_c[k], self.g_u[k], self.z[k], self.wl.w, c_x, c_e,
                               c_z, self.r[k], self.ws)
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


def cpu_baseline(wl, inputs):
    """The fp64 oracle, as it stands, on the same workload: one whole step
    (every attention level's patch attention over its displaced buffer, then
    the guided sampler step with rel-MAE), repeated until about 10 s of host
    work; reported like `value` (attention FLOP of the step / step time)."""
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
        levels.append((x.q_patch(p), k_eff, v_eff, 1.0 / lv.d ** 0.5, lv.flops()))
    st = inputs.sampler_stream(wl)
    g_c, g_u = st.next_pair()
    sched = oracle.DDIMSchedule(wl.steps) if wl.sampler == "ddim" else oracle.EulerSchedule(wl.steps)
    flops = sum(lv[4] for lv in levels)
    reps, t0 = 0, time.perf_counter()
    while True:
        for q, k, v, scale, _ in levels:
            oracle.attention(q, k, v, scale)
        sched.step(st.x_T, g_c, g_u, wl.w, reps % wl.steps)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 200:
            break
    return {"value": reps * flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} whole steps of the {wl.name} workload: patch attention of every "
                      f"level ({flops / 1e9:.2f} GFLOP per step, fp64) and the guided "
                      f"{wl.sampler} step with rel-MAE on the latent, {dt:.1f} s"}


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
    sampler = Sampler(wl, dfp, torch, inputs, args.eta)
    torch.cuda.synchronize()

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

    # ---- per-kernel durations (HIP events on the launch stream)
    reps = args.kernel_reps
    kern = {}
    for L in levels:
        # the attention launch the step runs: fused with the landing, or plain
        fn = (lambda L=L: L.attend_fresh(dfp)) if L.fused else (lambda L=L: L.attend(dfp))
        mean, mn = time_kernel(torch, fn, reps)
        kern[f"attn_{L.level.name}"] = {
            "us_mean": mean, "us_min": mn,
            "tflops": L.level.flops() / (mean * 1e-6) / 1e12,
            "frac_bf16_peak": L.level.flops() / (mean * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
            "flop": L.level.flops(),
            "launch": "dfp_patch_attention_fresh (attention + landing of the fresh K/V)"
                      if L.fused else "dfp_patch_attention"}
        if not L.fused:
            mean, mn = time_kernel(torch, lambda L=L: L.scatter(dfp), reps)
            kern[f"scatter_{L.level.name}"] = {
                "us_mean": mean, "us_min": mn,
                "gbps": L.fresh_bytes / (mean * 1e-6) / 1e9, "bytes": L.fresh_bytes}
    ctr = [0]

    def cfg():
        sampler.step(dfp, ctr[0])
        ctr[0] += 1
    mean, mn = time_kernel(torch, cfg, reps)
    kern["cfg_step"] = {"us_mean": mean, "us_min": mn,
                        "gbps": sampler.bytes / (mean * 1e-6) / 1e9,
                        "frac_hbm_peak": sampler.bytes / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                        "bytes": sampler.bytes}

    # displaced GroupNorm (the corrected_async_gn mode) on the workload's
    # first U-Net level: 320 channels in 32 groups over the latent grid, one
    # patch's row band; a DiT has no GroupNorm
    if wl.name.startswith("sdxl") or wl.name == "tiny-f32":
        _, _, hl, wdl = wl.latent
        pg = wl.levels[0].P
        gi = inputs.group_norm_inputs(2, 320, 32, (hl // pg) * wdl, pg, 1, wl.seed + 300)
        gx = torch.from_numpy(gi.x).cuda()
        gy = torch.empty_like(gx)
        gst = torch.from_numpy(gi.stats).cuda()
        gga, gbe = torch.from_numpy(gi.gamma).cuda(), torch.from_numpy(gi.beta).cuda()
        gws = dfp.group_norm_workspace(2, 320, 32, (hl // pg) * wdl)
        mean, mn = time_kernel(torch, lambda: dfp.displaced_group_norm(
            gy, gx, gst, 32, 1, 1e-5, gga, gbe, True, gws), reps)
        gb = 8 * gx.numel()   # x read, y written; the per-group sums are 0.02%
        kern["displaced_group_norm"] = {
            "us_mean": mean, "us_min": mn, "gbps": gb / (mean * 1e-6) / 1e9,
            "frac_hbm_peak": gb / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS, "bytes": gb,
            "shape": f"x [2, 320, {(hl // pg) * wdl}] (patch 1 of {pg}), 32 groups"}
        del gx, gy, gst, gws

    # the same fused step streaming a batch of 32 latents in one call: the
    # kernel's bandwidth once the per-call latency (launch, reduction tail)
    # is amortised
    nb = 32
    xs = torch.randn((nb, wl.n_latent), device="cuda")
    gcs, gus = torch.randn_like(xs), torch.randn_like(xs)
    rs = torch.empty(nb, device="cuda")
    wss = dfp.cfg_workspace(wl.n_latent, nb)
    c_x, c_e, _ = sampler.coeffs[-1]   # the last step's: c_x ~ 1, so repeats stay bounded
    mean, mn = time_kernel(torch, lambda: dfp.cfg_step(xs, gcs, gus, wl.w, c_x, c_e, rs, wss),
                           max(reps // 4, 5))
    sb = 16 * xs.numel()
    kern["cfg_step_batch32"] = {"us_mean": mean, "us_min": mn, "gbps": sb / (mean * 1e-6) / 1e9,
                                "frac_hbm_peak": sb / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                                "bytes": sb}
    del xs, gcs, gus

    dom = max(levels, key=lambda L: L.level.flops())
    lv = dom.level
    dom_ks = dfp.attention_plan(lv.B, lv.H, lv.n, lv.N_kv, lv.d, dom.ws is not None)[0]
    dom_nf = (2 if dom.text else 1) if dom.fused else 0   # fresh ranges the launch reads
    dk = kern[f"attn_{dom.level.name}"]
    traffic = measured_traffic(
        os.path.join(ROOT, "patch_attention_cfg_amd", "csrc", "attention_bf16.hip"),
        dom.level.name)
    roofline = {"bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dk["tflops"] / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": f"attn_fwd_bf16<{dom.level.d}, {dom_ks}, {dom_nf}> "
                          f"({dom.level.name}, "
                          f"{dom.level.flops() / 1e9:.2f} GFLOP per launch)"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inputs)

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
            "workload": {"sdxl1024": "SDXL-1024-shaped", "sdxl2048": "SDXL-2048-shaped",
                         "sdxl3840": "SDXL-3840-shaped", "dit1024": "DiT/flow-shaped"}[wl.name]
                        + (" one-device patch sweep: every patch of each attention level in order"
                           " + fused CFG step" if args.sweep else
                           " patch-parallel step: one patch per attention level + fused CFG step"),
            "kv_landing": {L.level.name: "fused into the attention launch" if L.fused
                           else "dfp_kv_scatter before the attention" for L in levels},
            "attention": [f"{L.level.name}: B{L.level.B} H{L.level.H} n_q{L.level.n} "
                          f"N_kv{L.level.N_kv} d{L.level.d} bf16" for L in levels],
            "latent": list(wl.latent), "sampler": f"{wl.sampler}{wl.steps} fp32"
            + (f" eta={sampler.eta}" if sampler.eta > 0 else ""), "w": wl.w,
            "launch": launch},
        "cfg_step_gbps": kern["cfg_step"]["gbps"],
        "cfg_step_frac_hbm_peak": kern["cfg_step"]["frac_hbm_peak"],
        "wall_s_timed": wall,
        "kernels": kern,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
