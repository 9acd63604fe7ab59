// group_norm.hip -- displaced GroupNorm of one patch: the group statistics
// combine every other patch's sums from the previous step (stale) with this
// patch's own sums from this step (fresh), then normalize the patch.
//
// Sources (page title, section):
//   "DistriFusion高级教程：自定义并行配置实现超高清图像生成的完整指南",
//   多设备配置优化 and 速度与质量平衡: a communication mode named
//   corrected_async_gn (asynchronous GroupNorm with a correction), given by
//   name only.
//   "终极性能对比：DistriFusion vs 传统推理方案", DistriFusion的革命性突破:
//   later steps reuse the previous step's activations of the other patches.
// Reading: per (image, group), S1 = fresh sum + the other patches' stale
// sums, S2 likewise for squares, N = P * n * C/G, mean = S1/N, biased
// variance S2/N - mean^2, eps inside the square root.
//
// The group's C/G channels of the patch are one contiguous run of C/G * n
// floats.  Runs of up to 64 Ki floats (n % 4 == 0, x and y 16-byte aligned):
// one workgroup per (image, group) keeps its run in registers between the
// two uses, so x is read once, and stages the group's gamma and beta in LDS
// alongside, so nothing but the statistics stands between the two.  Longer
// runs, given a workspace: every run is cut into chunks of 4 Ki floats
// spread over the whole GPU, in two launches -- launch 1 stores each chunk's
// fp64 sums; launch 2 has every chunk add its group's chunk sums in chunk
// order (the same order in every chunk, so all agree bit for bit), form the
// statistics, read and normalize its floats again, and the group's first
// chunk lands the fresh sums.  No atomics and no counters: the launch
// boundary orders the two.  Otherwise one workgroup streams each run twice.
// Sums are fp64 per thread, per wavefront (fixed butterfly) and across
// wavefronts and chunks in a fixed order, so the statistics are bitwise
// reproducible.
#include <cmath>

#include "dfp_common.h"

namespace {

constexpr int kGnThreads = 1024;
constexpr int kGnWaves = kGnThreads / dfp::kWave;
constexpr int kGnVec = 16;   // float4 per thread held in registers
constexpr int64_t kGnResidentFloats = (int64_t)kGnThreads * kGnVec * 4;
// Chunked path: 256-thread workgroups over 4 Ki-float chunks (16 floats per
// thread), at most kGnMaxChunks per run (longer chunks beyond).
constexpr int kGcThreads = 256;
constexpr int kGcWaves = kGcThreads / dfp::kWave;
constexpr int64_t kGcChunk = (int64_t)kGcThreads * 4 * 4;
constexpr int kGnMaxChunks = 4096;

int64_t run_chunks(int64_t run) {
    const int64_t c = (run + kGcChunk - 1) / kGcChunk;
    return c < kGnMaxChunks ? c : kGnMaxChunks;
}
// Floats per chunk of a run split nch ways; with float4 access a multiple
// of 4, so every chunk starts on a float4 of its run (and, with n % 4 == 0,
// no float4 crosses a channel).
__host__ __device__ inline int64_t chunk_span(int64_t run, int nch, bool vec) {
    const int64_t per = (run + nch - 1) / nch;
    return vec ? (per + 3) / 4 * 4 : per;
}
size_t gn_workspace_need(int64_t groups, int64_t chunks) {
    return (size_t)groups * chunks * 2 * sizeof(double);
}

struct GnArgs {
    float *y;
    const float *x;
    double *stats;   // [B][G][P][2]
    const float *gamma, *beta;
    int C, G, P, p;
    int64_t n;
    float eps;
    int land;
    int reverse;     // chunked path: launch 2 walks the chunks last first
};

// Sum of every thread's pair across a workgroup of WAVES wavefronts, in
// fixed order; the result is valid in thread 0.
template <int WAVES>
__device__ __forceinline__ void block_sums(double &s1, double &s2) {
    __shared__ double w1[WAVES], w2[WAVES];
    const int tid = threadIdx.x, wave = tid / dfp::kWave, lane = tid % dfp::kWave;
    s1 = dfp::wave_sum(s1);
    s2 = dfp::wave_sum(s2);
    if (lane == 0) {
        w1[wave] = s1;
        w2[wave] = s2;
    }
    __syncthreads();
    if (tid == 0) {
        double f1 = 0.0, f2 = 0.0;
        for (int k = 0; k < WAVES; ++k) {
            f1 += w1[k];
            f2 += w2[k];
        }
        s1 = f1;
        s2 = f2;
    }
}

// The other patches' stale sums of one group, [P][2] doubles, for the
// chunked path's second launch: threads 0 .. 2P-1 load them at the
// kernel's start, so their round trip overlaps the chunk's loads instead of
// following the workgroup's reduction, and store them in LDS before the
// statistics' barrier (measured 2.6% faster at x [2, 320, 8192]; the
// register path measured slower with it and reads them after its
// reduction).  More than kStLds patches: read from memory after the
// barrier.  Either way the statistics add the same values in the same
// order.
constexpr int kStLds = 64;
struct StaleSums {
    double v = 0.0;
    __device__ __forceinline__ static bool staged(const GnArgs &a) { return a.P <= kStLds; }
    __device__ __forceinline__ void load(const GnArgs &a, int64_t grp) {
        const int t = threadIdx.x;
        if (staged(a) && t < 2 * a.P && t / 2 != a.p) v = a.stats[grp * a.P * 2 + t];
    }
    __device__ __forceinline__ void stage(const GnArgs &a, double *s_st) const {
        if (staged(a) && (int)threadIdx.x < 2 * a.P) s_st[threadIdx.x] = v;
    }
};

// The group's (mean, rstd) from its fresh sums (f1, f2) and the other
// patches' stale sums (from `staged` when the caller staged them, else from
// memory); the fresh sums land in the patch's slot.
__device__ __forceinline__ float2 stats_from_sums(const GnArgs &a, int b, int g, double f1,
                                                  double f2, const double *staged) {
    double *st = a.stats + ((int64_t)b * a.G + g) * a.P * 2;
    const double *src = staged ? staged : st;
    double t1 = f1, t2 = f2;
    for (int q = 0; q < a.P; ++q)
        if (q != a.p) {
            t1 += src[2 * q];
            t2 += src[2 * q + 1];
        }
    const double N = (double)a.P * (double)a.n * (double)(a.C / a.G);
    const double mean = t1 / N;
    const double var = t2 / N - mean * mean;
    if (a.land) {
        st[2 * a.p] = f1;
        st[2 * a.p + 1] = f2;
    }
    return make_float2((float)mean, (float)(1.0 / sqrt(var + (double)a.eps)));
}

// One workgroup per group: its sums, then (mean, rstd) in every thread.
__device__ __forceinline__ float2 group_stats(const GnArgs &a, int b, int g, double s1,
                                              double s2, const double *staged) {
    __shared__ float mean_rstd[2];
    block_sums<kGnWaves>(s1, s2);
    if (threadIdx.x == 0) {
        const float2 mr = stats_from_sums(a, b, g, s1, s2, staged);
        mean_rstd[0] = mr.x;
        mean_rstd[1] = mr.y;
    }
    __syncthreads();
    return make_float2(mean_rstd[0], mean_rstd[1]);
}

__device__ __forceinline__ void accum4(double &s1, double &s2, float4 v) {
    s1 += (double)v.x + (double)v.y + (double)v.z + (double)v.w;
    s2 = fma((double)v.x, (double)v.x, s2);
    s2 = fma((double)v.y, (double)v.y, s2);
    s2 = fma((double)v.z, (double)v.z, s2);
    s2 = fma((double)v.w, (double)v.w, s2);
}

__device__ __forceinline__ float4 affine4(float4 v, float mean, float sc, float be) {
    return make_float4((v.x - mean) * sc + be, (v.y - mean) * sc + be, (v.z - mean) * sc + be,
                       (v.w - mean) * sc + be);
}

template <bool AFFINE>
__device__ __forceinline__ float4 normalize4(const GnArgs &a, float4 v, int c, float2 mr) {
    const float ga = AFFINE && a.gamma ? a.gamma[c] : 1.f;
    const float be = AFFINE && a.beta ? a.beta[c] : 0.f;
    return affine4(v, mr.x, mr.y * ga, be);
}

// gamma and beta of a group's channels [c0, c0 + cnt) staged in LDS by the
// register-resident path: the first cnt threads load them before the x
// loads (so they share that round trip), store them after, and the
// statistics' barrier publishes them; the normalization then reads no
// memory after the statistics.  Groups of more channels read them from
// memory.
constexpr int kGbLds = 256;
struct GammaBeta {
    float ga = 1.f, be = 0.f;
    template <bool AFFINE>
    __device__ __forceinline__ void load(const GnArgs &a, int c0, int cnt) {
        if (AFFINE && cnt <= kGbLds && (int)threadIdx.x < cnt) {
            if (a.gamma) ga = a.gamma[c0 + threadIdx.x];
            if (a.beta) be = a.beta[c0 + threadIdx.x];
        }
    }
    template <bool AFFINE>
    __device__ __forceinline__ void stage(float *s_ga, float *s_be, int cnt) const {
        if (AFFINE && cnt <= kGbLds && (int)threadIdx.x < cnt) {
            s_ga[threadIdx.x] = ga;
            s_be[threadIdx.x] = be;
        }
    }
};

// The group's run in registers: n % 4 == 0 (a float4 never crosses a
// channel), x and y 16-byte aligned, C/G * n <= kGnResidentFloats.
template <bool AFFINE>
__global__ __launch_bounds__(kGnThreads) void gn_resident_kernel(GnArgs a) {
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int cg = a.C / a.G;
    const int n4 = (int)(a.n / 4);
    const int len4 = cg * n4;
    const int64_t off = ((int64_t)b * a.C + (int64_t)g * cg) * a.n;
    const float4 *xg = reinterpret_cast<const float4 *>(a.x + off);
    __shared__ float s_ga[kGbLds], s_be[kGbLds];
    const bool gb_lds = AFFINE && cg <= kGbLds;
    GammaBeta gb;
    gb.load<AFFINE>(a, g * cg, cg);
    float4 v[kGnVec];
#pragma unroll
    for (int k = 0; k < kGnVec; ++k) {
        const int i = tid + k * kGnThreads;
        v[k] = i < len4 ? xg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    gb.stage<AFFINE>(s_ga, s_be, cg);
    // only the slots that hold the run: the fp64 sums are the costly part of
    // this kernel, and adding the padding's zeros would not change them
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int k = 0; k < kGnVec; ++k)
        if (tid + k * kGnThreads < len4) accum4(s1, s2, v[k]);
    const float2 mr = group_stats(a, b, g, s1, s2, nullptr);
    float4 *yg = reinterpret_cast<float4 *>(a.y + off);
#pragma unroll
    for (int k = 0; k < kGnVec; ++k) {
        const int i = tid + k * kGnThreads;
        if (i >= len4) continue;
        if (gb_lds) {
            const int lc = i / n4;
            yg[i] = affine4(v[k], mr.x, mr.y * s_ga[lc], s_be[lc]);
        } else {
            yg[i] = normalize4<AFFINE>(a, v[k], g * cg + i / n4, mr);
        }
    }
}

// Any run length and alignment: two passes over x, scalar.
template <bool AFFINE>
__global__ __launch_bounds__(kGnThreads) void gn_stream_kernel(GnArgs a) {
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int cg = a.C / a.G;
    const int64_t len = (int64_t)cg * a.n;
    const int64_t off = ((int64_t)b * a.C + (int64_t)g * cg) * a.n;
    const float *xg = a.x + off;
    double s1 = 0.0, s2 = 0.0;
    for (int64_t i = tid; i < len; i += kGnThreads) {
        const double v = (double)xg[i];
        s1 += v;
        s2 = fma(v, v, s2);
    }
    const float2 mr = group_stats(a, b, g, s1, s2, nullptr);
    float *yg = a.y + off;
    for (int64_t i = tid; i < len; i += kGnThreads) {
        const int c = g * cg + (int)(i / a.n);
        const float ga = AFFINE && a.gamma ? a.gamma[c] : 1.f;
        const float be = AFFINE && a.beta ? a.beta[c] : 0.f;
        yg[i] = (xg[i] - mr.x) * (mr.y * ga) + be;
    }
}

// Chunked path, launch 1: chunk blockIdx.x of group (blockIdx.y, blockIdx.z)
// sums its floats and stores the pair.  VEC: float4 loads (n % 4 == 0, x
// 16-byte aligned).
template <bool VEC>
__global__ __launch_bounds__(kGcThreads) void gn_chunk_sums_kernel(GnArgs a, double *partials) {
    const int chunk = blockIdx.x, nch = gridDim.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int64_t run = (int64_t)(a.C / a.G) * a.n;
    const int64_t per = chunk_span(run, nch, VEC);
    const int64_t lo = min(run, (int64_t)chunk * per), hi = min(run, lo + per);
    const float *xg = a.x + ((int64_t)b * a.C + (int64_t)g * (a.C / a.G)) * a.n;
    double s1 = 0.0, s2 = 0.0;
    if (VEC) {
        const float4 *x4 = reinterpret_cast<const float4 *>(xg + lo);
        const int64_t m4 = (hi - lo) / 4;
        for (int64_t i = tid; i < m4; i += kGcThreads) accum4(s1, s2, x4[i]);
    } else {
        for (int64_t i = lo + tid; i < hi; i += kGcThreads) {
            const double v = (double)xg[i];
            s1 += v;
            s2 = fma(v, v, s2);
        }
    }
    block_sums<kGcWaves>(s1, s2);
    if (tid == 0) {
        double *pp = partials + (((int64_t)b * a.G + g) * nch + chunk) * 2;
        pp[0] = s1;
        pp[1] = s2;
    }
}

// Chunked path, launch 2: every chunk adds its group's chunk sums in chunk
// order (thread t takes chunks t, t + 256, ..., then the fixed block sum),
// forms (mean, rstd) -- the group's chunk 0 also lands the fresh sums -- and
// normalizes its floats.
template <bool VEC, bool AFFINE>
__global__ __launch_bounds__(kGcThreads) void gn_chunk_norm_kernel(GnArgs a,
                                                                   const double *partials) {
    // With `reverse` the chunks go last first, each on the XCD that read it
    // in launch 1 (workgroup i runs on XCD i % 8, and the permutation keeps
    // i % 8), so the most recently read chunks come first.  Any order gives
    // the same results.
    const int nch = gridDim.x;
    int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (a.reverse) {   // set only for grids of fewer than 2^31 workgroups
        const uint32_t wg = blockIdx.x + (uint32_t)nch * (blockIdx.y + gridDim.y * blockIdx.z);
        const uint32_t all = (uint32_t)nch * gridDim.y * gridDim.z;
        const uint32_t lin = (all / 8 - 1 - wg / 8) * 8 + wg % 8;
        const uint32_t rest = lin / (uint32_t)nch;
        chunk = (int)(lin - rest * (uint32_t)nch);
        g = (int)(rest % gridDim.y);
        b = (int)(rest / gridDim.y);
    }
    const int tid = threadIdx.x;
    const int cg = a.C / a.G;
    const int64_t run = (int64_t)cg * a.n;
    const int64_t per = chunk_span(run, nch, VEC);
    const int64_t lo = min(run, (int64_t)chunk * per), hi = min(run, lo + per);
    const int64_t off = ((int64_t)b * a.C + (int64_t)g * cg) * a.n;
    const int64_t grp = (int64_t)b * a.G + g;
    __shared__ double s_st[2 * kStLds];
    StaleSums stale;
    stale.load(a, grp);
    // this chunk's floats first: they do not depend on the statistics
    constexpr int kHeld = 4;   // float4 per thread held across the statistics
    const int64_t m4 = VEC ? (hi - lo) / 4 : 0;
    const float4 *x4 = reinterpret_cast<const float4 *>(a.x + off + lo);
    float4 v[kHeld];
    if (VEC) {
#pragma unroll
        for (int k = 0; k < kHeld; ++k) {
            const int64_t i = tid + (int64_t)k * kGcThreads;
            v[k] = i < m4 ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    double f1 = 0.0, f2 = 0.0;
    for (int k = tid; k < nch; k += kGcThreads) {
        f1 += partials[(grp * nch + k) * 2];
        f2 += partials[(grp * nch + k) * 2 + 1];
    }
    stale.stage(a, s_st);
    __shared__ float mean_rstd[2];
    block_sums<kGcWaves>(f1, f2);
    if (tid == 0) {
        GnArgs ac = a;
        ac.land = a.land && chunk == 0;
        const float2 mr =
            stats_from_sums(ac, b, g, f1, f2, StaleSums::staged(a) ? s_st : nullptr);
        mean_rstd[0] = mr.x;
        mean_rstd[1] = mr.y;
    }
    __syncthreads();
    const float2 mr = make_float2(mean_rstd[0], mean_rstd[1]);
    if (VEC) {
        float4 *y4 = reinterpret_cast<float4 *>(a.y + off + lo);
#pragma unroll
        for (int k = 0; k < kHeld; ++k) {
            const int64_t i = tid + (int64_t)k * kGcThreads;
            if (i < m4) y4[i] = normalize4<AFFINE>(a, v[k], g * cg + (int)((lo + 4 * i) / a.n), mr);
        }
        for (int64_t i = tid + (int64_t)kHeld * kGcThreads; i < m4; i += kGcThreads)
            y4[i] = normalize4<AFFINE>(a, x4[i], g * cg + (int)((lo + 4 * i) / a.n), mr);
    } else {
        for (int64_t i = lo + tid; i < hi; i += kGcThreads) {
            const int c = g * cg + (int)(i / a.n);
            const float ga = AFFINE && a.gamma ? a.gamma[c] : 1.f;
            const float be = AFFINE && a.beta ? a.beta[c] : 0.f;
            a.y[off + i] = (a.x[off + i] - mr.x) * (mr.y * ga) + be;
        }
    }
}

bool aligned(const void *p, uintptr_t to) { return (reinterpret_cast<uintptr_t>(p) % to) == 0; }

}  // namespace

extern "C" size_t dfp_group_norm_workspace_bytes(int B, int C, int G, int64_t n) {
    if (B <= 0 || C <= 0 || G <= 0 || C % G != 0 || n <= 0) return 0;
    const int64_t run = (int64_t)(C / G) * n;
    if (run <= kGnResidentFloats && n % 4 == 0) return 0;   // the register path needs none
    return gn_workspace_need((int64_t)B * G, run_chunks(run));
}

extern "C" dfp_status dfp_displaced_group_norm(float *y, const float *x, double *stats,
                                               const float *gamma, const float *beta, int B,
                                               int C, int G, int64_t n, int P, int p, float eps,
                                               int land, void *workspace, size_t ws_bytes,
                                               hipStream_t stream) {
    if (!y || !x || !stats) return DFP_ERR_INVALID_ARG;
    if (B <= 0 || C <= 0 || G <= 0 || C % G != 0 || n <= 0 || P <= 0 || p < 0 || p >= P)
        return DFP_ERR_INVALID_ARG;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return DFP_ERR_INVALID_ARG;
    if (!aligned(stats, 8)) return DFP_ERR_INVALID_ARG;
    if (B > 65535) return DFP_ERR_UNSUPPORTED;
    // partial overlap of y and x would let one workgroup read what another wrote
    const int64_t total = (int64_t)B * C * n;
    if (y != x && (const float *)y < x + total && x < (const float *)y + total)
        return DFP_ERR_INVALID_ARG;
    const bool affine = gamma || beta;
    GnArgs a{y, x, stats, gamma, beta, C, G, P, p, n, eps, land ? 1 : 0, 0};
    const int64_t run = (int64_t)(C / G) * n;
    const bool resident = n % 4 == 0 && run <= kGnResidentFloats && aligned(x, 16) &&
                          aligned(y, 16);
    const int64_t groups = (int64_t)B * G;
    const int64_t chunks = run_chunks(run);
    const bool chunked = !resident && G <= 65535 && workspace && aligned(workspace, 8) &&
                         ws_bytes >= gn_workspace_need(groups, chunks);
    const dim3 grid((unsigned)G, (unsigned)B), block(kGnThreads);
    if (chunked) {
        // y partially overlapping x is refused above; y == x (in place) is
        // safe: a chunk writes only the floats it read, after reading them
        double *partials = static_cast<double *>(workspace);
        const bool vec = n % 4 == 0 && aligned(x, 16) && aligned(y, 16);
        const dim3 cgrid((unsigned)chunks, (unsigned)G, (unsigned)B), cblock(kGcThreads);
        // x larger than the eight XCDs' L2s together (8 x 4 MiB): launch 2
        // starts from the chunks launch 1 read last, measured faster there
        // (the L2 miss counts stay the same: the misses are served faster).
        // For a smaller x the original order measured faster.
        a.reverse = total * 4 > (int64_t(32) << 20) && (chunks * groups) % 8 == 0 &&
                    chunks * groups < (int64_t(1) << 31);
        if (vec)
            hipLaunchKernelGGL(gn_chunk_sums_kernel<true>, cgrid, cblock, 0, stream, a, partials);
        else
            hipLaunchKernelGGL(gn_chunk_sums_kernel<false>, cgrid, cblock, 0, stream, a, partials);
        if (vec && affine)
            hipLaunchKernelGGL((gn_chunk_norm_kernel<true, true>), cgrid, cblock, 0, stream, a,
                               partials);
        else if (vec)
            hipLaunchKernelGGL((gn_chunk_norm_kernel<true, false>), cgrid, cblock, 0, stream, a,
                               partials);
        else if (affine)
            hipLaunchKernelGGL((gn_chunk_norm_kernel<false, true>), cgrid, cblock, 0, stream, a,
                               partials);
        else
            hipLaunchKernelGGL((gn_chunk_norm_kernel<false, false>), cgrid, cblock, 0, stream, a,
                               partials);
    } else if (resident) {
        if (affine) hipLaunchKernelGGL(gn_resident_kernel<true>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(gn_resident_kernel<false>, grid, block, 0, stream, a);
    } else {
        if (affine) hipLaunchKernelGGL(gn_stream_kernel<true>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(gn_stream_kernel<false>, grid, block, 0, stream, a);
    }
    return dfp::launch_status();
}
