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
// floats.  Runs of up to 64 Ki floats: one workgroup per (image, group)
// keeps its run in registers between the two uses (one read of x).  Longer
// runs, given a workspace: two launches over chunks of every run, across
// the whole GPU -- partial sums published per chunk, the last chunk of each
// group to arrive forms the statistics (and lands the fresh sums); then
// every chunk normalizes.  Without a workspace one workgroup streams each
// run twice.  Sums are fp64 per thread, per wavefront (fixed butterfly) and
// across wavefronts and chunks in a fixed order, so the statistics are
// bitwise reproducible.
#include <cmath>

#include "dfp_common.h"

namespace {

constexpr int kGnThreads = 1024;
constexpr int kGnWaves = kGnThreads / dfp::kWave;
constexpr int kGnVec = 16;   // float4 per thread held in registers
constexpr int64_t kGnResidentFloats = (int64_t)kGnThreads * kGnVec * 4;
// Chunked path: 256-thread workgroups over 16 Ki-float chunks (16 floats per
// thread per pass), at most kGnMaxChunks per run.
constexpr int kGcThreads = 256;
constexpr int kGcWaves = kGcThreads / dfp::kWave;
constexpr int64_t kGcChunk = (int64_t)kGcThreads * 16 * 4;
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
size_t gn_counter_bytes(int64_t groups) { return ((size_t)groups * 4 + 255) / 256 * 256; }
size_t gn_workspace_need(int64_t groups, int64_t chunks) {
    return gn_counter_bytes(groups) + (size_t)groups * chunks * 2 * sizeof(double) +
           (size_t)groups * 2 * sizeof(float);
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

// The group's (mean, rstd) from its fresh sums (f1, f2) and the other
// patches' stale sums; the fresh sums land in the patch's slot.
__device__ __forceinline__ float2 stats_from_sums(const GnArgs &a, int b, int g, double f1,
                                                  double f2) {
    double *st = a.stats + ((int64_t)b * a.G + g) * a.P * 2;
    double t1 = f1, t2 = f2;
    for (int q = 0; q < a.P; ++q)
        if (q != a.p) {
            t1 += st[2 * q];
            t2 += st[2 * q + 1];
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
                                              double s2) {
    __shared__ float mean_rstd[2];
    block_sums<kGnWaves>(s1, s2);
    if (threadIdx.x == 0) {
        const float2 mr = stats_from_sums(a, b, g, s1, s2);
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

template <bool AFFINE>
__device__ __forceinline__ float4 normalize4(const GnArgs &a, float4 v, int c, float2 mr) {
    const float ga = AFFINE && a.gamma ? a.gamma[c] : 1.f;
    const float be = AFFINE && a.beta ? a.beta[c] : 0.f;
    const float sc = mr.y * ga;
    return make_float4((v.x - mr.x) * sc + be, (v.y - mr.x) * sc + be, (v.z - mr.x) * sc + be,
                       (v.w - mr.x) * sc + be);
}

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
    float4 v[kGnVec];
#pragma unroll
    for (int k = 0; k < kGnVec; ++k) {
        const int i = tid + k * kGnThreads;
        v[k] = i < len4 ? xg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int k = 0; k < kGnVec; ++k) accum4(s1, s2, v[k]);
    const float2 mr = group_stats(a, b, g, s1, s2);
    float4 *yg = reinterpret_cast<float4 *>(a.y + off);
#pragma unroll
    for (int k = 0; k < kGnVec; ++k) {
        const int i = tid + k * kGnThreads;
        if (i < len4) yg[i] = normalize4<AFFINE>(a, v[k], g * cg + i / n4, mr);
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
    const float2 mr = group_stats(a, b, g, s1, s2);
    float *yg = a.y + off;
    for (int64_t i = tid; i < len; i += kGnThreads) {
        const int c = g * cg + (int)(i / a.n);
        const float ga = AFFINE && a.gamma ? a.gamma[c] : 1.f;
        const float be = AFFINE && a.beta ? a.beta[c] : 0.f;
        yg[i] = (xg[i] - mr.x) * (mr.y * ga) + be;
    }
}

// Chunked path, launch 1: chunk blockIdx.x of group (blockIdx.y, blockIdx.z)
// sums its floats and publishes them; the last chunk of the group to
// arrive adds the chunks' sums in chunk order, forms the statistics, lands
// the fresh sums and resets the counter.  VEC: float4 loads (n % 4 == 0,
// x 16-byte aligned).
template <bool VEC>
__global__ __launch_bounds__(kGcThreads) void gn_chunk_sums_kernel(GnArgs a, double *partials,
                                                                   unsigned *counters,
                                                                   float *mean_rstd) {
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
    __shared__ int is_last;
    const int64_t grp = (int64_t)b * a.G + g;
    if (tid == 0) {
        double *pp = partials + (grp * nch + chunk) * 2;
        dfp::publish(pp, s1);
        dfp::publish(pp + 1, s2);
        dfp::published_wait();
        is_last = dfp::arrive(counters + grp) == (unsigned)nch - 1;
    }
    __syncthreads();
    if (!is_last || tid != 0) return;
    double f1 = 0.0, f2 = 0.0;
    for (int k = 0; k < nch; ++k) {
        f1 += dfp::fetch_published(partials + (grp * nch + k) * 2);
        f2 += dfp::fetch_published(partials + (grp * nch + k) * 2 + 1);
    }
    const float2 mr = stats_from_sums(a, b, g, f1, f2);
    mean_rstd[grp * 2] = mr.x;
    mean_rstd[grp * 2 + 1] = mr.y;
    dfp::publish(counters + grp, 0u);
}

// Chunked path, launch 2: every chunk normalizes its floats.
template <bool VEC, bool AFFINE>
__global__ __launch_bounds__(kGcThreads) void gn_chunk_norm_kernel(GnArgs a,
                                                                   const float *mean_rstd) {
    const int chunk = blockIdx.x, nch = gridDim.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int cg = a.C / a.G;
    const int64_t run = (int64_t)cg * a.n;
    const int64_t per = chunk_span(run, nch, VEC);
    const int64_t lo = min(run, (int64_t)chunk * per), hi = min(run, lo + per);
    const int64_t off = ((int64_t)b * a.C + (int64_t)g * cg) * a.n;
    const int64_t grp = (int64_t)b * a.G + g;
    const float2 mr = make_float2(mean_rstd[grp * 2], mean_rstd[grp * 2 + 1]);
    if (VEC) {
        const float4 *x4 = reinterpret_cast<const float4 *>(a.x + off + lo);
        float4 *y4 = reinterpret_cast<float4 *>(a.y + off + lo);
        const int64_t m4 = (hi - lo) / 4;
        for (int64_t i = tid; i < m4; i += kGcThreads)
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
    if (run <= kGnResidentFloats) return 0;
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
    GnArgs a{y, x, stats, gamma, beta, C, G, P, p, n, eps, land ? 1 : 0};
    const int64_t run = (int64_t)(C / G) * n;
    const bool resident = n % 4 == 0 && run <= kGnResidentFloats && aligned(x, 16) &&
                          aligned(y, 16);
    const int64_t groups = (int64_t)B * G;
    const int64_t chunks = run_chunks(run);
    const bool chunked = !resident && run > kGnResidentFloats && G <= 65535 && workspace &&
                         aligned(workspace, 256) &&
                         ws_bytes >= gn_workspace_need(groups, chunks);
    const dim3 grid((unsigned)G, (unsigned)B), block(kGnThreads);
    if (chunked) {
        unsigned *counters = static_cast<unsigned *>(workspace);
        double *partials = reinterpret_cast<double *>(static_cast<char *>(workspace) +
                                                      gn_counter_bytes(groups));
        float *mr = reinterpret_cast<float *>(partials + groups * chunks * 2);
        const bool vec = n % 4 == 0 && aligned(x, 16) && aligned(y, 16);
        const dim3 cgrid((unsigned)chunks, (unsigned)G, (unsigned)B), cblock(kGcThreads);
        if (vec)
            hipLaunchKernelGGL(gn_chunk_sums_kernel<true>, cgrid, cblock, 0, stream, a, partials,
                               counters, mr);
        else
            hipLaunchKernelGGL(gn_chunk_sums_kernel<false>, cgrid, cblock, 0, stream, a, partials,
                               counters, mr);
        if (vec && affine)
            hipLaunchKernelGGL((gn_chunk_norm_kernel<true, true>), cgrid, cblock, 0, stream, a, mr);
        else if (vec)
            hipLaunchKernelGGL((gn_chunk_norm_kernel<true, false>), cgrid, cblock, 0, stream, a, mr);
        else if (affine)
            hipLaunchKernelGGL((gn_chunk_norm_kernel<false, true>), cgrid, cblock, 0, stream, a, mr);
        else
            hipLaunchKernelGGL((gn_chunk_norm_kernel<false, false>), cgrid, cblock, 0, stream, a,
                               mr);
    } else if (resident) {
        if (affine) hipLaunchKernelGGL(gn_resident_kernel<true>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(gn_resident_kernel<false>, grid, block, 0, stream, a);
    } else {
        if (affine) hipLaunchKernelGGL(gn_stream_kernel<true>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(gn_stream_kernel<false>, grid, block, 0, stream, a);
    }
    return dfp::launch_status();
}
