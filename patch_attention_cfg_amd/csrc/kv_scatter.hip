// kv_scatter.hip -- land a patch's fresh K/V in the persistent buffer.
//
// "终极性能对比：DistriFusion vs 传统推理方案", "DistriFusion的革命性突破":
// after the warm-up steps each device reuses the previous step's activations
// for the other patches; its own patch region is refreshed every step.  The
// copy below is that refresh on the device: a bit-exact move of n rows per
// (batch, head), K row-major and V transposed (channel-major), with no
// arithmetic.  Both paths move 16-byte vectors; the V path transposes a
// 64 x 64 element tile through LDS so both its reads (along channels) and its
// writes (along tokens) stay coalesced.
#include "dfp_common.h"

namespace {

// K: every (b,h) owns one contiguous run of n*d elements in k_new and one in
// k_buf starting at row0*d; both runs are multiples of 16 bytes.
__global__ __launch_bounds__(256) void k_rows_copy(uint4 *__restrict__ dst,
                                                   const uint4 *__restrict__ src,
                                                   int64_t vec_per_bh,
                                                   int64_t dst_bh_stride_vec,
                                                   int64_t dst_off_vec,
                                                   int64_t total_vec) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total_vec; v += stride) {
        const int64_t bh = v / vec_per_bh;
        const int64_t r = v - bh * vec_per_bh;
        dst[bh * dst_bh_stride_vec + dst_off_vec + r] = src[v];
    }
}

// V: dst[bh][c][row0 + i] = src[bh][i][c] for i < n, c < d.
// Element type E is only a bit container (uint16_t for bf16, uint32_t for f32).
template <typename E>
__global__ __launch_bounds__(256) void v_transpose_copy(E *__restrict__ dst,
                                                        const E *__restrict__ src,
                                                        int n, int d, int64_t ldv,
                                                        int row0) {
    constexpr int T = 64;                      // tile edge (tokens x channels)
    constexpr int VE = 16 / sizeof(E);         // elements per 16-byte vector
    constexpr int PAD = 4 / sizeof(E) + 0;     // one dword of padding per row
    __shared__ E tile[T][T + PAD];

    const int i0 = blockIdx.x * T;             // token tile
    const int c0 = blockIdx.y * T;             // channel tile
    const int64_t bh = blockIdx.z;
    const E *s = src + bh * (int64_t)n * d;
    E *o = dst + bh * (int64_t)d * ldv;

    // load: rows i, 16-byte vectors along channels (d is a multiple of VE)
    constexpr int VPR = T / VE;                // vectors per tile row
    for (int t = threadIdx.x; t < T * VPR; t += blockDim.x) {
        const int i = t / VPR, cv = t - i * VPR;
        const int gi = i0 + i, gc = c0 + cv * VE;
        E vals[VE];
        if (gi < n && gc < d) {
            const uint4 q = *reinterpret_cast<const uint4 *>(s + (int64_t)gi * d + gc);
            __builtin_memcpy(vals, &q, 16);
        } else {
#pragma unroll
            for (int k = 0; k < VE; ++k) vals[k] = 0;
        }
#pragma unroll
        for (int k = 0; k < VE; ++k) tile[i][cv * VE + k] = vals[k];
    }
    __syncthreads();

    // store: channel rows c, VE consecutive tokens per thread
    const bool aligned = ((row0 + i0) % VE) == 0;
    for (int t = threadIdx.x; t < T * VPR; t += blockDim.x) {
        const int c = t / VPR, iv = t - c * VPR;
        const int gc = c0 + c, gi = i0 + iv * VE;
        if (gc >= d || gi >= n) continue;
        E *row = o + (int64_t)gc * ldv + row0 + gi;
        if (aligned && gi + VE <= n) {
            E vals[VE];
#pragma unroll
            for (int k = 0; k < VE; ++k) vals[k] = tile[iv * VE + k][c];
            uint4 q;
            __builtin_memcpy(&q, vals, 16);
            *reinterpret_cast<uint4 *>(row) = q;
        } else {
            for (int k = 0; k < VE && gi + k < n; ++k) row[k] = tile[iv * VE + k][c];
        }
    }
}

}  // namespace

extern "C" dfp_status dfp_kv_scatter(void *k_buf, void *v_buf_t, const void *k_new,
                                     const void *v_new, int B, int H, int N_buf, int d,
                                     int row0, int n, dfp_dtype dt, hipStream_t stream) {
    if (B <= 0 || H <= 0 || N_buf <= 0 || d <= 0 || n < 0 || row0 < 0 ||
        (int64_t)row0 + n > N_buf)
        return DFP_ERR_INVALID_ARG;
    if (n == 0) return DFP_OK;  // empty tensors may carry null data pointers
    if ((k_buf == nullptr) != (k_new == nullptr) || (v_buf_t == nullptr) != (v_new == nullptr))
        return DFP_ERR_INVALID_ARG;
    auto misaligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
    if (misaligned(k_buf) || misaligned(k_new) || misaligned(v_buf_t) || misaligned(v_new))
        return DFP_ERR_INVALID_ARG;
    if (dt != DFP_BF16 && dt != DFP_F32) return DFP_ERR_UNSUPPORTED;
    const int esize = dt == DFP_BF16 ? 2 : 4;
    const int VE = 16 / esize;
    if (d % VE != 0) return DFP_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    if (BH > 65535) return DFP_ERR_UNSUPPORTED;  // grid z limit of the V path

    if (k_buf) {
        const int64_t vec_per_row = (int64_t)d / VE;
        const int64_t vec_per_bh = vec_per_row * n;
        const int64_t total = vec_per_bh * BH;
        int64_t blocks = (total + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(k_rows_copy, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<uint4 *>(k_buf), static_cast<const uint4 *>(k_new),
                           vec_per_bh, vec_per_row * N_buf, vec_per_row * row0, total);
        if (dfp::launch_status() != DFP_OK) return DFP_ERR_HIP;
    }
    if (v_buf_t) {
        const int64_t ldv = dfp_v_ld(N_buf, dt);
        dim3 grid((unsigned)((n + 63) / 64), (unsigned)((d + 63) / 64), (unsigned)BH);
        if (dt == DFP_BF16)
            hipLaunchKernelGGL(v_transpose_copy<uint16_t>, grid, dim3(256), 0, stream,
                               static_cast<uint16_t *>(v_buf_t),
                               static_cast<const uint16_t *>(v_new), n, d, ldv, row0);
        else
            hipLaunchKernelGGL(v_transpose_copy<uint32_t>, grid, dim3(256), 0, stream,
                               static_cast<uint32_t *>(v_buf_t),
                               static_cast<const uint32_t *>(v_new), n, d, ldv, row0);
        if (dfp::launch_status() != DFP_OK) return DFP_ERR_HIP;
    }
    return DFP_OK;
}
