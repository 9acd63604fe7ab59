// kv_scatter.hip -- land a patch's fresh K/V in the persistent buffer.
//
// "终极性能对比：DistriFusion vs 传统推理方案", "DistriFusion的革命性突破":
// after the warm-up steps each device reuses the previous step's activations
// for the other patches; its own patch region is refreshed every step.  The
// copy below is that refresh on the device: a bit-exact move of n rows per
// (batch, head), K row-major and V transposed (channel-major), with no
// arithmetic.  Both paths move 16-byte vectors; the V path transposes a
// 64 x 64 element tile through LDS so both its reads (along channels) and its
// writes (along tokens) stay coalesced.  K and V share one launch (the copy
// is latency-bound at these sizes, so a second launch would cost as much as
// the data).  The fresh rows may come in any layout whose rows of d elements
// are contiguous and 16-byte aligned (element strides per batch, head and
// row): [B][H][n][d] and a projection's [B][n][H][d] alike.
#include "dfp_common.h"

namespace {

struct ScatterArgs {
    uint4 *k_dst;             // K buffer, 16-byte vectors
    const uint4 *k_src;
    int64_t k_vec_per_bh;     // n * d / VE
    int64_t k_dst_bh_stride;  // N_buf * d / VE
    int64_t k_dst_off;        // row0 * d / VE
    int64_t k_total;          // BH * k_vec_per_bh
    void *v_dst;              // V^T buffer [BH][d][ldv]
    const void *v_src;        // fresh V rows, element strides below
    int n, d, row0, H;
    int64_t ldv;
    int64_t sb, sh, sn;       // fresh rows' element strides: batch, head, row
    int vec_per_row;          // d / VE
    int dense;                // fresh rows are [B][H][n][d] with no gaps
    int v_tiles_i, v_tiles_c;   // 64-token and 64-channel tiles per (b,h)
    int v_blocks;               // blocks [0, v_blocks) transpose V; the rest copy K
};

// Element offset of fresh row i of (b,h) = bh.
__device__ __forceinline__ int64_t src_row(const ScatterArgs &a, int64_t bh, int64_t i) {
    const int64_t b = bh / a.H, h = bh - b * a.H;
    return b * a.sb + h * a.sh + i * a.sn;
}

// K: every (b,h) owns rows row0.. of its k_buf run; a dense source is one
// contiguous run of n*d elements per (b,h), a strided one n rows of d.
template <int VE>
__device__ __forceinline__ void k_rows_copy(const ScatterArgs &a, int64_t first, int64_t stride) {
    for (int64_t v = first; v < a.k_total; v += stride) {
        const int64_t bh = v / a.k_vec_per_bh;
        const int64_t r = v - bh * a.k_vec_per_bh;
        uint4 q;
        if (a.dense) {
            q = a.k_src[v];
        } else {
            const int64_t i = r / a.vec_per_row, cv = r - i * a.vec_per_row;
            q = a.k_src[(src_row(a, bh, i) >> (VE == 8 ? 3 : 2)) + cv];
        }
        a.k_dst[bh * a.k_dst_bh_stride + a.k_dst_off + r] = q;
    }
}

// V: dst[bh][c][row0 + i] = src[bh][i][c] for one 64 x 64 (token x channel)
// tile.  Element type E is only a bit container (uint16_t for bf16,
// uint32_t for f32).
template <typename E>
__device__ __forceinline__ void v_tile_transpose(const ScatterArgs &a, int tile) {
    constexpr int T = 64;                      // tile edge (tokens x channels)
    constexpr int VE = 16 / sizeof(E);         // elements per 16-byte vector
    constexpr int PAD = 4 / sizeof(E);         // one dword of padding per row
    __shared__ E sm_tile[T][T + PAD];

    const int ti = tile % a.v_tiles_i;
    const int rest = tile / a.v_tiles_i;
    const int tc = rest % a.v_tiles_c;
    const int64_t bh = rest / a.v_tiles_c;
    const int i0 = ti * T, c0 = tc * T;
    const int n = a.n, d = a.d;
    const E *s = static_cast<const E *>(a.v_src) + src_row(a, bh, 0);
    E *o = static_cast<E *>(a.v_dst) + bh * (int64_t)d * a.ldv;

    // load: rows i, 16-byte vectors along channels (d is a multiple of VE)
    constexpr int VPR = T / VE;                // vectors per tile row
    for (int t = threadIdx.x; t < T * VPR; t += blockDim.x) {
        const int i = t / VPR, cv = t - i * VPR;
        const int gi = i0 + i, gc = c0 + cv * VE;
        E vals[VE];
        if (gi < n && gc < d) {
            const uint4 q = *reinterpret_cast<const uint4 *>(s + (int64_t)gi * a.sn + gc);
            __builtin_memcpy(vals, &q, 16);
        } else {
#pragma unroll
            for (int k = 0; k < VE; ++k) vals[k] = 0;
        }
#pragma unroll
        for (int k = 0; k < VE; ++k) sm_tile[i][cv * VE + k] = vals[k];
    }
    __syncthreads();

    // store: channel rows c, VE consecutive tokens per thread
    const bool aligned = ((a.row0 + i0) % VE) == 0;
    for (int t = threadIdx.x; t < T * VPR; t += blockDim.x) {
        const int c = t / VPR, iv = t - c * VPR;
        const int gc = c0 + c, gi = i0 + iv * VE;
        if (gc >= d || gi >= n) continue;
        E *row = o + (int64_t)gc * a.ldv + a.row0 + gi;
        if (aligned && gi + VE <= n) {
            E vals[VE];
#pragma unroll
            for (int k = 0; k < VE; ++k) vals[k] = sm_tile[iv * VE + k][c];
            uint4 q;
            __builtin_memcpy(&q, vals, 16);
            *reinterpret_cast<uint4 *>(row) = q;
        } else {
            for (int k = 0; k < VE && gi + k < n; ++k) row[k] = sm_tile[iv * VE + k][c];
        }
    }
}

// One launch lands both K and V: the first v_blocks workgroups transpose one
// V tile each, the others copy K rows (grid-stride).
template <typename E>
__global__ __launch_bounds__(256) void kv_scatter_kernel(ScatterArgs a) {
    if ((int)blockIdx.x < a.v_blocks) {
        v_tile_transpose<E>(a, blockIdx.x);
    } else {
        const int64_t kb = blockIdx.x - a.v_blocks;
        const int64_t k_blocks = gridDim.x - a.v_blocks;
        k_rows_copy<16 / sizeof(E)>(a, kb * blockDim.x + threadIdx.x, k_blocks * blockDim.x);
    }
}

}  // namespace

extern "C" dfp_status dfp_kv_scatter_strided(void *k_buf, void *v_buf_t, const void *k_new,
                                             const void *v_new, int B, int H, int N_buf, int d,
                                             int row0, int n, int64_t stride_b,
                                             int64_t stride_h, int64_t stride_n, dfp_dtype dt,
                                             hipStream_t stream) {
    if (B <= 0 || H <= 0 || N_buf <= 0 || d <= 0 || n < 0 || row0 < 0 ||
        (int64_t)row0 + n > N_buf)
        return DFP_ERR_INVALID_ARG;
    if (n == 0) return DFP_OK;  // empty tensors may carry null data pointers
    if ((k_buf == nullptr) != (k_new == nullptr) || (v_buf_t == nullptr) != (v_new == nullptr))
        return DFP_ERR_INVALID_ARG;
    if (!k_buf && !v_buf_t) return DFP_OK;
    auto misaligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
    if (misaligned(k_buf) || misaligned(k_new) || misaligned(v_buf_t) || misaligned(v_new))
        return DFP_ERR_INVALID_ARG;
    if (dt != DFP_BF16 && dt != DFP_F32) return DFP_ERR_UNSUPPORTED;
    const int esize = dt == DFP_BF16 ? 2 : 4;
    const int VE = 16 / esize;
    if (d % VE != 0) return DFP_ERR_UNSUPPORTED;
    // every fresh row must start on a 16-byte boundary
    if (stride_b < 0 || stride_h < 0 || stride_n < d || stride_b % VE || stride_h % VE ||
        stride_n % VE)
        return DFP_ERR_INVALID_ARG;
    const int64_t BH = (int64_t)B * H;

    ScatterArgs a{};
    a.n = n;
    a.d = d;
    a.row0 = row0;
    a.H = H;
    a.sb = stride_b;
    a.sh = stride_h;
    a.sn = stride_n;
    a.vec_per_row = d / VE;
    a.dense = stride_n == d && (H == 1 || stride_h == (int64_t)n * d) &&
              (B == 1 || stride_b == (int64_t)H * n * d);
    int64_t k_blocks = 0, v_blocks = 0;
    if (k_buf) {
        const int64_t vec_per_row = (int64_t)d / VE;
        a.k_dst = static_cast<uint4 *>(k_buf);
        a.k_src = static_cast<const uint4 *>(k_new);
        a.k_vec_per_bh = vec_per_row * n;
        a.k_dst_bh_stride = vec_per_row * N_buf;
        a.k_dst_off = vec_per_row * row0;
        a.k_total = a.k_vec_per_bh * BH;
        k_blocks = (a.k_total + 255) / 256;
        if (k_blocks > 8192) k_blocks = 8192;
    }
    if (v_buf_t) {
        a.v_dst = v_buf_t;
        a.v_src = v_new;
        a.ldv = dfp_v_ld(N_buf, dt);
        a.v_tiles_i = (n + 63) / 64;
        a.v_tiles_c = (d + 63) / 64;
        v_blocks = (int64_t)a.v_tiles_i * a.v_tiles_c * BH;
    }
    if (v_blocks + k_blocks > 0x7FFFFFFF) return DFP_ERR_UNSUPPORTED;
    a.v_blocks = (int)v_blocks;
    const dim3 grid((unsigned)(v_blocks + k_blocks));
    if (dt == DFP_BF16)
        hipLaunchKernelGGL(kv_scatter_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(kv_scatter_kernel<uint32_t>, grid, dim3(256), 0, stream, a);
    return dfp::launch_status();
}

extern "C" dfp_status dfp_kv_scatter(void *k_buf, void *v_buf_t, const void *k_new,
                                     const void *v_new, int B, int H, int N_buf, int d,
                                     int row0, int n, dfp_dtype dt, hipStream_t stream) {
    return dfp_kv_scatter_strided(k_buf, v_buf_t, k_new, v_new, B, H, N_buf, d, row0, n,
                                  (int64_t)H * n * d, (int64_t)n * d, d, dt, stream);
}
