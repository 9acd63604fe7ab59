// attention.hip -- C-ABI entry points of patch attention, and the fp32 path.
//
// dfp_patch_attention validates its arguments and dispatches to the bf16
// matrix-core kernel (attention_bf16.hip) or to the fp32 kernel below;
// dfp_patch_attention_fresh runs the bf16 kernel with the patch's fresh
// rows read from this step's tensors (and landed in the buffer by the same
// launch).  The
// fp32 kernel exists for full-precision checks of the method on small
// workloads; it is plain vector-ALU code (one query per lane, online
// softmax, K and V^T tiles broadcast from LDS) with no performance target.
//
// What is computed ("终极性能对比：DistriFusion vs 传统推理方案",
// "DistriFusion的革命性突破"): softmax attention of the patch's queries over
// every row of the displaced buffer (fresh rows for the patch, previous-step
// rows elsewhere).
#include <cmath>

#include "dfp_common.h"
#include "dfp_internal.h"

namespace {

constexpr int kF32Keys = 32;     // keys per LDS tile
constexpr int kF32Threads = 64;  // one wavefront, one query per lane

template <int D>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ Vt,
    float *__restrict__ O, int n_q, int N_kv, int64_t ldv, float c_log2, int q_tiles) {
    __shared__ __attribute__((aligned(16))) float Ks[kF32Keys][D];
    __shared__ __attribute__((aligned(16))) float Vs[D][kF32Keys];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x / q_tiles;
    const int qt = blockIdx.x - bh * q_tiles;
    const float *Kh = K + (int64_t)bh * N_kv * D;
    const float *Vh = Vt + (int64_t)bh * D * ldv;
    const int q_row = qt * kF32Threads + tid;
    const bool q_valid = q_row < n_q;

    float q[D], o[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        q[c] = q_valid ? Q[((int64_t)bh * n_q + q_row) * D + c] : 0.f;
        o[c] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    for (int j0 = 0; j0 < N_kv; j0 += kF32Keys) {
        __syncthreads();  // previous tile fully consumed
        for (int e = tid; e < kF32Keys * D / 4; e += kF32Threads) {
            const int row = e / (D / 4), col = (e % (D / 4)) * 4;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j0 + row < N_kv)
                kv = *reinterpret_cast<const float4 *>(Kh + (int64_t)(j0 + row) * D + col);
            *reinterpret_cast<float4 *>(&Ks[row][col]) = kv;
        }
        for (int e = tid; e < D * kF32Keys / 4; e += kF32Threads) {
            const int row = e / (kF32Keys / 4), col = (e % (kF32Keys / 4)) * 4;
            float vals[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                vals[k] = (j0 + col + k < N_kv) ? Vh[(int64_t)row * ldv + j0 + col + k] : 0.f;
            *reinterpret_cast<float4 *>(&Vs[row][col]) =
                make_float4(vals[0], vals[1], vals[2], vals[3]);
        }
        __syncthreads();

        float s[kF32Keys];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kF32Keys; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) acc = fmaf(q[c], Ks[j][c], acc);
            s[j] = (j0 + j < N_kv) ? acc : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx * c_log2);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < kF32Keys; ++j) {
            s[j] = exp2f(fmaf(s[j], c_log2, -m_new));
            lsum += s[j];
        }
        l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
        for (int c = 0; c < D; ++c) {
            float acc = o[c] * alpha;
#pragma unroll
            for (int j = 0; j < kF32Keys; ++j) acc = fmaf(s[j], Vs[c][j], acc);
            o[c] = acc;
        }
    }

    if (q_valid) {
        const float inv = 1.0f / l_run;
        float *orow = O + ((int64_t)bh * n_q + q_row) * D;
#pragma unroll
        for (int c = 0; c < D; c += 4)
            *reinterpret_cast<float4 *>(orow + c) =
                make_float4(o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv);
    }
}

dfp_status attn_f32_launch(void *o, const void *q, const void *k, const void *vt, int BH,
                           int n_q, int N_kv, int d, float scale, hipStream_t stream) {
    const int q_tiles = (n_q + kF32Threads - 1) / kF32Threads;
    const int64_t blocks = (int64_t)q_tiles * BH;
    if (blocks > 0x7FFFFFFF) return DFP_ERR_UNSUPPORTED;
    const int64_t ldv = dfp_v_ld(N_kv, DFP_F32);
    const float c_log2 = scale * 1.4426950408889634f;
    if (d == 64)
        hipLaunchKernelGGL(attn_fwd_f32<64>, dim3((unsigned)blocks), dim3(kF32Threads), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(vt), static_cast<float *>(o), n_q, N_kv,
                           ldv, c_log2, q_tiles);
    else if (d == 128)
        hipLaunchKernelGGL(attn_fwd_f32<128>, dim3((unsigned)blocks), dim3(kF32Threads), 0,
                           stream, static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(vt), static_cast<float *>(o), n_q, N_kv,
                           ldv, c_log2, q_tiles);
    else
        return DFP_ERR_UNSUPPORTED;
    return dfp::launch_status();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" dfp_status dfp_patch_attention(void *o, const void *q, const void *k_buf,
                                          const void *v_buf_t, int B, int H, int n_q, int N_kv,
                                          int d, float scale, dfp_dtype dt, void *workspace,
                                          size_t ws_bytes, hipStream_t stream) {
    if (B <= 0 || H <= 0 || N_kv <= 0 || n_q < 0) return DFP_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !std::isfinite(scale)) return DFP_ERR_INVALID_ARG;
    if (dt != DFP_BF16 && dt != DFP_F32) return DFP_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return DFP_ERR_UNSUPPORTED;
    if (n_q == 0) return DFP_OK;  // empty tensors may carry null data pointers
    if (!o || !q || !k_buf || !v_buf_t) return DFP_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(q) || !aligned16(k_buf) || !aligned16(v_buf_t))
        return DFP_ERR_INVALID_ARG;
    const int64_t BH = (int64_t)B * H;
    if (BH > 0x7FFFFFFF) return DFP_ERR_UNSUPPORTED;
    if (dt == DFP_BF16)
        return dfp_attn_bf16_launch(o, q, k_buf, v_buf_t, (int)BH, n_q, N_kv, d, scale, workspace,
                                    ws_bytes, nullptr, stream);
    return attn_f32_launch(o, q, k_buf, v_buf_t, (int)BH, n_q, N_kv, d, scale, stream);
}

extern "C" dfp_status dfp_patch_attention_fresh(void *o, const void *q, void *k_buf, void *v_buf_t,
                                                const dfp_fresh_rows *fresh, int n_fresh, int B,
                                                int H, int n_q, int N_kv, int d, int land,
                                                float scale, dfp_dtype dt, void *workspace,
                                                size_t ws_bytes, hipStream_t stream) {
    if (B <= 0 || H <= 0 || N_kv <= 0 || n_q < 0) return DFP_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !std::isfinite(scale)) return DFP_ERR_INVALID_ARG;
    if (!fresh || n_fresh < 1) return DFP_ERR_INVALID_ARG;
    if (n_fresh > 2) return DFP_ERR_UNSUPPORTED;
    for (int r = 0; r < n_fresh; ++r) {
        const dfp_fresh_rows &f = fresh[r];
        if (f.row0 < 0 || f.n <= 0 || (int64_t)f.row0 + f.n > N_kv) return DFP_ERR_INVALID_ARG;
        if (!f.k || !f.v_t || !aligned16(f.k) || !aligned16(f.v_t)) return DFP_ERR_INVALID_ARG;
    }
    if (n_fresh == 2 && fresh[0].row0 < fresh[1].row0 + fresh[1].n &&
        fresh[1].row0 < fresh[0].row0 + fresh[0].n)
        return DFP_ERR_INVALID_ARG;   // overlapping ranges
    if (dt != DFP_BF16) return DFP_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return DFP_ERR_UNSUPPORTED;
    for (int r = 0; r < n_fresh; ++r)
        if (fresh[r].row0 % 64 != 0 || fresh[r].n % 64 != 0) return DFP_ERR_UNSUPPORTED;
    if (n_q == 0 && !land) return DFP_OK;
    if (!k_buf || !v_buf_t || !aligned16(k_buf) || !aligned16(v_buf_t))
        return DFP_ERR_INVALID_ARG;
    if (n_q > 0 && (!o || !q || !aligned16(o) || !aligned16(q))) return DFP_ERR_INVALID_ARG;
    const int64_t BH = (int64_t)B * H;
    if (BH > 0x7FFFFFFF) return DFP_ERR_UNSUPPORTED;
    const dfp_fresh_launch launch{fresh, n_fresh, k_buf, v_buf_t, land ? 1 : 0};
    return dfp_attn_bf16_launch(o, q, k_buf, v_buf_t, (int)BH, n_q, N_kv, d, scale, workspace,
                                ws_bytes, &launch, stream);
}

extern "C" dfp_status dfp_attention_plan(int B, int H, int n_q, int N_kv, int d, int with_workspace,
                                         int *key_groups, int *splits, int64_t *workgroups) {
    if (B <= 0 || H <= 0 || n_q <= 0 || N_kv <= 0) return DFP_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return DFP_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    if (BH > 0x7FFFFFFF) return DFP_ERR_UNSUPPORTED;
    int ks = 1, sp = 1;
    int64_t wg = 0;
    dfp_attn_bf16_plan((int)BH, n_q, N_kv, d, with_workspace != 0, &ks, &sp, &wg);
    if (key_groups) *key_groups = ks;
    if (splits) *splits = sp;
    if (workgroups) *workgroups = wg;
    return DFP_OK;
}
