// attention_bf16.hip -- one patch's queries attending over the displaced
// full-image K/V buffer, bf16 in / bf16 out, fp32 accumulation, on CDNA4
// matrix cores (v_mfma_f32_32x32x16_bf16).
//
// What is computed ("终极性能对比：DistriFusion vs 传统推理方案",
// "DistriFusion的革命性突破"; "xDiT: an Inference Engine for Diffusion
// Transformers (DiTs) with Massive Parallelism", 三.2): the buffer already
// holds this step's K/V for the patch's own rows and the previous step's
// K/V for every other row, so the patch's output is plain softmax attention
// over all N_kv buffer rows.  The kernel streams the buffer tile by tile
// with an online (running max / running sum) softmax, so its memory is
// O(tile) whatever N_kv is, and the result equals two-pass softmax up to
// rounding.
//
// Layout of the work (per workgroup: 4 wavefronts x 32 query rows):
//   * Each wavefront keeps its 32 queries in registers as the B operand of
//     S^T = K Q^T (32 keys x 32 queries per MFMA block).  Computing S^T
//     rather than S leaves every score of one query in one lane pair
//     (lane l and l^32), so the row max needs one cross-lane exchange and
//     the probabilities are already in the B-operand layout of
//     O^T = V^T P^T -- no LDS round trip and no transpose for P.
//   * K tiles sit in LDS row-major [key][d]; V is stored transposed in HBM
//     ([d][token], see dfp.h) so V^T tiles land in LDS as [d][key] and feed
//     the A operand of O^T = V^T P^T with plain 8-byte reads.
//   * LDS rows are padded (K: +16 B, V^T: +8 B) so the 32 rows one MFMA
//     operand read touches fall in distinct banks.
//   * Two LDS stages: the next tile's global loads are issued before the
//     current tile's math and stored after it (one barrier per tile).
//   * exp(x) is evaluated as exp2 with log2(e) * scale folded into one FMA.
#include <cmath>

#include "dfp_common.h"
#include "dfp_internal.h"

namespace {

using dfp::bf16x8_t;
using dfp::f32x16_t;

constexpr int kWaves = 4;
constexpr int kQPW = 32;                  // query rows per wavefront
constexpr int kBlockM = kWaves * kQPW;    // query rows per workgroup
constexpr int kBlockN = 64;               // keys per tile
constexpr int kThreads = kWaves * dfp::kWave;

template <int D>
struct Smem {
    static constexpr int K_LD = D + 8;            // bf16 per K row in LDS
    static constexpr int V_LD = kBlockN + 4;      // bf16 per V^T row in LDS
    static constexpr int K_TILE = kBlockN * K_LD;
    static constexpr int V_TILE = D * V_LD;
    static constexpr int STAGE = K_TILE + V_TILE;
    static constexpr int K_CHUNKS = kBlockN * D / 8 / kThreads;  // 16-byte chunks per thread
    static constexpr int V_CHUNKS = D * kBlockN / 8 / kThreads;
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Zero the bf16 lanes of a 16-byte chunk whose key index is >= N_kv.
__device__ __forceinline__ uint4 mask_keys(uint4 v, int key0, int N_kv) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k_lo = key0 + 2 * e, k_hi = k_lo + 1;
        uint32_t lo = k_lo < N_kv ? (w[e] & 0xFFFFu) : 0u;
        uint32_t hi = k_hi < N_kv ? (w[e] & 0xFFFF0000u) : 0u;
        w[e] = lo | hi;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int D>
struct TileLoader {
    uint4 k[Smem<D>::K_CHUNKS];
    uint4 v[Smem<D>::V_CHUNKS];

    // Global -> registers for the tile starting at key j0.
    __device__ __forceinline__ void load(const uint16_t *__restrict__ Kh,
                                         const uint16_t *__restrict__ Vh, int j0, int N_kv,
                                         int64_t ldv, int tid) {
        constexpr int KCPR = D / 8;  // K chunks per key row
#pragma unroll
        for (int c = 0; c < Smem<D>::K_CHUNKS; ++c) {
            const int idx = tid + c * kThreads;
            const int row = idx / KCPR, col = idx % KCPR;
            const int key = j0 + row;
            k[c] = key < N_kv
                       ? *reinterpret_cast<const uint4 *>(Kh + (int64_t)key * D + col * 8)
                       : zero4();
        }
        constexpr int VCPR = kBlockN / 8;  // V^T chunks per channel row
#pragma unroll
        for (int c = 0; c < Smem<D>::V_CHUNKS; ++c) {
            const int idx = tid + c * kThreads;
            const int row = idx / VCPR, col = idx % VCPR;
            const int key0 = j0 + col * 8;
            if (key0 + 8 <= N_kv)
                v[c] = *reinterpret_cast<const uint4 *>(Vh + (int64_t)row * ldv + key0);
            else if (key0 < N_kv)  // ldv pads rows to 8 keys: the read stays in the row
                v[c] = mask_keys(*reinterpret_cast<const uint4 *>(Vh + (int64_t)row * ldv + key0),
                                 key0, N_kv);
            else
                v[c] = zero4();
        }
    }

    // Registers -> LDS stage.
    __device__ __forceinline__ void store(uint16_t *stage, int tid) const {
        constexpr int KCPR = D / 8;
        uint16_t *Ks = stage;
        uint16_t *Vs = stage + Smem<D>::K_TILE;
#pragma unroll
        for (int c = 0; c < Smem<D>::K_CHUNKS; ++c) {
            const int idx = tid + c * kThreads;
            const int row = idx / KCPR, col = idx % KCPR;
            *reinterpret_cast<uint4 *>(Ks + row * Smem<D>::K_LD + col * 8) = k[c];
        }
        constexpr int VCPR = kBlockN / 8;
#pragma unroll
        for (int c = 0; c < Smem<D>::V_CHUNKS; ++c) {
            const int idx = tid + c * kThreads;
            const int row = idx / VCPR, col = idx % VCPR;
            // V^T rows are 8-byte aligned in LDS (V_LD*2 = 136 B): two 8-byte stores
            uint2 *dst = reinterpret_cast<uint2 *>(Vs + row * Smem<D>::V_LD + col * 8);
            dst[0] = make_uint2(v[c].x, v[c].y);
            dst[1] = make_uint2(v[c].z, v[c].w);
        }
    }
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
    bf16x8_t r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ Vt, uint16_t *__restrict__ O, int n_q, int N_kv, int64_t ldv,
    float c_log2, int q_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<D>::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;   // query column of this lane in every MFMA block
    const int g = lane >> 5;    // which half of the K=16 slice this lane feeds

    const int bh = blockIdx.x / q_tiles;
    const int qt = blockIdx.x - bh * q_tiles;
    const uint16_t *Qh = Q + (int64_t)bh * n_q * D;
    const uint16_t *Kh = K + (int64_t)bh * N_kv * D;
    const uint16_t *Vh = Vt + (int64_t)bh * D * ldv;
    const int q_row = qt * kBlockM + wave * kQPW + ql;
    const bool q_valid = q_row < n_q;

    // Q^T as the B operand: lane (ql, g) holds d = kc*16 + g*8 .. +7 of its query.
    bf16x8_t qreg[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
        qreg[kc] = as_bf16x8(q_valid ? *reinterpret_cast<const uint4 *>(
                                           Qh + (int64_t)q_row * D + kc * 16 + g * 8)
                                     : zero4());

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY;  // running max, in log2 units (scores * c_log2)
    float l_run = 0.f;        // this lane's share of the running sum

    const int ntiles = (N_kv + kBlockN - 1) / kBlockN;
    TileLoader<D> ld;
    ld.load(Kh, Vh, 0, N_kv, ldv, tid);
    ld.store(smem, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * kBlockN;
        const uint16_t *Ks = smem + (t & 1) * Smem<D>::STAGE;
        const uint16_t *Vs = Ks + Smem<D>::K_TILE;
        const bool more = t + 1 < ntiles;
        if (more) ld.load(Kh, Vh, j0 + kBlockN, N_kv, ldv, tid);

        // S^T = K Q^T for two 32-key blocks.  s[mb][i] is the score of key
        // j0 + mb*32 + (i/4)*8 + g*4 + i%4 against query ql.
        f32x16_t s[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
            for (int kc = 0; kc < D / 16; ++kc) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
                    Ks + (mb * 32 + ql) * Smem<D>::K_LD + kc * 16 + g * 8);
                s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kc], s[mb], 0, 0, 0);
            }
        }

        if (j0 + kBlockN > N_kv) {  // ragged last tile: drop keys past the buffer
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j0 + mb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
                    if (key >= N_kv) s[mb][i] = -INFINITY;
                }
        }

        // online softmax: tile max across the lane pair, rescale, exponentiate
        float mx = s[0][0];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx * c_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][i], c_log2, -m_new));
                s[mb][i] = p;
                lsum += p;
            }
        l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

        // O^T += V^T P^T over four 16-key slices.  MFMA k index g*8 + j of
        // slice kc2 is key kc2*16 + (j/4)*8 + g*4 + j%4 on both operands.
#pragma unroll
        for (int kc2 = 0; kc2 < kBlockN / 16; ++kc2) {
            const int mb = kc2 >> 1, half = kc2 & 1;
            bf16x8_t pb;
#pragma unroll
            for (int j = 0; j < 8; ++j) pb[j] = (__bf16)s[mb][half * 8 + j];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const uint16_t *vrow = Vs + (db * 32 + ql) * Smem<D>::V_LD + kc2 * 16 + g * 4;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 8);
                const bf16x8_t a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
            }
        }

        if (more) ld.store(smem + ((t + 1) & 1) * Smem<D>::STAGE, tid);
        __syncthreads();
    }

    // normalise and store: oacc[db][i] is channel db*32 + (i/4)*8 + g*4 + i%4
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (q_valid) {
        uint16_t *orow = O + ((int64_t)bh * n_q + q_row) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                __bf16 vals[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) vals[e] = (__bf16)(oacc[db][r * 4 + e] * inv);
                uint2 pk;
                __builtin_memcpy(&pk, vals, 8);
                *reinterpret_cast<uint2 *>(orow + db * 32 + r * 8 + g * 4) = pk;
            }
    }
}

}  // namespace

dfp_status dfp_attn_bf16_launch(void *o, const void *q, const void *k, const void *vt, int BH,
                                int n_q, int N_kv, int d, float scale, hipStream_t stream) {
    const int q_tiles = (n_q + kBlockM - 1) / kBlockM;
    const int64_t blocks = (int64_t)q_tiles * BH;
    if (blocks > 0x7FFFFFFF) return DFP_ERR_UNSUPPORTED;
    const int64_t ldv = dfp_v_ld(N_kv, DFP_BF16);
    const float c_log2 = scale * 1.4426950408889634f;
    if (d == 64)
        hipLaunchKernelGGL(attn_fwd_bf16<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                           static_cast<const uint16_t *>(vt), static_cast<uint16_t *>(o), n_q,
                           N_kv, ldv, c_log2, q_tiles);
    else if (d == 128)
        hipLaunchKernelGGL(attn_fwd_bf16<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                           static_cast<const uint16_t *>(vt), static_cast<uint16_t *>(o), n_q,
                           N_kv, ldv, c_log2, q_tiles);
    else
        return DFP_ERR_UNSUPPORTED;
    return dfp::launch_status();
}
