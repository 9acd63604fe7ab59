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
// with an online softmax, so its memory is O(tile) whatever N_kv is, and
// the result equals two-pass softmax up to rounding.
//
// Work layout (one workgroup = NW wavefronts x 32 query rows, over one
// contiguous range of 64-key tiles; NW = 4 for d=64, 8 for d=128):
//   * Each wavefront keeps its 32 queries in registers as the B operand of
//     S^T = K Q^T (32 keys x 32 queries per MFMA block).  Computing S^T
//     leaves every score of one query in one lane pair (l, l^32), so the
//     row max needs one cross-lane swap and the probabilities already sit
//     in the B-operand layout of O^T = V^T P^T: no LDS round trip and no
//     transpose for P.
//   * K and V^T tiles move from HBM straight into LDS with
//     buffer_load_dwordx4 ... lds (no VGPR staging).  V is stored
//     transposed in HBM ([d][token]) so V^T tiles feed the A operand of
//     O^T = V^T P^T directly.  The lanes of the Q.K^T A operand load K rows
//     in a permuted order (key_row) that leaves each lane's probabilities
//     on 8 consecutive keys, so every MFMA operand is one 16-byte LDS read.
//     LDS rows are unpadded; 16-byte slot s of row r is stored at s ^ swz(r),
//     so each 16-lane group of a 16-byte operand read covers all 64 banks
//     once.
//   * Four LDS stages per operand: tile t+3's K and tile t+1's V are in
//     flight while step t computes, and step t's own copies (K(t+4),
//     V(t+2)) are issued between its MFMAs; one barrier per step.  The main
//     loop runs four steps per trip so that every stage address is a
//     compile-time constant, and copies full tiles through one buffer
//     resource per (batch, head) with the tile start as the scalar offset.
//   * Each step is one basic block holding three independent streams:
//     tile t+1's Q.K^T MFMAs, tile t-1's P.V MFMAs and tile t's softmax
//     VALU work, interleaved in a fixed order (alternating accumulators,
//     LDS operands read two MFMAs ahead).
//   * Softmax VALU work per score: one FMA (log2(e) * scale and the
//     reference folded in), one exp2, half a bf16 pack and half a dot2 --
//     the row sum is taken on the bf16-rounded probabilities the P.V
//     product uses.  Q enters the MFMA unscaled: folding the scale into a
//     bf16 copy of Q would add a rounding whose score error grows with
//     the score's size.
//   * The reference max is the first tile's row max and stays fixed while
//     the scores stay below it + 12 (log2 units).  Every probability is
//     bounded by the tile's row-sum share, so a share of at most 2^12
//     proves that; a larger one sends the wavefront down a rare path that
//     raises the reference to the tile max and rescales O and the running
//     sum.  Numerator and denominator share the reference, so the result
//     is exactly the softmax whichever reference is used.
//   * Split-KV for small grids: the key range is cut into `splits` ranges
//     handled by different workgroups; each writes an fp32 partial
//     (unnormalised O, running max, running sum) to the workspace, and the
//     last workgroup of a query tile to finish (integer counter) merges the
//     partials in split order, so the result is bitwise reproducible.
//   * Two key groups (the KS = 2 instantiations, d=64) for grids far too
//     small to fill the GPU: a workgroup of four wavefronts takes 64
//     queries, two query wavefronts per key group, each group streaming one
//     half of the key range through its own four-stage ring; at the end the
//     second group hands its (O, m, l) to the first through LDS.  Half the
//     steps per workgroup, no workspace, no cross-workgroup hand-off.
//   * Workgroups are mapped to XCDs so that each XCD streams a contiguous
//     range of (batch, head) buffers, keeping their K/V in that XCD's L2.
//   * Fresh rows (the NF = 1, 2 instantiations): key tiles of up to two
//     ranges -- the patch's own rows, a DiT's text rows -- are copied from
//     this step's K and channel-major V instead of the buffer, and extra
//     workgroups after the attention ones land those rows in the buffer
//     meanwhile.  No attention workgroup reads the buffer rows being landed,
//     so the landing needs no ordering inside the launch.
#include <cmath>
#include <cstdlib>

#include "dfp_common.h"
#include "dfp_internal.h"

namespace {

using dfp::bf16x8_t;
using dfp::f32x16_t;
using dfp::f32x4_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kMaxTileSum = 4096.0f;   // a tile's row-sum share above this raises the max
constexpr int kMaxSplits = 8;            // key-range splits per query tile, at most
constexpr int kCoherent = 16;            // buffer cache policy sc1: device-coherent access
constexpr int kNumXcd = 8;

struct Params {
    const uint16_t *Q;
    const uint16_t *K;
    const uint16_t *Vt;
    uint16_t *O;
    float *part_o;       // [BH*q_tiles][splits][BLOCK_M][D] unnormalised partial O
    float *part_ml;      // [BH*q_tiles][splits][BLOCK_M][2] running max / sum
    unsigned *counters;  // [BH*q_tiles] arrival counters (zero between calls)
    int64_t ldv;
    int n_q;
    int N_kv;
    float c_log2;
    int q_tiles;
    int splits;
    int tiles_per_split;
    int total_wg;        // attention workgroups; landing workgroups follow them
    // Fresh rows (dfp_patch_attention_fresh), up to two ranges r: key tiles
    // [f_t0[r], f_t1[r]), rows [f_row0[r], f_row0[r] + f_n[r]), are read
    // from Kf[r] / Vtf[r] instead of the buffer, and land_wg workgroups
    // after the attention ones copy them into it.
    const uint16_t *Kf[2];   // [BH][f_n][D]
    const uint16_t *Vtf[2];  // [BH][D][f_n]
    uint16_t *Kw;            // the buffer again, writable (landing)
    uint16_t *Vtw;
    int f_t0[2], f_t1[2], f_row0[2], f_n[2];
    int BH;
    int land_wg;
};

// KS key groups per workgroup: KS = 1 is the normal layout; with KS = 2
// (d=64 only) the wavefronts form two groups of NWQ that take the two halves
// of the workgroup's key range for the same NWQ x 32 queries, each with its
// own LDS ring, and are merged through LDS at the end -- twice the key
// parallelism for grids too small to fill the GPU, without the memory
// round trips of a split across workgroups.
// Fewest steps per key group for which the two-group loop uses unrolled
// four-step trips.
constexpr int kStaticMinSteps = 16;

template <int D, int KS>
struct Cfg {
    static constexpr int NW = D == 64 ? 4 : 8;   // wavefronts per workgroup
    static constexpr int NWQ = NW / KS;          // wavefronts per key group
    static constexpr int WG_PER_CU = (D == 64 && KS == 1) ? 2 : 1;   // resident per CU
    static constexpr int THREADS = NW * dfp::kWave;
    static constexpr int BLOCK_M = NWQ * 32;     // query rows per workgroup
    static constexpr int BN = 64;                // keys per tile
    static constexpr int K_ROW = D * 2;          // bytes per K row in LDS (no padding)
    static constexpr int V_ROW = BN * 2;         // bytes per V^T row in LDS
    static constexpr int K_SLOTS = K_ROW / 16;   // 16-byte slots per row
    static constexpr int V_SLOTS = V_ROW / 16;
    static constexpr int K_TILE = BN * K_ROW;    // bytes per stage
    static constexpr int V_TILE = D * V_ROW;
    static constexpr int K_DMA = K_TILE / 1024;  // 64-lane x 16-byte copies per tile
    static constexpr int V_DMA = V_TILE / 1024;
    static constexpr int DMA_W = (K_DMA + V_DMA) / NWQ;  // copies per wavefront per step
    static constexpr int K_DMA_W = K_DMA / NWQ;          // ... of which K
    static constexpr int STAGES = 4;
    static constexpr int SB = BN / 32;           // 32-key score blocks per tile
    static constexpr int DB = D / 32;            // 32-channel output blocks
    static constexpr int KC = D / 16;            // K=16 slices of the Q.K^T product
    static constexpr int KC2 = BN / 16;          // K=16 slices of the P.V product
    static_assert(KS == 1 || (KS == 2 && D == 64), "two key groups at d=64 only");
    static_assert(K_DMA % NWQ == 0 && V_DMA % NWQ == 0, "every wavefront issues as many copies");
    static_assert(DMA_W == 4 || DMA_W == 8, "the end-of-step wait keeps this step's copies");
};

// LDS swizzle: 16-byte slot s of row r is stored at slot s ^ swz(r).  A
// 16-byte read of one slot by 16 consecutive lanes on 16 consecutive rows
// (the MFMA operand pattern) then touches every one of the 64 banks once:
// with 128-byte rows two rows share a 256-byte bank sweep and swz spreads
// the pairs; with 256-byte rows swz alone must separate 16 rows.
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int r) {
    return ROW_BYTES == 128 ? (r >> 1) & 7 : r & 15;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
    bf16x8_t r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

// XCD-aware logical workgroup index: the hardware deals workgroup i to XCD
// i % 8, so give XCD x the contiguous logical range of its share.
__device__ __forceinline__ int logical_wg(int i, int total) {
    const int x = i % kNumXcd, j = i / kNumXcd;
    const int base = total / kNumXcd, rem = total % kNumXcd;
    return x * base + (x < rem ? x : rem) + j;
}

// Max / sum of x over the lane pair (l, l^32): v_permlane32_swap of x with
// itself yields x of lanes 0-31 in the first result and x of lanes 32-63 in
// the second, in both halves of the wave.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef int int32x4_t __attribute__((ext_vector_type(4)));

// A raw buffer resource (V#) covering `bytes` bytes from `base`; accesses at
// or past the end read as zero instead of faulting, and a zero size makes
// every access read zero without touching memory.  Built from uniform
// values, so it lives in scalar registers.
__device__ __forceinline__ int32x4_t buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    int32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;   // gfx9-family raw buffer: dword data, no swizzle
    return r;
}

// One 64-lane HBM -> LDS copy instruction (buffer_load_dwordx4 ... lds):
// lane l reads the 16 bytes at byte offset `voff` of the buffer and writes
// them to LDS byte address lds + 16 l.  It is issued from inline assembly
// so that the compiler, which cannot tell which LDS stage a copy lands in,
// does not wait for copies in flight before every LDS read; the kernel
// instead waits for them explicitly (vmcnt) right before the barrier that
// publishes a stage.  M0 carries the LDS address; nothing else in this
// kernel uses M0 (checked on the built code object).
__device__ __forceinline__ void lds_dma16(int32x4_t rsrc, uint32_t voff, uint32_t soff,
                                          uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(
                     __builtin_amdgcn_readfirstlane(lds)),
                 "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}

// Wait until every copy this wavefront issued has landed in LDS.
__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most the 4 copies issued last are still in flight (this
// step's own; every earlier copy has landed).
template <int N>
__device__ __forceinline__ void wait_dma_keep() {
    static_assert(N == 4 || N == 8, "copies per wavefront per step");
    if constexpr (N == 4)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// Direct HBM -> LDS copies of one K tile (rows [j0, j0+64)) and one V^T tile
// (columns [j0, j0+64)).  Copy instruction i of a tile writes LDS slots
// [64 i, 64 i + 64): slot z = 64 i + lane is row z / SLOTS, stored slot
// z % SLOTS, which holds 16-byte chunk (z % SLOTS) ^ swz(row) of that row.
// Wavefront w of a key group issues instructions w, w + NWQ, ... of the K tile, then of the
// V^T tile (DMA_W in all).  Every lane's byte offset from the tile start is
// fixed for the kernel; the buffer resource starts at the tile.  K rows
// past N_kv fall outside the resource and read as zero (their scores are
// masked anyway); V^T reads past a row's end land in the next row or read
// as zero, and keys >= N_kv are zeroed in LDS afterwards.
template <int D, int KS>
struct TileDma {
    using C = Cfg<D, KS>;
    uint32_t off[C::DMA_W];   // byte offset of this lane's chunk within a tile
    // A fresh range r stores V^T rows with pitch ldn_r instead of ldv.  At
    // d=64 (registers to spare) each V^T copy keeps its fresh offset per
    // range (offf); at d=128, whose plain kernel already fills the register
    // file, copy e of a fresh tile reads at off[e] + row * dpitch[r] with
    // row = vrow0(e) + lane / 8: one lane term and one scalar per range.
    static constexpr bool kPerCopyFresh = D == 64;
    uint32_t offf[2][C::DMA_W - C::K_DMA_W];
    uint32_t lane_dp[2];      // (lane / 8) * dpitch[r]
    uint32_t dpitch[2];       // (ldn_r - ldv) * 2 bytes, modulo 2^32 (uniform)
    int wave;

    __device__ __forceinline__ void init(int wv, int lane, int64_t ldv, int64_t ldn0,
                                         int64_t ldn1) {
        wave = __builtin_amdgcn_readfirstlane(wv);
#pragma unroll
        for (int e = 0; e < C::DMA_W; ++e) {
            if (e < C::K_DMA_W) {
                const int z = (wave + e * C::NWQ) * 64 + lane;
                const int row = z / C::K_SLOTS, slot = (z % C::K_SLOTS) ^ swz<C::K_ROW>(row);
                off[e] = (uint32_t)(row * C::K_ROW + slot * 16);
            } else {
                const int z = (wave + (e - C::K_DMA_W) * C::NWQ) * 64 + lane;
                const int row = z / C::V_SLOTS, slot = (z % C::V_SLOTS) ^ swz<C::V_ROW>(row);
                off[e] = (uint32_t)(row * ldv * 2 + slot * 16);
                offf[0][e - C::K_DMA_W] = (uint32_t)(row * ldn0 * 2 + slot * 16);
                offf[1][e - C::K_DMA_W] = (uint32_t)(row * ldn1 * 2 + slot * 16);
            }
        }
        static_assert(C::V_SLOTS == 8, "a V^T copy covers 8 channel rows of 64 lanes");
        dpitch[0] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((ldn0 - ldv) * 2));
        dpitch[1] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((ldn1 - ldv) * 2));
        lane_dp[0] = (uint32_t)(lane >> 3) * dpitch[0];
        lane_dp[1] = (uint32_t)(lane >> 3) * dpitch[1];
    }

    // First V^T row of copy e (e >= K_DMA_W) of this wavefront (uniform).
    __device__ __forceinline__ uint32_t vrow0(int e) const {
        return (uint32_t)(wave + (e - C::K_DMA_W) * C::NWQ) * 8u;
    }

    // LDS byte address written by copy e of this wavefront.
    __device__ __forceinline__ uint32_t lds_of(int e, uint32_t k_stage, uint32_t v_stage) const {
        return e < C::K_DMA_W ? k_stage + (uint32_t)(wave + e * C::NWQ) * 1024u
                              : v_stage + (uint32_t)(wave + (e - C::K_DMA_W) * C::NWQ) * 1024u;
    }
};

// Per-step copy job: the buffer resources and LDS stages of the K tile and
// the V^T tile one step's copies fill.  A tile outside the workgroup's key
// range gets an empty resource (its copies read zeros, touch no memory).
struct CopyJob {
    int32x4_t rk, rv;
    uint32_t sk, sv;   // byte offsets added to every lane's address (tile start)
    uint32_t lk, lv;
    int vsel;          // the V^T tile's source: 0 buffer, 1 + r fresh range r
    uint32_t vlane;    // fresh V^T tile, d=128: this lane's row-pitch term (else 0)
    uint32_t vpitch;   // fresh V^T tile, d=128: pitch difference per row (else 0)
};

struct Ctx {
    const uint16_t *Kh;
    const uint16_t *Vh;
    const uint16_t *Kf[2];   // this (batch, head)'s fresh rows, per range
    const uint16_t *Vf[2];
    int64_t ldv;
    int N_kv, t_begin, t_end;
    int key_end;     // keys >= key_end are masked: min(N_kv, t_end * 64)
    int t_stop;      // one past the tile of the group's last step (>= t_end)
    uint32_t goff;   // LDS byte offset of this key group's ring (0 for KS = 1)
    int f_t0[2], f_t1[2], f_n[2];
    float c;   // log2(e) * scale
    int tid, ql, g;
};

// The fresh range (0, 1) key tile t of a launch with NF ranges comes from,
// or -1 for the buffer.
template <int NF>
__device__ __forceinline__ int fresh_range(const Ctx &x, int t) {
    if (NF >= 1 && (unsigned)(t - x.f_t0[0]) < (unsigned)(x.f_t1[0] - x.f_t0[0])) return 0;
    if (NF >= 2 && (unsigned)(t - x.f_t0[1]) < (unsigned)(x.f_t1[1] - x.f_t0[1])) return 1;
    return -1;
}

// Value of range r's field (selects on values: an indexed choice would put
// the arrays in scratch memory).
template <typename T>
__device__ __forceinline__ T of_range(int r, T a0, T a1) {
    return r == 1 ? a1 : a0;
}

template <int D, int KS, int NF>
__device__ __forceinline__ CopyJob copy_job(const Ctx &x, const TileDma<D, KS> &dma, int tk, int tv,
                                            uint32_t lk, uint32_t lv) {
    using C = Cfg<D, KS>;
    const int jk = tk * C::BN, jv = tv * C::BN;
    CopyJob j;
    const int kr = tk < x.t_end ? fresh_range<NF>(x, tk) : -1;
    const int vr = tv < x.t_end ? fresh_range<NF>(x, tv) : -1;
    if (kr >= 0) {
        const int r = jk - of_range(kr, x.f_t0[0], x.f_t0[1]) * C::BN;   // row in the range
        j.rk = buffer_rsrc(of_range(kr, x.Kf[0], x.Kf[1]) + (int64_t)r * D,
                           (uint32_t)(of_range(kr, x.f_n[0], x.f_n[1]) - r) * D * 2);
    } else {
        j.rk = buffer_rsrc(x.Kh + (int64_t)jk * D,
                           tk < x.t_end ? (uint32_t)(x.N_kv - jk) * D * 2 : 0u);
    }
    if (vr >= 0) {
        const int r = jv - of_range(vr, x.f_t0[0], x.f_t0[1]) * C::BN;
        j.rv = buffer_rsrc(of_range(vr, x.Vf[0], x.Vf[1]) + r,
                           (uint32_t)((int64_t)D * of_range(vr, x.f_n[0], x.f_n[1]) - r) * 2);
    } else {
        j.rv = buffer_rsrc(x.Vh + jv,
                           tv < x.t_end ? (uint32_t)((int64_t)D * x.ldv - jv) * 2 : 0u);
    }
    j.sk = 0u;
    j.sv = 0u;
    j.lk = lk;
    j.lv = lv;
    j.vsel = vr + 1;
    j.vlane = vr < 0 ? 0u : of_range(vr, dma.lane_dp[0], dma.lane_dp[1]);
    j.vpitch = vr < 0 ? 0u : of_range(vr, dma.dpitch[0], dma.dpitch[1]);
    return j;
}

template <int D, int KS>
__device__ __forceinline__ void issue_copy(const TileDma<D, KS> &dma, const CopyJob &j, int e) {
    using C = Cfg<D, KS>;
    // select values, not arrays: a selected array address would force the
    // offsets into scratch memory
    uint32_t voff = dma.off[e];
    if (e >= C::K_DMA_W) {
        if constexpr (TileDma<D, KS>::kPerCopyFresh) {
            const int i = e >= C::K_DMA_W ? e - C::K_DMA_W : 0;
            const uint32_t f0 = dma.offf[0][i], f1 = dma.offf[1][i];
            voff = j.vsel == 0 ? voff : (j.vsel == 1 ? f0 : f1);
        } else {
            voff += j.vlane + dma.vrow0(e) * j.vpitch;   // 0 for buffer tiles
        }
    }
    lds_dma16(e < C::K_DMA_W ? j.rk : j.rv, voff, e < C::K_DMA_W ? j.sk : j.sv,
              dma.lds_of(e, j.lk, j.lv));
}

// Zero V^T columns of keys >= N_kv in a landed tile: the ragged last tile
// (its columns past N_kv are buffer padding, which may hold anything), or a
// whole tile past the range (N_kv <= j0).
template <int D, int KS>
__device__ __forceinline__ void zero_tail_v(char *Vs, int j0, int N_kv, int tid) {
    using C = Cfg<D, KS>;
    const int first = N_kv - j0;   // first masked key within the tile (<= 63)
    for (int e = tid; e < D * C::BN; e += C::NWQ * dfp::kWave) {   // tid: within the key group
        const int row = e / C::BN, kk = e % C::BN;
        if (kk >= first) {
            const int slot = (kk / 8) ^ swz<C::V_ROW>(row);
            *reinterpret_cast<uint16_t *>(Vs + row * C::V_ROW + slot * 16 + (kk % 8) * 2) = 0;
        }
    }
}

// Key order inside a 32-key score block.  The MFMA leaves accumulator
// element i of lane (ql, g) in block row (i/4)*8 + g*4 + i%4; the A-operand
// lane for block row r loads K row key_row(r), which swaps bits 2 and 3 of
// r.  Element i then holds key (i/8)*16 + g*8 + ((i/4)%2)*4 + i%4, so each
// half (i < 8, i >= 8) of a lane's scores covers 8 consecutive keys: the
// matching V^T operand of P.V is one 16-byte LDS read.
__device__ __forceinline__ int key_row(int r) {
    return (r & ~12) | ((r >> 1) & 4) | ((r << 1) & 8);
}
__device__ __forceinline__ int score_key(int i, int g) {
    return (i >> 3) * 16 + g * 8 + ((i >> 2) & 1) * 4 + (i & 3);
}

// Per-lane LDS byte offsets of the MFMA operands inside a stage: K slice kc
// of key row key_row(ql) (+ sb*32 rows, a constant), V^T slice kc2 of
// channel ql (+ db*32 rows).  The swizzle depends only on the row modulo 32,
// so one offset per slice serves every block.
template <int D, int KS>
struct OperandOffsets {
    using C = Cfg<D, KS>;
    uint32_t k[C::KC];
    uint32_t v[C::KC2];
    // goff: LDS offset of the key group's ring, folded in once
    __device__ __forceinline__ void init(int ql, int g, uint32_t goff) {
        const int kr = key_row(ql);
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc)
            k[kc] = goff + (uint32_t)(kr * C::K_ROW + (((kc * 2 + g) ^ swz<C::K_ROW>(kr)) * 16));
#pragma unroll
        for (int kc2 = 0; kc2 < C::KC2; ++kc2)
            v[kc2] = goff + (uint32_t)(ql * C::V_ROW + (((kc2 * 2 + g) ^ swz<C::V_ROW>(ql)) * 16));
    }
};

template <int D, int KS>
__device__ __forceinline__ bf16x8_t k_operand(const char *Ks, const OperandOffsets<D, KS> &oo, int kc,
                                              int sb) {
    return *reinterpret_cast<const bf16x8_t *>(Ks + oo.k[kc] + sb * 32 * Cfg<D, KS>::K_ROW);
}

template <int D, int KS>
__device__ __forceinline__ bf16x8_t v_operand(const char *Vs, const OperandOffsets<D, KS> &oo, int kc2,
                                              int db) {
    return *reinterpret_cast<const bf16x8_t *>(Vs + oo.v[kc2] + db * 32 * Cfg<D, KS>::V_ROW);
}

// S^T = K Q^T for one tile: s[sb][i] is the score of key
// sb*32 + score_key(i, g) (tile-relative) against query ql.
template <int D, int KS>
__device__ __forceinline__ void qk_tile(f32x16_t (&s)[(Cfg<D, KS>::SB)], const char *Ks,
                                        const bf16x8_t (&qreg)[(Cfg<D, KS>::KC)],
                                        const OperandOffsets<D, KS> &oo) {
    using C = Cfg<D, KS>;
    const f32x16_t zero = {};
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb)
            s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand<D, KS>(Ks, oo, kc, sb), qreg[kc],
                                                            kc == 0 ? zero : s[sb], 0, 0, 0);
}

// O^T += V^T P^T over one tile's 16-key slices.  MFMA k index g*8 + j of
// slice kc2 is key kc2*16 + g*8 + j on both operands.
template <int D, int KS>
__device__ __forceinline__ void pv_tile(f32x16_t (&oacc)[(Cfg<D, KS>::DB)],
                                        const bf16x8_t (&pm)[(Cfg<D, KS>::SB)][2], const char *Vs,
                                        const OperandOffsets<D, KS> &oo) {
    using C = Cfg<D, KS>;
#pragma unroll
    for (int kc2 = 0; kc2 < C::KC2; ++kc2)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                v_operand<D, KS>(Vs, oo, kc2, db), pm[kc2 >> 1][kc2 & 1], oacc[db], 0, 0, 0);
}

// The fixed order of one step's MFMAs: pairs of Q.K^T MFMAs alternate with
// pairs of P.V MFMAs, so consecutive MFMAs never share an accumulator.
template <int D, int KS>
struct Steps {
    using C = Cfg<D, KS>;
    static constexpr int NQ = C::SB * C::KC;             // Q.K^T MFMAs per tile
    static constexpr int NV = C::KC2 * C::DB;            // P.V MFMAs per tile
    static constexpr int N = NQ + NV;
    static_assert(NQ == NV, "steps alternate pairs of Q.K^T and P.V MFMAs");
    static_assert(N >= 4, "a step's first two operands are Q.K^T operands");
    static constexpr bool is_qk(int i) { return (i & 3) < 2; }
    static constexpr int idx(int i) { return (i >> 2) * 2 + (i & 1); }
    static constexpr int CHUNKS = C::SB * 8;             // pairs of probabilities
    static constexpr int CHUNK_EVERY = N / CHUNKS;       // MFMAs per softmax chunk
    // copy e of the step is issued after MFMA copy_at(e), spread evenly
    static constexpr int copy_at(int e) { return e * (N / C::DMA_W) + 1; }
};

template <int D, int KS>
__device__ __forceinline__ bf16x8_t step_operand(int i, const char *Kn, const char *Vp,
                                                 const OperandOffsets<D, KS> &oo) {
    using C = Cfg<D, KS>;
    using S = Steps<D, KS>;
    if (S::is_qk(i)) {
        const int q = S::idx(i);
        return k_operand<D, KS>(Kn, oo, q / C::SB, q % C::SB);
    }
    const int v = S::idx(i);
    return v_operand<D, KS>(Vp, oo, v / C::DB, v % C::DB);
}

// One step's basic block: s_next = K(t+1) Q^T (from Kn), O^T += V(t-1)^T
// P(t-1)^T (from Vp, p_prev), and the softmax of tile t:
// p = 2^(s * c - m) rounded to bf16, with this tile's row-sum share (dot2
// with ones) on the rounded values accumulated in l_tile.  The step's
// DMA_W copies are issued between its MFMAs, so the copy engine is fed
// evenly instead of in a burst.  Operands are read two MFMAs ahead; `carry`
// brings in this step's first two (read by the previous step) and takes
// out the next step's first two, read from Kn_next (K(t+2), already
// published) so they are in flight across the step boundary.
template <int D, int KS>
__device__ __forceinline__ void region(f32x16_t (&s_next)[(Cfg<D, KS>::SB)],
                                       f32x16_t (&oacc)[(Cfg<D, KS>::DB)],
                                       bf16x8_t (&p_cur)[(Cfg<D, KS>::SB)][2], float &l_tile,
                                       const f32x16_t (&s_cur)[(Cfg<D, KS>::SB)],
                                       const bf16x8_t (&p_prev)[(Cfg<D, KS>::SB)][2],
                                       const char *Kn, const char *Vp, const char *Kn_next,
                                       bf16x8_t (&carry)[2], const bf16x8_t (&qreg)[(Cfg<D, KS>::KC)],
                                       float c, float m_run, const OperandOffsets<D, KS> &oo,
                                       const TileDma<D, KS> &dma, const CopyJob &job) {
    using C = Cfg<D, KS>;
    using S = Steps<D, KS>;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    const f32x16_t zero = {};
    bf16x8_t ring[3];
    ring[0] = carry[0];
    ring[1] = carry[1];
#pragma unroll
    for (int i = 0; i < S::N; ++i) {
        ring[(i + 2) % 3] = i + 2 < S::N ? step_operand<D, KS>(i + 2, Kn, Vp, oo)
                                         : step_operand<D, KS>(i + 2 - S::N, Kn_next, Vp, oo);
        const bf16x8_t a = ring[i % 3];
        if (S::is_qk(i)) {
            const int q = S::idx(i), kc = q / C::SB, sb = q % C::SB;
            s_next[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kc],
                                                                  kc == 0 ? zero : s_next[sb],
                                                                  0, 0, 0);
        } else {
            const int v = S::idx(i), kc2 = v / C::DB, db = v % C::DB;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p_prev[kc2 >> 1][kc2 & 1],
                                                                oacc[db], 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < C::DMA_W; ++e)
            if (i == S::copy_at(e)) issue_copy<D, KS>(dma, job, e);
        if (i % S::CHUNK_EVERY == S::CHUNK_EVERY - 1) {
            const int k = i / S::CHUNK_EVERY;      // chunk: two consecutive scores
            const int sb = k / 8, h = (k % 8) / 4, j = (k % 4) * 2;
            bf16x2_t pr;
            pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[sb][h * 8 + j], c, -m_run));
            pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[sb][h * 8 + j + 1], c, -m_run));
            l_tile = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_tile, false);
            p_cur[sb][h][j] = pr[0];
            p_cur[sb][h][j + 1] = pr[1];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    carry[0] = ring[S::N % 3];
    carry[1] = ring[(S::N + 1) % 3];
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
        for (int h = 0; h < 2; ++h) asm volatile("" ::"v"(p_cur[sb][h]));
}

template <int D, int KS>
struct State {
    f32x16_t oacc[(Cfg<D, KS>::DB)];
    float m_run;   // reference max, log2 units (scores * log2(e) * scale)
    float l_run;   // this lane's share of the running sum
};

// Rare path: some probability of tile t exceeded kMaxTileSum (the scores
// outgrew the reference).  Raise the reference to the tile max (never
// lower it), rescale O and l to it and recompute the tile's
// probabilities.
template <int D, int KS>
__device__ __forceinline__ void raise_reference(
    State<D, KS> &st, const f32x16_t (&s_cur)[(Cfg<D, KS>::SB)], bf16x8_t (&p_cur)[(Cfg<D, KS>::SB)][2],
    float &l_tile, float c) {
    using C = Cfg<D, KS>;
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[sb][i]);
    mx = pair_max(mx) * c - st.m_run;   // tile max relative to the reference
    const float delta = mx > 0.f ? mx : 0.f;
    st.m_run += delta;
    const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.oacc[db][i] *= alpha;
    st.l_run *= alpha;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    l_tile = 0.f;
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                bf16x2_t pr;
                pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[sb][h * 8 + j], c, -st.m_run));
                pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[sb][h * 8 + j + 1], c, -st.m_run));
                l_tile = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_tile, false);
                p_cur[sb][h][j] = pr[0];
                p_cur[sb][h][j + 1] = pr[1];
            }
}

// Split-KV merge: the other splits' partials a merging lane loads in one
// batch of coherent loads (all in flight together), bounded by registers:
// 4 splits at d=64, one at d=128.
template <int D>
struct MergeBatch {
    static constexpr int N = D == 64 ? 4 : 1;
};

template <int D, int KS>
struct Smem {
    char k[(Cfg<D, KS>::STAGES)][(Cfg<D, KS>::K_TILE)];
    char v[(Cfg<D, KS>::STAGES)][(Cfg<D, KS>::V_TILE)];
};

// One pipeline step for tile t, r = t - t_begin.  Tile t' of K and of V^T
// lives in stage (t' - t_begin) % 4 (V "tile t_begin - 1", all zeros, in
// stage 3).  On entry K(t+1), K(t+2), V(t-1) and V(t) are published (landed,
// behind a barrier) and K(t+3), V(t+1) are in flight.  The step computes
// (reading K(t+1), V(t-1), and K(t+2) for the next step's first operands)
// while its copies of K(t+4) and V(t+2) go into the stages of K(t) and
// V(t-2), freed by the previous barrier; it then waits until only its own
// copies are in flight and publishes K(t+3), V(t+1) with a barrier.  A tile
// is thus published one step before it is read and copied two steps ahead.
template <int D, int KS, bool RAGGED, int NF>
__device__ __forceinline__ void tile_step(int t, const Ctx &x, State<D, KS> &st, Smem<D, KS> &sm,
                                          const TileDma<D, KS> &dma, const OperandOffsets<D, KS> &oo,
                                          f32x16_t (&s_cur)[(Cfg<D, KS>::SB)],
                                          f32x16_t (&s_next)[(Cfg<D, KS>::SB)],
                                          const bf16x8_t (&p_prev)[(Cfg<D, KS>::SB)][2],
                                          bf16x8_t (&p_cur)[(Cfg<D, KS>::SB)][2],
                                          bf16x8_t (&carry)[2],
                                          const bf16x8_t (&qreg)[(Cfg<D, KS>::KC)]) {
    using C = Cfg<D, KS>;
    constexpr int BN = C::BN;
    const int r = t - x.t_begin;
    const int sk1 = (r + 1) & 3, sk2 = (r + 2) & 3, sv_prev = (r + 3) & 3;
    const int j0 = t * BN;
    if (RAGGED && j0 + BN > x.key_end) {   // ragged last tile: drop keys past the range
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = j0 + sb * 32 + score_key(i, x.g);
                if (key >= x.key_end) s_cur[sb][i] = -INFINITY;
            }
    }
    const CopyJob job = copy_job<D, KS, NF>(x, dma, t + 4, t + 2, lds_addr(sm.k[r & 3]) + x.goff,
                                            lds_addr(sm.v[(r + 2) & 3]) + x.goff);

    float l_tile = 0.f;
    region<D, KS>(s_next, st.oacc, p_cur, l_tile, s_cur, p_prev, sm.k[sk1], sm.v[sv_prev], sm.k[sk2],
              carry, qreg, x.c, st.m_run, oo, dma, job);
    // each probability is at most the tile's row-sum share, so a share
    // within kMaxTileSum proves none outgrew the reference
    if (__any(!(l_tile <= kMaxTileSum))) raise_reference<D, KS>(st, s_cur, p_cur, l_tile, x.c);
    st.l_run += l_tile;

    wait_dma_keep<C::DMA_W>();                 // K(t+3), V(t+1) have landed
    __syncthreads();
    if (RAGGED) {
        // V(t+1) is ragged, or a padding step's tile past the range
        const bool tail = j0 + 2 * BN > x.key_end && t + 1 < x.t_stop;
        if (tail) zero_tail_v<D, KS>(sm.v[(r + 1) & 3] + x.goff, j0 + BN, x.key_end, x.tid);
        if (KS > 1 || tail) __syncthreads();   // one barrier count for both key groups
    }
}

// The same step with the stage ring position R4 = (t - t_begin) % 4 known at
// compile time (LDS operand addresses become immediates) and copies of full
// in-range tiles only: fixed buffer resources over the whole (batch, head)
// (and over its fresh rows) with the tile start as the scalar offset.
template <int D, int KS, int R4, int NF>
__device__ __forceinline__ void tile_step_static(int t, const Ctx &x, State<D, KS> &st, Smem<D, KS> &sm,
                                                 const TileDma<D, KS> &dma,
                                                 const OperandOffsets<D, KS> &oo,
                                                 const int32x4_t &rk_all, const int32x4_t &rv_all,
                                                 const int32x4_t (&rk_f)[2],
                                                 const int32x4_t (&rv_f)[2],
                                                 f32x16_t (&s_cur)[(Cfg<D, KS>::SB)],
                                                 f32x16_t (&s_next)[(Cfg<D, KS>::SB)],
                                                 const bf16x8_t (&p_prev)[(Cfg<D, KS>::SB)][2],
                                                 bf16x8_t (&p_cur)[(Cfg<D, KS>::SB)][2],
                                                 bf16x8_t (&carry)[2],
                                                 const bf16x8_t (&qreg)[(Cfg<D, KS>::KC)]) {
    using C = Cfg<D, KS>;
    constexpr int BN = C::BN;
    constexpr int sk1 = (R4 + 1) & 3, sk2 = (R4 + 2) & 3, sv_prev = (R4 + 3) & 3;
    CopyJob job;
    const int kr = fresh_range<NF>(x, t + 4), vr = fresh_range<NF>(x, t + 2);
    job.rk = kr < 0 ? rk_all : of_range(kr, rk_f[0], rk_f[1]);
    job.rv = vr < 0 ? rv_all : of_range(vr, rv_f[0], rv_f[1]);
    job.sk = (uint32_t)(t + 4 - (kr < 0 ? 0 : of_range(kr, x.f_t0[0], x.f_t0[1]))) *
             (uint32_t)(BN * D * 2);
    job.sv = (uint32_t)(t + 2 - (vr < 0 ? 0 : of_range(vr, x.f_t0[0], x.f_t0[1]))) *
             (uint32_t)(BN * 2);
    job.lk = lds_addr(sm.k[R4]) + x.goff;
    job.lv = lds_addr(sm.v[(R4 + 2) & 3]) + x.goff;
    job.vsel = vr + 1;
    job.vlane = vr < 0 ? 0u : of_range(vr, dma.lane_dp[0], dma.lane_dp[1]);
    job.vpitch = vr < 0 ? 0u : of_range(vr, dma.dpitch[0], dma.dpitch[1]);
    float l_tile = 0.f;
    region<D, KS>(s_next, st.oacc, p_cur, l_tile, s_cur, p_prev, sm.k[sk1], sm.v[sv_prev], sm.k[sk2],
              carry, qreg, x.c, st.m_run, oo, dma, job);
    if (__any(!(l_tile <= kMaxTileSum))) raise_reference<D, KS>(st, s_cur, p_cur, l_tile, x.c);
    st.l_run += l_tile;
    wait_dma_keep<C::DMA_W>();
    __syncthreads();
}

// Copy fresh range r into the buffer.
template <int D, int KS>
__device__ __forceinline__ void land_range(const Params &p, int r) {
    // 32-bit vector indices (the launcher checks that they fit)
    constexpr int U = 4;
    const int f_n = r == 1 ? p.f_n[1] : p.f_n[0];
    const int f_row0 = r == 1 ? p.f_row0[1] : p.f_row0[0];
    const uint32_t stride = (uint32_t)p.land_wg * Cfg<D, KS>::THREADS;
    const uint32_t first = (uint32_t)((int)blockIdx.x - p.total_wg) * Cfg<D, KS>::THREADS + threadIdx.x;
    const uint32_t per_bh = (uint32_t)f_n * D / 8;   // vectors of one (b,h)'s fresh K rows
    const uint32_t per_row = (uint32_t)f_n / 8;      // vectors of one fresh V^T channel row
    const uint32_t nk = per_bh * p.BH, nv = per_row * p.BH * D;
    const uint4 *kf = reinterpret_cast<const uint4 *>(r == 1 ? p.Kf[1] : p.Kf[0]);
    const uint4 *vf = reinterpret_cast<const uint4 *>(r == 1 ? p.Vtf[1] : p.Vtf[0]);
    uint4 *kw = reinterpret_cast<uint4 *>(p.Kw + (int64_t)f_row0 * D);
    uint4 *vw = reinterpret_cast<uint4 *>(p.Vtw + f_row0);
    const uint32_t kw_bh = (uint32_t)p.N_kv * D / 8;   // buffer vectors per (b,h)
    const uint32_t vw_row = (uint32_t)(p.ldv / 8);      // buffer vectors per V^T row
    for (uint32_t v0 = first; v0 < nk; v0 += U * stride) {
        uint4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = v0 + u * stride;
            a[u] = v < nk ? kf[v] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = v0 + u * stride, bh = v / per_bh;
            if (v < nk) kw[(uint64_t)bh * kw_bh + (v - bh * per_bh)] = a[u];
        }
    }
    for (uint32_t v0 = first; v0 < nv; v0 += U * stride) {
        uint4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = v0 + u * stride;
            a[u] = v < nv ? vf[v] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = v0 + u * stride, row = v / per_row;
            if (v < nv) vw[(uint64_t)row * vw_row + (v - row * per_row)] = a[u];
        }
    }
}

// Landing workgroups of a fresh launch: copy every fresh range into the
// buffer (K rows row-major, V^T channel rows), as dfp_kv_scatter would.  No
// attention workgroup of the launch reads those buffer rows.  Four 16-byte
// vectors per thread per pass, all loads before the stores.
template <int D, int KS, int NF>
__device__ __forceinline__ void land_fresh(const Params &p) {
#pragma unroll
    for (int r = 0; r < NF; ++r) land_range<D, KS>(p, r);
}

template <int D, int KS, int NF>
__global__ __launch_bounds__((Cfg<D, KS>::THREADS), (Cfg<D, KS>::WG_PER_CU)) void attn_fwd_bf16(Params p) {
    using C = Cfg<D, KS>;
    constexpr int BN = C::BN;
    __shared__ __attribute__((aligned(16))) Smem<D, KS> sm_all[KS];   // one ring per key group
    __shared__ int s_last;
    Smem<D, KS> &sm = sm_all[0];   // stage addresses; a group's offset comes from x.goff
    if (NF > 0 && (int)blockIdx.x >= p.total_wg) {
        land_fresh<D, KS, NF>(p);
        return;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = tid >> 6;
    // key group (uniform per wavefront, so its ranges stay in scalar registers)
    const int gk = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave_all / C::NWQ);
    const int wave = KS == 1 ? wave_all : wave_all % C::NWQ;   // wavefront within the group
    const int tid_g = tid - gk * C::NWQ * dfp::kWave;           // thread within the group
    const int ql = lane & 31;   // query column of this lane in every MFMA block
    const int g = lane >> 5;    // which half of the K=16 slice this lane feeds

    const int L = logical_wg(blockIdx.x, p.total_wg);
    const int split = L % p.splits;
    const int qtile_id = L / p.splits;          // bh * q_tiles + qt
    const int bh = qtile_id / p.q_tiles;
    const int qt = qtile_id - bh * p.q_tiles;

    const int n_q = p.n_q, N_kv = p.N_kv;
    const uint16_t *Qh = p.Q + (int64_t)bh * n_q * D;
    const int q_row = qt * C::BLOCK_M + wave * 32 + ql;
    const bool q_valid = q_row < n_q;

    Ctx x;
    x.Kh = p.K + (int64_t)bh * N_kv * D;
    x.Vh = p.Vt + (int64_t)bh * D * p.ldv;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const bool on = r < NF;
        x.Kf[r] = on ? p.Kf[r] + (int64_t)bh * p.f_n[r] * D : nullptr;
        x.Vf[r] = on ? p.Vtf[r] + (int64_t)bh * D * p.f_n[r] : nullptr;
        x.f_t0[r] = on ? p.f_t0[r] : 0;
        x.f_t1[r] = on ? p.f_t1[r] : 0;
        x.f_n[r] = on ? p.f_n[r] : 0;
    }
    x.ldv = p.ldv;
    x.N_kv = N_kv;
    const int ntiles = (N_kv + BN - 1) / BN;
    const int wg_t0 = split * p.tiles_per_split;
    const int wg_t1 = min(ntiles, wg_t0 + p.tiles_per_split);
    // Steps per key group, the same for every wavefront: with two groups the
    // first takes ceil(n/2) tiles, the second the rest, padded to as many
    // steps with a masked tile past its range (the range holds >= 2 tiles).
    const int half = KS == 1 ? wg_t1 - wg_t0 : (wg_t1 - wg_t0 + 1) / 2;
    const int R = half;
    x.t_begin = wg_t0 + gk * half;
    x.t_end = gk == 0 ? wg_t0 + half : wg_t1;
    x.key_end = min(N_kv, x.t_end * BN);
    x.t_stop = x.t_begin + R;
    x.goff = KS == 1 ? 0u : (uint32_t)(gk * sizeof(Smem<D, KS>));
    x.c = p.c_log2;
    x.tid = tid_g;
    x.ql = ql;
    x.g = g;

    // Q^T as the B operand: lane (ql, g) holds d = kc*16 + g*8 .. +7 of its
    // query.  Q enters the product unscaled (exact); scale * log2(e) is
    // applied to the fp32 scores.
    bf16x8_t qreg[C::KC];
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
        qreg[kc] = as_bf16x8(q_valid ? *reinterpret_cast<const uint4 *>(
                                           Qh + (int64_t)q_row * D + kc * 16 + g * 8)
                                     : zero4());

    State<D, KS> st;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.oacc[db][i] = 0.f;
    st.l_run = 0.f;

    // Prologue: K(t0..t0+2) and V(t0) landed, V "tile t0-1" (stage 3)
    // zeroed, since the first step's P.V uses zero probabilities against
    // it; K(t0+3) and V(t0+1) in flight (the loop's entry state) while S(t0),
    // the reference max and the first step's first operands are computed.
    TileDma<D, KS> dma;
    dma.init(wave, lane, p.ldv, x.f_n[0], x.f_n[1]);
    OperandOffsets<D, KS> oo;
    oo.init(ql, g, x.goff);
    const int t0 = x.t_begin;
    {
        const uint32_t go = x.goff;
        const CopyJob j0 = copy_job<D, KS, NF>(x, dma, t0, t0, lds_addr(sm.k[0]) + go,
                                               lds_addr(sm.v[0]) + go);
        const CopyJob j1 = copy_job<D, KS, NF>(x, dma, t0 + 1, t0 + 1, lds_addr(sm.k[1]) + go,
                                               lds_addr(sm.v[1]) + go);
        const CopyJob j2 = copy_job<D, KS, NF>(x, dma, t0 + 2, t0 + 2, lds_addr(sm.k[2]) + go,
                                               lds_addr(sm.v[2]) + go);
#pragma unroll
        for (int e = 0; e < C::DMA_W; ++e) issue_copy<D, KS>(dma, j0, e);   // K(t0), V(t0)
#pragma unroll
        for (int e = 0; e < C::K_DMA_W; ++e) issue_copy<D, KS>(dma, j1, e);   // K(t0+1)
#pragma unroll
        for (int e = 0; e < C::K_DMA_W; ++e) issue_copy<D, KS>(dma, j2, e);   // K(t0+2)
    }
    for (int e = tid_g; e < C::V_TILE / 16; e += C::NWQ * dfp::kWave)
        reinterpret_cast<uint4 *>(sm.v[3] + x.goff)[e] = zero4();
    wait_dma_all();
    __syncthreads();
    // K(t0+3), V(t0+1) go out now, before S(t0) (stages K3 and V1 are
    // untouched by the prologue), at d=64; at d=128, whose registers are
    // full, their copy job would stay live across S(t0) and spill inside
    // the main loop, so they go out after it.
    auto copy_k3_v1 = [&]() {
        const CopyJob j3 = copy_job<D, KS, NF>(x, dma, t0 + 3, t0 + 1, lds_addr(sm.k[3]) + x.goff,
                                               lds_addr(sm.v[1]) + x.goff);
#pragma unroll
        for (int e = 0; e < C::DMA_W; ++e) issue_copy<D, KS>(dma, j3, e);
    };
    if constexpr (D == 64) {
        // The compiler does not count the copies: its wait for Q's loads (an
        // in-order counter) must come before this copy, or it would hold the
        // first product until the copy lands.  An empty use here places it.
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) asm volatile("" ::"v"(qreg[kc]));
        copy_k3_v1();
    }
    if (t0 * BN + BN > x.key_end)   // lone ragged tile
        zero_tail_v<D, KS>(sm.v[0] + x.goff, t0 * BN, x.key_end, tid_g);

    f32x16_t sA[C::SB], sB[C::SB];
    bf16x8_t pA[C::SB][2], pB[C::SB][2];
    qk_tile<D, KS>(sA, sm.k[0], qreg, oo);
    // The reference max is the first tile's max over valid keys; it stays
    // fixed until a later tile outgrows it (raise_reference).  A key group's
    // first tile always holds valid keys.
    {
        const int nvalid = x.key_end - t0 * BN;
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = sb * 32 + score_key(i, g);
                if (key >= nvalid) sA[sb][i] = -INFINITY;
                mx = fmaxf(mx, sA[sb][i]);
            }
        st.m_run = pair_max(mx) * p.c_log2;
    }
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) pB[sb][h][j] = (__bf16)0.0f;
    bf16x8_t carry[2] = {step_operand<D, KS>(0, sm.k[1], sm.v[0], oo),
                         step_operand<D, KS>(1, sm.k[1], sm.v[0], oo)};
    if constexpr (D != 64) copy_k3_v1();
    __syncthreads();   // stage 0 of K is free; V(t0)'s zeroed tail is visible

    // Two register sets alternate roles from step to step, so the loop runs
    // two steps per trip and never copies scores or probabilities.  Only
    // the last tile can be ragged: the final one or two steps take the path
    // that masks it.
    if constexpr (KS == 1) {
        int t = t0;
        {
            // full tiles only: every copy of a static trip lands tiles below n_full
            const int n_full = min(x.t_end, N_kv / BN);
            const int32x4_t rk_all = buffer_rsrc(x.Kh, (uint32_t)N_kv * D * 2);
            const int32x4_t rv_all = buffer_rsrc(x.Vh, (uint32_t)((int64_t)D * x.ldv * 2));
            const int32x4_t rk_f[2] = {buffer_rsrc(x.Kf[0], (uint32_t)x.f_n[0] * D * 2),
                                       buffer_rsrc(x.Kf[1], (uint32_t)x.f_n[1] * D * 2)};
            const int32x4_t rv_f[2] = {
                buffer_rsrc(x.Vf[0], (uint32_t)((int64_t)D * x.f_n[0] * 2)),
                buffer_rsrc(x.Vf[1], (uint32_t)((int64_t)D * x.f_n[1] * 2))};
            for (; t + 8 <= n_full; t += 4) {
                tile_step_static<D, KS, 0, NF>(t, x, st, sm, dma, oo, rk_all, rv_all, rk_f, rv_f,
                                               sA, sB, pB, pA, carry, qreg);
                tile_step_static<D, KS, 1, NF>(t + 1, x, st, sm, dma, oo, rk_all, rv_all, rk_f,
                                               rv_f, sB, sA, pA, pB, carry, qreg);
                tile_step_static<D, KS, 2, NF>(t + 2, x, st, sm, dma, oo, rk_all, rv_all, rk_f,
                                               rv_f, sA, sB, pB, pA, carry, qreg);
                tile_step_static<D, KS, 3, NF>(t + 3, x, st, sm, dma, oo, rk_all, rv_all, rk_f,
                                               rv_f, sB, sA, pA, pB, carry, qreg);
            }
        }
        for (; t + 2 < x.t_end; t += 2) {
            tile_step<D, KS, false, NF>(t, x, st, sm, dma, oo, sA, sB, pB, pA, carry, qreg);
            tile_step<D, KS, false, NF>(t + 1, x, st, sm, dma, oo, sB, sA, pA, pB, carry, qreg);
        }
        if (t + 1 < x.t_end) {
            tile_step<D, KS, true, NF>(t, x, st, sm, dma, oo, sA, sB, pB, pA, carry, qreg);
            tile_step<D, KS, true, NF>(t + 1, x, st, sm, dma, oo, sB, sA, pA, pB, carry, qreg);
            pv_tile<D, KS>(st.oacc, pB, sm.v[(t + 1 - t0) & 3], oo);
        } else {
            // a ragged last tile after an unmasked step: V(t) has landed and
            // is first read after this step's barrier
            if (t > t0 && (t + 1) * BN > x.key_end)
                zero_tail_v<D, KS>(sm.v[(t - t0) & 3], t * BN, x.key_end, x.tid);
            tile_step<D, KS, true, NF>(t, x, st, sm, dma, oo, sA, sB, pB, pA, carry, qreg);
            pv_tile<D, KS>(st.oacc, pA, sm.v[(t - t0) & 3], oo);
        }
    } else {
        // Two key groups step in lockstep (the same barriers every step), so
        // every loop bound is the same for all wavefronts: r counts steps
        // from the group's first tile.  The second group's range can be one
        // tile shorter; its last real tile and the masked padding step fall
        // in the masked steps at the end.
        const int h1 = wg_t1 - (wg_t0 + half);   // tiles of the second group (half or half-1)
        const int full = N_kv / BN;
        const int r_full = min(min(wg_t0 + half, full) - wg_t0, min(wg_t1, full) - (wg_t0 + half));
        const int32x4_t rk_all = buffer_rsrc(x.Kh, (uint32_t)N_kv * D * 2);
        const int32x4_t rv_all = buffer_rsrc(x.Vh, (uint32_t)((int64_t)D * x.ldv * 2));
        const int32x4_t rk_f[2] = {buffer_rsrc(x.Kf[0], (uint32_t)x.f_n[0] * D * 2),
                                   buffer_rsrc(x.Kf[1], (uint32_t)x.f_n[1] * D * 2)};
        const int32x4_t rv_f[2] = {buffer_rsrc(x.Vf[0], (uint32_t)((int64_t)D * x.f_n[0] * 2)),
                                   buffer_rsrc(x.Vf[1], (uint32_t)((int64_t)D * x.f_n[1] * 2))};
        int r = 0;
        // Unrolled four-step trips only for long ranges: a short range runs
        // each copy of the step code about once, and after other kernels
        // every copy is an instruction-cache miss (fewer copies, fewer misses).
        const int r_static = r_full >= kStaticMinSteps ? r_full : 0;
        for (; r + 8 <= r_static; r += 4) {
            const int t = x.t_begin + r;
            tile_step_static<D, KS, 0, NF>(t, x, st, sm, dma, oo, rk_all, rv_all, rk_f, rv_f, sA,
                                           sB, pB, pA, carry, qreg);
            tile_step_static<D, KS, 1, NF>(t + 1, x, st, sm, dma, oo, rk_all, rv_all, rk_f, rv_f,
                                           sB, sA, pA, pB, carry, qreg);
            tile_step_static<D, KS, 2, NF>(t + 2, x, st, sm, dma, oo, rk_all, rv_all, rk_f, rv_f,
                                           sA, sB, pB, pA, carry, qreg);
            tile_step_static<D, KS, 3, NF>(t + 3, x, st, sm, dma, oo, rk_all, rv_all, rk_f, rv_f,
                                           sB, sA, pA, pB, carry, qreg);
        }
        for (; r + 2 < h1; r += 2) {
            const int t = x.t_begin + r;
            tile_step<D, KS, false, NF>(t, x, st, sm, dma, oo, sA, sB, pB, pA, carry, qreg);
            tile_step<D, KS, false, NF>(t + 1, x, st, sm, dma, oo, sB, sA, pA, pB, carry, qreg);
        }
        // a ragged tile right after an unmasked step: V(t) has landed and is
        // first read after the next step's barrier
        if (r > 0 && (x.t_begin + r + 1) * BN > x.key_end)
            zero_tail_v<D, KS>(sm.v[r & 3] + x.goff, (x.t_begin + r) * BN, x.key_end, x.tid);
        for (; r + 1 < R; r += 2) {
            const int t = x.t_begin + r;
            tile_step<D, KS, true, NF>(t, x, st, sm, dma, oo, sA, sB, pB, pA, carry, qreg);
            tile_step<D, KS, true, NF>(t + 1, x, st, sm, dma, oo, sB, sA, pA, pB, carry, qreg);
        }
        if (r < R) {
            tile_step<D, KS, true, NF>(x.t_begin + r, x, st, sm, dma, oo, sA, sB, pB, pA, carry,
                                       qreg);
            pv_tile<D, KS>(st.oacc, pA, sm.v[r & 3], oo);
        } else {
            pv_tile<D, KS>(st.oacc, pB, sm.v[(r - 1) & 3], oo);
        }
    }
    wait_dma_all();   // no copy may outlive the workgroup's LDS

    if constexpr (KS == 2) {
        // The second key group hands its (O, m, l) to the first through LDS
        // (its own ring, now idle); the first merges them into its
        // registers, lane for lane in the same accumulator layout.
        constexpr int PER = C::DB * 16 + 2;   // floats per lane
        static_assert(C::NWQ * dfp::kWave * PER * 4 <= (int)sizeof(Smem<D, KS>), "fits a ring");
        float *xch = reinterpret_cast<float *>(&sm_all[1]) + (wave * dfp::kWave + lane) * PER;
        __syncthreads();   // both groups are done with their rings
        if (gk == 1) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) xch[db * 16 + i] = st.oacc[db][i];
            xch[C::DB * 16] = st.m_run;
            xch[C::DB * 16 + 1] = st.l_run;
        }
        __syncthreads();
        if (gk == 1) return;
        const float m1 = xch[C::DB * 16], l1 = xch[C::DB * 16 + 1];
        const float mstar = fmaxf(st.m_run, m1);
        const float a0 = __builtin_amdgcn_exp2f(st.m_run - mstar);
        const float a1 = __builtin_amdgcn_exp2f(m1 - mstar);
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                st.oacc[db][i] = fmaf(a0, st.oacc[db][i], a1 * xch[db * 16 + i]);
        st.l_run = fmaf(a0, st.l_run, a1 * l1);
        st.m_run = mstar;
    }

    const float l_tot = pair_sum(st.l_run);

    // st.oacc[db][i] is channel db*32 + (i/4)*8 + g*4 + i%4 of query ql
    if (p.splits == 1) {
        if (!q_valid) return;
        const float inv = 1.0f / l_tot;
        uint16_t *orow = p.O + ((int64_t)bh * n_q + q_row) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                __bf16 vals[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) vals[e] = (__bf16)(st.oacc[db][rr * 4 + e] * inv);
                uint2 pk;
                __builtin_memcpy(&pk, vals, 8);
                *reinterpret_cast<uint2 *>(orow + db * 32 + rr * 8 + g * 4) = pk;
            }
        return;
    }

    // split-KV: publish this range's partial, the last arrival merges.
    // Partials travel through coherent 16-byte stores and loads (cache
    // policy sc1: they bypass the non-coherent part of the cache hierarchy
    // for device scope), see dfp::publish.  The planner splits one-group
    // launches only.
    if constexpr (KS == 1) {
        // Each wavefront restages its 32 rows through LDS, one 32-channel
        // block at a time, so that a store covers eight rows' 128-byte runs
        // instead of 32 rows' 32-byte pieces; a lane keeps what it stored
        // (own[db][i]: row (lane + 64 i) / 8 of the wavefront, channels
        // db*32 + ((lane + 64 i) % 8) * 4 + 0..3), and a merging lane loads
        // the other splits' partials from the same addresses.
        constexpr int LDW = 36;                      // staged row: 32 floats + 4 pad
        float *wst = reinterpret_cast<float *>(&sm_all[0]) + wave * (32 * LDW);
        float *wts = reinterpret_cast<float *>(&sm_all[0]) + C::NW * 32 * LDW;
        static_assert((C::NW * 32 * LDW + C::BLOCK_M * kMaxSplits) * 4 <= (int)sizeof(Smem<D, KS>),
                      "staging and row weights fit the ring");
        const int row = wave * 32 + ql;
        const int64_t slot = (int64_t)qtile_id * p.splits + split;
        const int64_t base = (int64_t)qtile_id * p.splits;
        __syncthreads();   // every wavefront is done with the ring
        f32x4_t own[C::DB][4];
        {
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                p.part_o + slot * C::BLOCK_M * D, 0, C::BLOCK_M * D * 4, 0x00020000);
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    *reinterpret_cast<f32x4_t *>(wst + ql * LDW + rr * 8 + g * 4) =
                        f32x4_t{st.oacc[db][rr * 4], st.oacc[db][rr * 4 + 1],
                                st.oacc[db][rr * 4 + 2], st.oacc[db][rr * 4 + 3]};
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the block is staged
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = lane + 64 * i;
                    own[db][i] = *reinterpret_cast<const f32x4_t *>(wst + (c >> 3) * LDW +
                                                                     (c & 7) * 4);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before reuse
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = lane + 64 * i;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(int32x4_t, own[db][i]), ro,
                        ((wave * 32 + (c >> 3)) * D + db * 32 + (c & 7) * 4) * 4, 0, kCoherent);
                }
            }
        }
        if (g == 0) {
            float *pml = p.part_ml + (slot * C::BLOCK_M + row) * 2;
            dfp::publish(pml, st.m_run);
            dfp::publish(pml + 1, l_tot);
        }
        dfp::published_wait();
        __syncthreads();
        if (tid == 0) s_last = (dfp::arrive(p.counters + qtile_id) == (unsigned)p.splits - 1);
        __syncthreads();
        if (!s_last) return;

        // merge: O = sum_s w_s O_s with w_s = 2^(m_s - m*) / sum_s' 2^(m_s' - m*) l_s',
        // in split order, every lane over the elements it holds; this split's
        // partial comes from registers, the others' in batches of loads that
        // are in flight together.  The arithmetic does not depend on which
        // split arrives last.
        constexpr int NB = MergeBatch<D>::N;
        f32x4_t acc[C::DB][4];
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[db][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < p.splits; s0 += NB) {
            f32x4_t v[NB][C::DB][4];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int sj = s0 + j;
                if (sj < p.splits && sj != split) {
                    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                        p.part_o + (base + sj) * C::BLOCK_M * D, 0, C::BLOCK_M * D * 4,
                        0x00020000);
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int c = lane + 64 * i;
                            v[j][db][i] = __builtin_bit_cast(
                                f32x4_t,
                                __builtin_amdgcn_raw_buffer_load_b128(
                                    ro, ((wave * 32 + (c >> 3)) * D + db * 32 + (c & 7) * 4) * 4,
                                    0, kCoherent));
                        }
                }
            }
            if (s0 == 0) {   // row weights into LDS while the first batch is in flight
                if (tid < C::BLOCK_M) {
                    float ms[kMaxSplits], ls[kMaxSplits];
#pragma unroll
                    for (int s = 0; s < kMaxSplits; ++s)
                        if (s < p.splits) {
                            const float *ml = p.part_ml + ((base + s) * C::BLOCK_M + tid) * 2;
                            ms[s] = dfp::fetch_published(ml);
                            ls[s] = dfp::fetch_published(ml + 1);
                        }
                    float mstar = -INFINITY;
#pragma unroll
                    for (int s = 0; s < kMaxSplits; ++s)
                        if (s < p.splits) mstar = fmaxf(mstar, ms[s]);
                    float den = 0.f;
#pragma unroll
                    for (int s = 0; s < kMaxSplits; ++s)
                        if (s < p.splits) {
                            ms[s] = __builtin_amdgcn_exp2f(ms[s] - mstar);
                            den = fmaf(ms[s], ls[s], den);
                        }
                    const float inv = 1.0f / den;
#pragma unroll
                    for (int s = 0; s < kMaxSplits; ++s)
                        if (s < p.splits) wts[tid * kMaxSplits + s] = ms[s] * inv;
                }
                __syncthreads();
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int sj = s0 + j;
                if (sj >= p.splits) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float w = wts[(wave * 32 + ((lane + 64 * i) >> 3)) * kMaxSplits + sj];
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const f32x4_t o_s = sj == split ? own[db][i] : v[j][db][i];
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[db][i][e] = fmaf(w, o_s[e], acc[db][i][e]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = lane + 64 * i;
            const int qr = qt * C::BLOCK_M + wave * 32 + (c >> 3);
            if (qr >= n_q) continue;
            uint16_t *orow = p.O + ((int64_t)bh * n_q + qr) * D + (c & 7) * 4;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                __bf16 vals[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) vals[e] = (__bf16)acc[db][i][e];
                uint2 pk;
                __builtin_memcpy(&pk, vals, 8);
                *reinterpret_cast<uint2 *>(orow + db * 32) = pk;
            }
        }
        if (tid == 0) dfp::publish(p.counters + qtile_id, 0u);
    }
}

// ---------------------------------------------------------------- planning
constexpr int kCus = 256;

struct Plan {
    int ks;   // key groups per workgroup (1, or 2 at d=64)
    int block_m, q_tiles, ntiles, splits, tiles_per_split;
};

// Pick the key-range split that minimises an estimate of the makespan,
// from per-step times measured for this kernel on MI355X: a 64-key step of
// one workgroup takes about T_ALONE when the workgroup has its CU to itself
// and T_SHARED when two share it (d=64 keeps two resident per CU, d=128
// one).  Workgroups beyond the resident slots run in later rounds.  Every
// workgroup pays a fixed prologue/epilogue; a split adds the hand-off
// latency and moves each fp32 partial through memory twice (publish, merge).
// At d=64 a grid too small to fill the GPU can instead use two key groups
// per workgroup (64 queries, one workgroup per CU, half the steps, an LDS
// merge): chosen when its estimate beats the best split.
Plan make_plan(int BH, int n_q, int N_kv, int d, bool can_split) {
    Plan pl;
    pl.ks = 1;
    pl.block_m = d == 64 ? Cfg<64, 1>::BLOCK_M : Cfg<128, 1>::BLOCK_M;
    const int bn = 64;
    pl.q_tiles = (n_q + pl.block_m - 1) / pl.block_m;
    pl.ntiles = (N_kv + bn - 1) / bn;
    pl.splits = 1;
    pl.tiles_per_split = pl.ntiles;
    const int per_cu = d == 64 ? Cfg<64, 1>::WG_PER_CU : Cfg<128, 1>::WG_PER_CU;
    const double t_alone = d == 64 ? 0.62e-6 : 1.7e-6;   // s per step, CU to itself
    const double t_shared = 1.09e-6;                     // s per step, two per CU (d=64)
    const double t_fixed = 3e-6;                         // prologue + epilogue
    // publish, arrive and row weights, then one memory round trip per batch
    // of partials the merge loads together (measured: 3 splits ~3.5 us,
    // 8 splits ~6.5 us at d=64)
    const int merge_batch = d == 64 ? MergeBatch<64>::N : MergeBatch<128>::N;
    const double merge_bw = 5e12;                        // partial bytes/s, written and read
    const double base = (double)BH * pl.q_tiles;
    double best = 1e300;
    const char *env = std::getenv("DFP_ATTN_SPLITS");
    const int forced = env ? std::atoi(env) : 0;
    for (int s = 1; s <= (can_split ? kMaxSplits : 1) && s <= pl.ntiles; ++s) {
        const int tps = (pl.ntiles + s - 1) / s;
        const int s_eff = (pl.ntiles + tps - 1) / tps;
        if (s_eff != s) continue;
        const double wgs = base * s;
        double t;
        if (per_cu == 1) {
            t = std::ceil(wgs / kCus) * tps * t_alone;
        } else {
            const double slots = (double)kCus * per_cu;
            const double full = std::floor(wgs / slots), rem = wgs - full * slots;
            t = full * tps * t_shared +
                (rem <= 0 ? 0.0 : tps * (rem <= kCus ? t_alone : t_shared));
        }
        t += t_fixed;
        if (s > 1)
            t += 2e-6 + std::ceil((double)s / merge_batch) * 1.5e-6 +
                 2.0 * wgs * pl.block_m * d * 4.0 / merge_bw;
        if (s == 1 || (forced > 0 ? s == forced : t < best * 0.98)) {
            best = t;
            pl.splits = s;
            pl.tiles_per_split = tps;
        }
        if (forced > 0 && s == forced) break;
    }
    const char *env_ks = std::getenv("DFP_ATTN_KS");
    const int forced_ks = env_ks ? std::atoi(env_ks) : 0;
    if (d == 64 && pl.ntiles >= 2 && forced <= 1 && forced_ks != 1) {
        const int q_tiles2 = (n_q + Cfg<64, 2>::BLOCK_M - 1) / Cfg<64, 2>::BLOCK_M;
        const double wgs2 = (double)BH * q_tiles2;   // one workgroup per CU
        // measured step times of this variant: 0.65 us in unrolled trips,
        // 0.80 us in short loops (run-time stages)
        const int steps2 = (pl.ntiles + 1) / 2;
        const double t_step2 = steps2 >= kStaticMinSteps ? 0.65e-6 : 0.80e-6;
        const double t2 = std::ceil(wgs2 / kCus) * steps2 * t_step2 + t_fixed +
                          0.5e-6;   // LDS merge
        if (forced_ks == 2 || (forced <= 0 && t2 < best * 0.98)) {
            pl.ks = 2;
            pl.block_m = Cfg<64, 2>::BLOCK_M;
            pl.q_tiles = q_tiles2;
            pl.splits = 1;
            pl.tiles_per_split = pl.ntiles;
        }
    }
    return pl;
}

size_t counters_bytes(int BH, int q_tiles) {
    return ((size_t)BH * q_tiles * sizeof(unsigned) + 255) / 256 * 256;
}

size_t need_bytes(int BH, int d, const Plan &pl) {
    if (pl.splits <= 1) return 0;
    const size_t slots = (size_t)BH * pl.q_tiles * pl.splits;
    return counters_bytes(BH, pl.q_tiles) + slots * pl.block_m * d * sizeof(float) +
           slots * pl.block_m * 2 * sizeof(float);
}

}  // namespace

size_t dfp_attn_workspace_bytes(int B, int H, int n_q, int N_kv, int d) {
    if (B <= 0 || H <= 0 || n_q <= 0 || N_kv <= 0 || (d != 64 && d != 128)) return 0;
    const int BH = B * H;
    return need_bytes(BH, d, make_plan(BH, n_q, N_kv, d, true));
}

void dfp_attn_bf16_plan(int BH, int n_q, int N_kv, int d, bool can_split, int *key_groups,
                        int *splits, int64_t *workgroups) {
    const Plan pl = make_plan(BH, n_q, N_kv, d, can_split);
    *key_groups = pl.ks;
    *splits = pl.splits;
    *workgroups = (int64_t)pl.q_tiles * BH * pl.splits;
}

dfp_status dfp_attn_bf16_launch(void *o, const void *q, const void *k, const void *vt, int BH,
                                int n_q, int N_kv, int d, float scale, void *ws, size_t ws_bytes,
                                const dfp_fresh_launch *fresh, hipStream_t stream) {
    // tile copies address one (batch, head)'s K and V^T with 32-bit offsets
    const int64_t ldv = dfp_v_ld(N_kv, DFP_BF16);
    if ((int64_t)N_kv * d * 2 >= (int64_t(1) << 31) || (int64_t)d * ldv * 2 >= (int64_t(1) << 31))
        return DFP_ERR_UNSUPPORTED;
    Plan pl = make_plan(BH, n_q, N_kv, d, true);
    if (pl.splits > 1 && (!ws || ws_bytes < need_bytes(BH, d, pl) ||
                          (reinterpret_cast<uintptr_t>(ws) & 255u) != 0))
        pl = make_plan(BH, n_q, N_kv, d, false);
    const int64_t blocks = (int64_t)pl.q_tiles * BH * pl.splits;
    // landing workgroups take the resident slots the attention grid leaves
    // free in its last round (at least 16, at most 64)
    int land_wg = 0;
    if (fresh && fresh->land) {
        const int64_t slots =
            (int64_t)kCus * (d == 64 && pl.ks == 1 ? Cfg<64, 1>::WG_PER_CU : 1);
        const int64_t free = (slots - blocks % slots) % slots;
        land_wg = (int)(free < 16 ? 16 : (free > 64 ? 64 : free));
    }
    if (blocks + land_wg > 0x7FFFFFFF) return DFP_ERR_UNSUPPORTED;
    // landing indexes 16-byte vectors of the fresh tensors with 32 bits
    if (fresh) {
        if ((int64_t)N_kv * d / 8 >= (int64_t(1) << 31)) return DFP_ERR_UNSUPPORTED;
        for (int r = 0; r < fresh->count; ++r)
            if ((int64_t)BH * fresh->ranges[r].n * d / 8 >= (int64_t(1) << 31))
                return DFP_ERR_UNSUPPORTED;
    }

    Params p{};
    p.Q = static_cast<const uint16_t *>(q);
    p.K = static_cast<const uint16_t *>(k);
    p.Vt = static_cast<const uint16_t *>(vt);
    p.O = static_cast<uint16_t *>(o);
    p.ldv = ldv;
    p.n_q = n_q;
    p.N_kv = N_kv;
    p.c_log2 = scale * 1.4426950408889634f;
    p.q_tiles = pl.q_tiles;
    p.splits = pl.splits;
    p.tiles_per_split = pl.tiles_per_split;
    p.total_wg = (int)blocks;
    p.BH = BH;
    if (fresh) {
        for (int r = 0; r < fresh->count; ++r) {
            const dfp_fresh_rows &fr = fresh->ranges[r];
            p.Kf[r] = static_cast<const uint16_t *>(fr.k);
            p.Vtf[r] = static_cast<const uint16_t *>(fr.v_t);
            p.f_row0[r] = fr.row0;
            p.f_n[r] = fr.n;
            p.f_t0[r] = fr.row0 / 64;
            p.f_t1[r] = (fr.row0 + fr.n) / 64;
        }
        p.Kw = static_cast<uint16_t *>(fresh->k_buf);
        p.Vtw = static_cast<uint16_t *>(fresh->v_buf_t);
        p.land_wg = land_wg;
    }
    if (pl.splits > 1) {
        char *w = static_cast<char *>(ws);
        p.counters = reinterpret_cast<unsigned *>(w);
        w += counters_bytes(BH, pl.q_tiles);
        const size_t slots = (size_t)BH * pl.q_tiles * pl.splits;
        p.part_o = reinterpret_cast<float *>(w);
        w += slots * pl.block_m * d * sizeof(float);
        p.part_ml = reinterpret_cast<float *>(w);
    }
    const dim3 grid((unsigned)(blocks + land_wg));
    const int nf = fresh ? fresh->count : 0;
    if (d == 64 && pl.ks == 2) {
        const dim3 block(Cfg<64, 2>::THREADS);
        if (nf == 0) hipLaunchKernelGGL((attn_fwd_bf16<64, 2, 0>), grid, block, 0, stream, p);
        else if (nf == 1) hipLaunchKernelGGL((attn_fwd_bf16<64, 2, 1>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_fwd_bf16<64, 2, 2>), grid, block, 0, stream, p);
    } else if (d == 64 && nf == 0)
        hipLaunchKernelGGL((attn_fwd_bf16<64, 1, 0>), grid, dim3(Cfg<64, 1>::THREADS), 0, stream, p);
    else if (d == 64 && nf == 1)
        hipLaunchKernelGGL((attn_fwd_bf16<64, 1, 1>), grid, dim3(Cfg<64, 1>::THREADS), 0, stream, p);
    else if (d == 64 && nf == 2)
        hipLaunchKernelGGL((attn_fwd_bf16<64, 1, 2>), grid, dim3(Cfg<64, 1>::THREADS), 0, stream, p);
    else if (d == 128 && nf == 0)
        hipLaunchKernelGGL((attn_fwd_bf16<128, 1, 0>), grid, dim3(Cfg<128, 1>::THREADS), 0, stream,
                           p);
    else if (d == 128 && nf == 1)
        hipLaunchKernelGGL((attn_fwd_bf16<128, 1, 1>), grid, dim3(Cfg<128, 1>::THREADS), 0, stream,
                           p);
    else if (d == 128 && nf == 2)
        hipLaunchKernelGGL((attn_fwd_bf16<128, 1, 2>), grid, dim3(Cfg<128, 1>::THREADS), 0, stream,
                           p);
    else
        return DFP_ERR_UNSUPPORTED;
    return dfp::launch_status();
}
