// Paged decode attention on the gfx950 matrix cores, for 16-bit caches and
// grouped-query attention.
//
// Operation: as decode_partition_kernel (PagedAttention digest,
// irregular6612.github.io, section "Method"): for each sequence and query
// head, softmax(scale * q K^T) V over the sequence's paged context, the G
// query heads of a K/V head sharing its K/V rows.
//
// Why matrix cores.  Per byte of K/V the G heads of a group need about G
// flops.  On the vector ALUs (one lane row per token row, DPP reductions)
// that costs ~31 G instructions per token and lane, which at G >= 4 no
// longer fits under the HBM time.  Here a wavefront takes 16 tokens per
// step and the group's heads, zero-padded to 16, form the other side of two
// 16x16 matrix products:
//
//   S^T[token][head] = K[token][:] . Q[head][:]     v_mfma_f32_16x16x32_{f16,bf16}
//   O^T[d][head]    += V^T[d][token] . P^T[token][head]   v_mfma_f32_16x16x16_{f16,bf16}
//
// Operand layouts (16x16xK products, lane L = 16 * g + c, c = L % 16):
//   A (M x K): lane L holds row c, the K-slice of group g;
//   B (K x N): lane L holds column c, the K-slice of group g;
//   C (M x N): lane L holds rows 4g..4g+3 of column c.
// Which channel goes to which K position is free as long as A and B agree,
// so:
//   * q.k: lane L loads 16 bytes of token c's key row (channels
//     32 ks + 8 g .. +7 for k-step ks) and the same channels of query head c;
//     the result gives lane L the scores of tokens 4g..4g+3 for head c;
//   * p.v: the contraction index is the token.  Lane L loads 16 bytes of
//     each of the rows of tokens 4g..4g+3 (channels E c .. E c + E - 1,
//     E = D / 16); output tile t (of E) takes channel E m + t for its row m.
//     One v_perm per register gathers element t of the four rows into the A
//     operand.  The B operand is this lane's own four probabilities: the
//     score layout above is exactly the P^T layout, so no data moves between
//     lanes.  Lane L ends holding, for head c, channels D/4 g .. D/4 g + D/4-1.
//   * Probabilities enter the product as 16-bit values.  To keep fp32
//     accuracy each p is split into hi = p truncated to 16 bits and
//     lo = (p - hi) truncated, and both products are accumulated (relative
//     weight error below 2^-16; the product of a 16-bit p and a 16-bit v is
//     exact in the fp32 accumulator).
// Softmax runs online per 16-token tile: the tile's maximum per head is
// shared across the four lane groups (two cross-row exchanges), the
// accumulators are rescaled only when some head's maximum grows, and the
// running sums are kept per lane and added at the end.
//
// Work decomposition, grid, LDS staging of block ids, longest-first mapping,
// workspace layout and device-side guards are those of
// decode_partition_kernel: one workgroup per (K/V head, sequence, partition).
#pragma once

#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 8  // wavefronts per workgroup of the matrix-core kernel
#endif


constexpr int kMfmaWaves = PA_MFMA_WAVES;
constexpr int kMfmaThreads = kMfmaWaves * kWave;
constexpr int kMfmaTile = 16;            // tokens per wavefront step
constexpr int kMfmaMergeFloats = 8192;   // LDS floats for the cross-wave merge (32 KB)

// Register budget of the kernel: wavefronts per SIMD it must fit (4, i.e.
// <= 128 VGPRs and 2 resident 8-wavefront workgroups per CU, for D <= 128;
// 2 for D = 256).  The balanced split launches that many workgroups per CU.
constexpr int mfma_waves_per_simd(int D) { return D <= 128 ? 4 : 2; }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  In each group of 16
// lanes, lanes 4r .. 4r + 3 each point at 4 consecutive 16-bit elements, the
// four together a 16-element row segment r (r = 0..3); lane i of the group
// receives column i of the 4 x 16 block, i.e. element i of segments 0..3.
// p must be 8-byte aligned and point into LDS.
__device__ __forceinline__ u32x2 lds_read_tr16_b64(const uint16_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p));
    return __builtin_bit_cast(u32x2, v);
}

// Matrix-core operations per 16-bit element type.
template <class T>
struct MfmaOps;

template <>
struct MfmaOps<F16> {
    __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                                     0, 0, 0);
    }
    // Two probabilities -> packed hi words and packed lo words (round toward zero).
    __device__ static __forceinline__ void split(float p0, float p1, uint32_t& hi, uint32_t& lo) {
        const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);
        const float r0 = p0 - static_cast<float>(h[0]);
        const float r1 = p1 - static_cast<float>(h[1]);
        hi = __builtin_bit_cast(uint32_t, h);
        lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    }
};

template <>
struct MfmaOps<BF16> {
    __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                         c, 0, 0, 0);
    }
    __device__ static __forceinline__ void split(float p0, float p1, uint32_t& hi, uint32_t& lo) {
        const uint32_t u0 = f32_as_u32(p0), u1 = f32_as_u32(p1);
        const float r0 = p0 - u32_as_f32(u0 & 0xFFFF0000u);
        const float r1 = p1 - u32_as_f32(u1 & 0xFFFF0000u);
        hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);  // upper halves: p0 low, p1 high
        lo = __builtin_amdgcn_perm(f32_as_u32(r1), f32_as_u32(r0), 0x07060302u);
    }
};

// NW consecutive 32-bit words (NW in {2, 4, 8}) from global memory.
template <int NW, int NT>
__device__ __forceinline__ void load_words(const void* p, uint32_t (&w)[NW]) {
    if constexpr (NW == 2) {
        u32x2 v;
        if constexpr (NT)
            v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        else
            v = *reinterpret_cast<const u32x2*>(p);
        w[0] = v.x;
        w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const uint4 v = load16<NT>(static_cast<const uint32_t*>(p) + 4 * i);
            w[4 * i + 0] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    }
}

template <int NW>
__device__ __forceinline__ void store_words(void* p, const uint32_t (&w)[NW]) {
#pragma unroll
    for (int i = 0; i < NW; ++i) static_cast<uint32_t*>(p)[i] = w[i];
}

__device__ __forceinline__ u32x4 as_u32x4(const uint4& v) { return u32x4{v.x, v.y, v.z, v.w}; }

// Sequence handled by grid row `row` under longest-first order: the one of
// rank `row` in decreasing context length, ties by index.  Needs
// num_seqs <= kMaxLptSeqs (host check); every thread returns the same value.
//
// pair_rows > 0: the grid rows of the first round of one workgroup per CU
// (rows < pair_rows) take the longest sequences, and the rows of the second
// round (pair_rows <= row < 2 pair_rows), which land in the CUs' second
// slots in dispatch order, take the next ones in increasing length, so a CU
// that holds one of the longest contexts gets one of the shorter ones
// beside it.  Later rows stay longest first.  The map is a permutation of
// the ranks.
template <int THREADS>
__device__ __forceinline__ int longest_first_seq(const int32_t* __restrict__ context_lens, int num_seqs, int row,
                                                 int tid, int pair_rows) {
    if (pair_rows > 0 && row >= pair_rows && row < 2 * pair_rows) {
        const int hi = min(2 * pair_rows, num_seqs);
        row = pair_rows + (hi - 1 - row);
    }
    __shared__ int s_len[kMaxLptSeqs];
    __shared__ int s_pick;
    for (int i = tid; i < num_seqs; i += THREADS) s_len[i] = context_lens[i];
    __syncthreads();
    for (int i = tid; i < num_seqs; i += THREADS) {
        const int c = s_len[i];
        int rank = 0;
        for (int j = 0; j < num_seqs; ++j) {
            const int cj = s_len[j];
            rank += (cj > c) || (cj == c && j < i);
        }
        if (rank == row) s_pick = i;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(s_pick);
}

template <class T, int D, int G, bool APPEND, bool NT, bool BALANCED>
__global__ __launch_bounds__(kMfmaThreads, mfma_waves_per_simd(D)) void decode_mfma_kernel(
    typename T::bits* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_m,
    float* __restrict__ ws_l, const typename T::bits* __restrict__ q, typename T::bits* __restrict__ kc,
    typename T::bits* __restrict__ vc, const typename T::bits* __restrict__ knew,
    const typename T::bits* __restrict__ vnew, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int num_seqs, int num_kv_heads, int log2_bs,
    int max_blocks_per_seq, int max_context_len, int64_t num_blocks, int part_tokens, int max_parts, int mode,
    int num_wgs, int32_t* __restrict__ meta, float qscale) {
    static_assert(sizeof(typename T::bits) == 2, "16-bit caches only");
    static_assert(D == 64 || D == 128 || D == 256, "head_dim");
    static_assert(G >= 1 && G <= 16, "group size");
    constexpr int KS = D / 32;  // q.k k-steps (8 channels per lane each)
    constexpr int E = D / 16;   // channels per lane of a V row = output tiles
    constexpr int DP = D + 4;   // padded LDS row
    constexpr int HC0 = kMfmaMergeFloats / (kMfmaWaves * DP);
    constexpr int HC = HC0 >= G ? G : (HC0 >= 8 ? 8 : (HC0 >= 4 ? 4 : (HC0 >= 2 ? 2 : 1)));  // heads per merge pass
    static_assert(HC >= 1 && G % HC == 0, "merge chunk");
    using Ops = MfmaOps<T>;

    // Per-wavefront K and V tiles (16 token rows each, rows padded by 32
    // bytes); after the token loop the same LDS holds the merge rows s_o.
    constexpr int LDW = D + 16;                      // tile row pitch (16-bit elements)
    constexpr int TILE_ELEMS = 2 * kMfmaTile * LDW;  // K then V
    constexpr int RPI = kWave * 8 / D;               // token rows per 16-byte-per-lane load
    constexpr int NLD = kMfmaTile / RPI;             // loads per lane per tile, each of K and V
    static_assert(kMfmaTile % RPI == 0, "tile rows per load");
    constexpr size_t kTileBytes = sizeof(uint16_t) * TILE_ELEMS * kMfmaWaves;
    constexpr size_t kMergeBytes = sizeof(float) * kMfmaWaves * HC * DP;
    extern __shared__ int s_blk[];  // this partition's block ids (dynamic size)
    __shared__ float s_m[kMfmaWaves][16], s_l[kMfmaWaves][16];
    __shared__ __align__(16) unsigned char s_raw[kTileBytes > kMergeBytes ? kTileBytes : kMergeBytes];
    auto s_o = reinterpret_cast<float (*)[HC][DP]>(s_raw);

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int c = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int num_heads = num_kv_heads * G;

    // One pass over tokens [t_begin, t_end) of K/V head hk of sequence s
    // (context ctx): the G heads' partial softmax state, merged across the
    // wavefronts, goes to `out` (single) or to workspace slot `slot`.
    auto run_segment = [&](int s, int hk, int ctx, int t_begin, int t_end, bool single, int slot) {
    const int64_t sh0 = static_cast<int64_t>(s) * num_heads + static_cast<int64_t>(hk) * G;
    const int bmask = (1 << log2_bs) - 1;
    const int j0 = t_begin >> log2_bs;
    const int nblk = ((t_end - 1) >> log2_bs) - j0 + 1;

    const int32_t* bt = block_tables + static_cast<int64_t>(s) * max_blocks_per_seq;
    for (int i = tid; i < nblk; i += kMfmaThreads) {
        const int b = bt[j0 + i];
        s_blk[i] = (b >= 0 && b < num_blocks) ? b : -1;
    }

    // B operand of q.k: query head c (zero for the padding heads c >= G).
    u32x4 qv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qv[ks] = (c < G) ? as_u32x4(load16(q + (sh0 + c) * D + 32 * ks + 8 * g)) : u32x4{0u, 0u, 0u, 0u};
    __syncthreads();  // s_blk is staged

    const uint32_t blk_stride = static_cast<uint32_t>(num_kv_heads << log2_bs) * D;
    const uint32_t head_off = (static_cast<uint32_t>(hk) << log2_bs) * D;
    const bool newest_here = APPEND && t_end == ctx;
    const int64_t kv_row = (static_cast<int64_t>(s) * num_kv_heads + hk) * D;  // row of knew/vnew

    f32x4 acc[E];
#pragma unroll
    for (int t = 0; t < E; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY;  // running maximum of head c's base-2 scores (same in the 4 lane groups)
    float l = 0.0f;       // running sum of exp2(score - m) over this lane's tokens
    int bad = 0;

    const int ntile = (t_end - t_begin + kMfmaTile - 1) / kMfmaTile;

    // This wavefront's tile buffers.
    uint16_t* const sK = reinterpret_cast<uint16_t*>(s_raw) + wave * TILE_ELEMS;
    uint16_t* const sV = sK + kMfmaTile * LDW;

    // Global loads of tile `it`, coalesced: load i of lane L reads 16 bytes
    // (chunk L % (D / 8)) of token row RPI i + L / (D / 8), for K and for V.
    // Tokens past the partition re-read its last token (always in bounds;
    // masked out of the softmax).  In the newest tile t_end == ctx, rows
    // whose clamped token is ctx - 1 (the newest token and the masked rows
    // past it) come from knew/vnew, never from the not-yet-written cache
    // slot, whose contents may be anything (a masked token still multiplies
    // its V row by p = 0, and 0 * NaN is NaN).
    const int ld_row = lane / (D / 8), ld_ch = lane % (D / 8);
    uint4 kreg[NLD], vreg[NLD];
    auto load_tile = [&](int it) {
        const int tb = t_begin + it * kMfmaTile;
        const bool newest = APPEND && newest_here && it == ntile - 1;  // wave-uniform
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int t = min(tb + RPI * i + ld_row, t_end - 1);
            const int b = s_blk[(t >> log2_bs) - j0];
            bad |= (b < 0);
            const uint64_t e = static_cast<uint64_t>(static_cast<uint32_t>(max(b, 0))) * blk_stride + head_off +
                               static_cast<uint32_t>(t & bmask) * D + 8 * ld_ch;
            const bool nw = newest && t == ctx - 1;
            kreg[i] = load16<NT>(nw ? knew + kv_row + 8 * ld_ch : kc + e);
            vreg[i] = load16<NT>(nw ? vnew + kv_row + 8 * ld_ch : vc + e);
        }
    };
    // Registers -> this wavefront's LDS tile; in append mode the lanes holding
    // the newest token's rows (read from knew/vnew) also store them to the
    // cache.
    auto store_tile = [&](int it) {
        // LDS accesses of one wavefront execute in order; the compiler must
        // not move this tile's stores above the previous tile's reads.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            *reinterpret_cast<uint4*>(sK + (RPI * i + ld_row) * LDW + 8 * ld_ch) = kreg[i];
            *reinterpret_cast<uint4*>(sV + (RPI * i + ld_row) * LDW + 8 * ld_ch) = vreg[i];
        }
        if constexpr (APPEND) {
            if (newest_here && it == ntile - 1) {
                const int t = ctx - 1;
                const int b = s_blk[(t >> log2_bs) - j0];
                const int tb = t_begin + it * kMfmaTile;
                const uint64_t e = static_cast<uint64_t>(static_cast<uint32_t>(max(b, 0))) * blk_stride + head_off +
                                   static_cast<uint32_t>(t & bmask) * D + 8 * ld_ch;
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    if (b >= 0 && tb + RPI * i + ld_row == t) {
                        *reinterpret_cast<uint4*>(kc + e) = kreg[i];
                        *reinterpret_cast<uint4*>(vc + e) = vreg[i];
                    }
                }
            }
        }
        asm volatile("" ::: "memory");
    };

    auto compute_tile = [&](int it) {
        const int tb = t_begin + it * kMfmaTile;
        // Scores S^T: lane (c, g) gets tokens tb + 4 g + j of head c; its K
        // operand is token c's channels 32 ks + 8 g .. +7.
        f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sc = Ops::qk(as_u32x4(*reinterpret_cast<const uint4*>(sK + c * LDW + 32 * ks + 8 * g)), qv[ks], sc);

        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = (tb + 4 * g + j < t_end) ? sc[j] * qscale : -INFINITY;
            mx = fmaxf(mx, x[j]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);  // finite: every tile holds a valid token
        if (__builtin_amdgcn_ballot_w64(m_new > m)) {
            const float alpha = fast_exp2(m - m_new);  // 0 on the first tile (m = -inf)
            l *= alpha;
#pragma unroll
            for (int t = 0; t < E; ++t) acc[t] *= alpha;
        }
        m = m_new;
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = fast_exp2(x[j] - m);
            l += p[j];
        }
        uint32_t ph0, pl0, ph1, pl1;
        Ops::split(p[0], p[1], ph0, pl0);
        Ops::split(p[2], p[3], ph1, pl1);
        const u32x2 bh = u32x2{ph0, ph1}, bl = u32x2{pl0, pl1};

        // O^T += V^T P^T, output tile t = channels 16 t .. 16 t + 15.  The A
        // operand (channel 16 t + c of tokens 4 g .. 4 g + 3) is one
        // transposing LDS read: lanes 4 r + q of group g point at token row
        // 4 g + r, channels 16 t + 4 q .. +3.
        const uint16_t* vt = sV + (4 * g + (c >> 2)) * LDW + 4 * (c & 3);
#pragma unroll
        for (int t = 0; t < E; ++t) {
            const u32x2 a = lds_read_tr16_b64(vt + 16 * t);
            acc[t] = Ops::pv(a, bh, acc[t]);
            acc[t] = Ops::pv(a, bl, acc[t]);
        }
    };

    // Software pipeline: the next tile's global loads are in flight while
    // the current tile is computed from LDS.
    int it = wave;
    if (it < ntile) {
        load_tile(it);
        while (true) {
            store_tile(it);
            const int nx = it + kMfmaWaves;
            if (nx < ntile) load_tile(nx);
            compute_tile(it);
            if (nx >= ntile) break;
            it = nx;
        }
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    bad = __syncthreads_or(bad);

    // Merge the wavefronts through LDS, HC heads per pass.
    if (g == 0) {
        s_m[wave][c] = m;
        s_l[wave][c] = l;
    }
#pragma unroll
    for (int c0 = 0; c0 < G; c0 += HC) {
        if (c >= c0 && c < c0 + HC) {
#pragma unroll
            for (int t = 0; t < E; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) s_o[wave][c - c0][16 * t + 4 * g + j] = acc[t][j];
        }
        __syncthreads();
        for (int idx = tid; idx < HC * D; idx += kMfmaThreads) {
            const int hl = idx / D, d = idx % D, h = c0 + hl;
            float M = s_m[0][h];
#pragma unroll
            for (int w = 1; w < kMfmaWaves; ++w) M = fmaxf(M, s_m[w][h]);
            float L = 0.0f, O = 0.0f;
#pragma unroll
            for (int w = 0; w < kMfmaWaves; ++w) {
                const float f = (s_m[w][h] == -INFINITY) ? 0.0f : fast_exp2(s_m[w][h] - M);
                L = fmaf(f, s_l[w][h], L);
                O = fmaf(f, s_o[w][hl][d], O);
            }
            if (bad) O = __builtin_nanf("");
            const int64_t sh = sh0 + h;
            if (single) {
                out[sh * D + d] = narrow<T>(O / L);
            } else {
                ws_o[(sh * max_parts + slot) * D + d] = O;
                if (d == 0) {
                    ws_m[sh * max_parts + slot] = M;
                    ws_l[sh * max_parts + slot] = L;
                }
            }
        }
        if (c0 + HC < G) __syncthreads();  // s_o is reused by the next pass
    }
    };

    // Classic plans: one workgroup per (K/V head, sequence row, partition).
    // Balanced split: every (sequence s, K/V head) pair with a valid
    // context of ctx_s tokens is cut into n_s = ceil(ctx_s / C) pieces of
    // ceil(ctx_s / n_s) <= C tokens (the last one shorter, never empty),
    // C = max(part_tokens, ceil(total / (num_wgs - pairs / 2))), total the
    // batch's tokens over all K/V heads: with ceil's half piece of slack per
    // pair, the pieces about fill the num_wgs resident workgroups.  The grid
    // has num_wgs + pairs workgroups (an upper bound); workgroup w takes the
    // w-th piece in (sequence, K/V head, piece) order, found from prefix sums
    // of Hk n_s.  A pair cut into one piece writes the output; otherwise
    // piece k is partial slot k and the merge kernel combines n_s of them.
    __shared__ int s_pre[kMaxLptSeqs + 1];
    int s, hk, ctx, t_begin, t_end, slot;
    bool single;
    if constexpr (!BALANCED) {
        hk = blockIdx.x;
        const int srow = blockIdx.y, part = blockIdx.z;
        s = mode == kPlanLongestFirst ? longest_first_seq<kMfmaThreads>(context_lens, num_seqs, srow, tid, num_wgs)
                                      : srow;
        ctx = __builtin_amdgcn_readfirstlane(context_lens[s]);
        if (ctx <= 0 || ctx > max_context_len) {
            if (part == 0) {
                const int64_t sh0 = static_cast<int64_t>(s) * num_heads + static_cast<int64_t>(hk) * G;
                const float v = (ctx == 0) ? 0.0f : __builtin_nanf("");
                for (int d = tid; d < G * D; d += kMfmaThreads) out[sh0 * D + d] = narrow<T>(v);
            }
            return;
        }
        t_begin = part * part_tokens;
        if (t_begin >= ctx) return;
        t_end = min(ctx, t_begin + part_tokens);
        single = ctx <= part_tokens;
        slot = part;
    } else {
        // Wave 0 reads the S <= kMaxLptSeqs context lengths (PER consecutive
        // sequences per lane), finds the piece length C from their total,
        // and writes the inclusive prefix sums of the pieces per K/V head to
        // s_pre[1..S] with a wavefront scan; one barrier publishes them.
        if (tid < kWave) {
            constexpr int PER = kMaxLptSeqs / kWave;
            int nv[PER];
            int tot = 0;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int i = tid * PER + k;
                const int n = i < num_seqs ? context_lens[i] : 0;
                nv[k] = (n > 0 && n <= max_context_len) ? n : 0;
                tot += nv[k];
            }
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
            const int64_t total = static_cast<int64_t>(num_kv_heads) * tot;
            const int pairs = num_seqs * num_kv_heads;
            const int64_t slots = max(1, num_wgs - pairs / 2);
            const int C = static_cast<int>(max(static_cast<int64_t>(part_tokens), (total + slots - 1) / slots));
            int run = 0;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                run += nv[k] > 0 ? (nv[k] + C - 1) / C : 0;  // pieces per K/V head
                nv[k] = run;
            }
            int incl = run;  // inclusive scan of the lane totals
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int v = __shfl_up(incl, off);
                if (tid >= off) incl += v;
            }
            const int excl = incl - run;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int i = tid * PER + k;
                if (i < num_seqs) s_pre[i + 1] = excl + nv[k];
            }
            if (tid == 0) {
                s_pre[0] = 0;
                if (blockIdx.x == 0) meta[0] = C;  // for the merge kernel
            }
        }
        __syncthreads();
        const int w = blockIdx.x;
        if (w >= num_kv_heads * __builtin_amdgcn_readfirstlane(s_pre[num_seqs])) return;
        // The sequence of piece w: the last s with Hk * pre[s] <= w.
        int lo = 0, hi = num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (num_kv_heads * s_pre[mid] <= w) lo = mid;
            else hi = mid - 1;
        }
        s = __builtin_amdgcn_readfirstlane(lo);
        const int pre_s = __builtin_amdgcn_readfirstlane(s_pre[s]);
        const int n = __builtin_amdgcn_readfirstlane(s_pre[s + 1]) - pre_s;  // > 0
        const int r = w - num_kv_heads * pre_s;
        hk = r / n;
        slot = r % n;
        ctx = __builtin_amdgcn_readfirstlane(context_lens[s]);
        const int len = (ctx + n - 1) / n;
        t_begin = slot * len;
        t_end = min(ctx, t_begin + len);
        single = n == 1;
    }
    run_segment(s, hk, ctx, t_begin, t_end, single, slot);
}

}  // namespace pa
