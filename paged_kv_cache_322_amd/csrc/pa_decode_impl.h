// Paged decode attention for gfx950: kernel templates, instantiated per
// element type by pa_decode_{f32,f16,bf16}.hip.
//
// Operation (PagedAttention digest, irregular6612.github.io, section
// "Method"): for each sequence s and query head h, attention of the single
// query q[s,h,:] over the sequence's context, whose K/V rows live in
// fixed-size physical blocks found through the sequence's block table.  With
// grouped-query attention, G consecutive query heads share one K/V head
// (G = num_heads / num_kv_heads; G = 1 is multi-head attention).
//
// Work decomposition.  The context of every (sequence, K/V head) is cut into
// KV partitions of P tokens; one workgroup of kWgWaves wavefronts handles one
// (K/V head, sequence, partition) for all G query heads of that K/V head, so
// every K/V byte is loaded once.  Decode attention is a matrix-vector product
// per query head: about G flops per byte.  This vector-ALU kernel serves
// multi-head attention (G = 1), fp32 caches and head sizes below 64; with
// 16-bit caches and G >= 2 the per-token ALU work (which grows with G) no
// longer hides under the HBM time and decode_mfma_kernel (pa_decode_mfma.h)
// runs instead.  Measured with 16-bit multi-head attention, the two kernels
// tie on long contexts and this one is ~15% faster on short ones (a tile
// pipeline of two steps per wavefront, which the matrix-core kernel cannot
// afford in registers).  Inside a workgroup:
//
//   * the partition's physical block ids are staged in LDS once;
//   * a wavefront processes U tokens per step.  A token's row of D elements
//     is spread over LPR = D / (16 / elem) lanes, each lane loading 16 bytes,
//     so one wave-wide load instruction covers 64 / LPR whole token rows and
//     every lane issues NL loads of K and NL loads of V per step.  The loads
//     of a wavefront's next step are issued before the current step is
//     computed (software pipelining);
//   * q.k partial dots are summed across a row's lanes with DPP permutes.
//     Each row of lanes keeps, per query head, its own running maximum,
//     running sum and fp32 accumulators for its slice of D (online softmax,
//     exponentials taken base 2 with log2(e) folded into the query), so the
//     loop needs no exchange between rows; rows are merged once at the end;
//   * wavefronts interleave steps, then merge their (max, sum, accumulators)
//     through LDS, one query head at a time;
//   * the workgroups of one sequence's K/V heads run together (adjacent
//     grid ids) and read the same blocks (head hk's rows of a block are one
//     contiguous run beside head hk + 1's), so each starts its walk at a
//     different step (head hk at step hk * niter / Hk, wrapping around):
//     at any moment they read different blocks.  (The softmax is
//     order-independent; only fp32 rounding depends on the order.)
//
// Grid order: the hardware dispatches workgroups in linear-id order, so the
// partition index is the slowest grid dimension, and for mid-sized batches
// grid row r takes the sequence of rank r in decreasing context length
// (longest first).  A sequence that fits one partition has its output
// written directly; for longer ones each partition writes its unnormalised
// accumulator, maximum and sum to the workspace and decode_merge_kernel
// combines them.
#pragma once

#include <math.h>

#include "pa_decode_mfma.h"
#include "pa_decode_siblings.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

#ifndef PA_WG_WAVES
#define PA_WG_WAVES 8  // wavefronts per workgroup
#endif
#ifndef PA_GQA_PREFETCH
#define PA_GQA_PREFETCH 1  // software-pipeline the loads also when a K/V head serves 4+ query heads
#endif
#ifndef PA_GQA_STEP
#define PA_GQA_STEP 8  // tokens per step when a K/V head serves 4+ query heads
#endif

constexpr int kWgWaves = PA_WG_WAVES;  // wavefronts per workgroup
constexpr int kThreads = kWgWaves * kWave;
static_assert(kMaxLptSeqs <= kThreads || kWgWaves < 8, "one thread ranks one sequence");
constexpr int kMergeMaxParts = 256;  // partition weights cached in LDS by the merge kernel
constexpr int kMergePre = 8;         // partitions whose accumulators the merge kernel loads up front

template <class T, int D, int G>
struct DecodeShape {
    static constexpr int VEC = kVec<T>;
    static constexpr int LPR = D / VEC;      // lanes per token row
    static constexpr int TPL = kWave / LPR;  // token rows per wave-wide load
    // Tokens per step: 16, or 8 when a K/V head serves 4+ query heads (the
    // per-head state then needs the registers).
    static constexpr int STEP_TOKENS = G <= 2 ? 16 : PA_GQA_STEP;
    static constexpr bool PREFETCH = G <= 2 || PA_GQA_PREFETCH;
    static constexpr int NL0 = STEP_TOKENS / TPL;
    static constexpr int NL = NL0 < 1 ? 1 : (NL0 > 8 ? 8 : NL0);  // loads of K (and of V) per lane per step
    static constexpr int U = NL * TPL;                              // tokens per wavefront step
    static_assert(LPR >= 1 && LPR <= kWave && (kWave % LPR) == 0, "unsupported head_dim");
};

// 16-byte non-temporal store of an appended row.  These rows are scattered
// over the pool and written while the kernel streams the cache: on 256
// sequences x 40 heads ordinary stores added 20 us to the call, these add 10.
__device__ __forceinline__ void store16_nt(void* p, const uint4& v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// APPEND: the newest token of every sequence (position ctx - 1) arrives in
// knew/vnew [S, Hk, D]; the workgroup whose partition holds it reads that
// token's rows from there and stores them into the caches.
// NT: K/V loads are non-temporal (streamed once; measured ~10% faster when no
// block is shared).  Without NT they are ordinary cached loads, so sequences
// that share blocks (forked samples, common prefixes) hit in L2 when their
// workgroups run close together.
template <class T, int D, int G, bool APPEND, bool NT>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(
    typename T::bits* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_m,
    float* __restrict__ ws_l, const typename T::bits* __restrict__ q, typename T::bits* __restrict__ kc,
    typename T::bits* __restrict__ vc, const typename T::bits* __restrict__ knew,
    const typename T::bits* __restrict__ vnew, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int num_seqs, int num_kv_heads, int log2_bs,
    int max_blocks_per_seq, int max_context_len, int64_t num_blocks, int part_tokens, int max_parts,
    int longest_first, float qscale) {
    using Sh = DecodeShape<T, D, G>;
    constexpr int VEC = Sh::VEC, LPR = Sh::LPR, TPL = Sh::TPL, NL = Sh::NL, U = Sh::U;
    using bits = typename T::bits;

    extern __shared__ int s_blk[];  // this partition's block ids (dynamic size)
    __shared__ float s_m[kWgWaves], s_l[kWgWaves];
    __shared__ float s_o[kWgWaves][D];

    const int hk = blockIdx.x, srow = blockIdx.y, part = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    int s = srow;
    if (longest_first) {
        // Grid row r handles the sequence of rank r in decreasing context
        // length (ties by index), so the longest contexts are dispatched
        // first.  num_seqs <= kMaxLptSeqs <= kThreads (host check).
        __shared__ int s_len[kMaxLptSeqs];
        __shared__ int s_pick;
        if (tid < num_seqs) s_len[tid] = context_lens[tid];
        __syncthreads();
        if (tid < num_seqs) {
            const int c = s_len[tid];
            int rank = 0;
            for (int j = 0; j < num_seqs; ++j) {
                const int cj = s_len[j];
                rank += (cj > c) || (cj == c && j < tid);
            }
            if (rank == srow) s_pick = tid;
        }
        __syncthreads();
        s = __builtin_amdgcn_readfirstlane(s_pick);  // uniform: keep s and all it decides in SGPRs
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int row = lane / LPR, col = lane % LPR;
    const int num_heads = num_kv_heads * G;
    const int64_t sh0 = static_cast<int64_t>(s) * num_heads + static_cast<int64_t>(hk) * G;  // first query head
    const int ctx = __builtin_amdgcn_readfirstlane(context_lens[s]);

    if (ctx <= 0 || ctx > max_context_len) {
        // Empty context -> zeros; impossible length -> NaN.  Partition 0 writes.
        if (part == 0) {
            const float v = (ctx == 0) ? 0.0f : __builtin_nanf("");
            for (int d = tid; d < G * D; d += kThreads) out[sh0 * D + d] = narrow<T>(v);
        }
        return;
    }
    const int t_begin = part * part_tokens;
    if (t_begin >= ctx) return;
    const int t_end = min(ctx, t_begin + part_tokens);
    const int bmask = (1 << log2_bs) - 1;
    const int j0 = t_begin >> log2_bs;
    const int nblk = ((t_end - 1) >> log2_bs) - j0 + 1;  // <= staged_blocks (host sizes the LDS)

    // Stage this partition's physical block ids; flag ids outside the pool.
    const int32_t* bt = block_tables + static_cast<int64_t>(s) * max_blocks_per_seq;
    for (int i = tid; i < nblk; i += kThreads) {
        const int b = bt[j0 + i];
        s_blk[i] = (b >= 0 && b < num_blocks) ? b : -1;
    }

    // This lane's slice of each query head, scaled by scale * log2(e).
    float qf[G][VEC];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        widen16<T>(load16(q + (sh0 + j) * D + col * VEC), qf[j]);
#pragma unroll
        for (int v = 0; v < VEC; ++v) qf[j][v] *= qscale;
    }
    __syncthreads();  // s_blk is staged

    // APPEND: in the workgroup whose partition holds the newest token (ctx-1),
    // the step that covers it (always the partition's last step) reads that
    // token's rows from knew/vnew instead of the caches, and the lanes
    // holding them store them into the caches.  All other steps are plain.
    const bool newest_here = APPEND && t_end == ctx;
    const int64_t kv_row = (static_cast<int64_t>(s) * num_kv_heads + hk) * D;  // row of knew/vnew

    // Element offsets: block b starts at b * blk_stride (host guarantees
    // Hk * B * D < 2^31); this lane's channels of K/V head hk at lane_off in it.
    const uint32_t blk_stride = static_cast<uint32_t>(num_kv_heads << log2_bs) * D;
    const uint32_t lane_off = (static_cast<uint32_t>(hk) << log2_bs) * D + col * VEC;

    float m[G];       // running max of this row's base-2 scores, per query head
    float l[G];       // running sum of exp2(score - m) over this row's tokens
    float acc[G][VEC];  // running sum of exp2(score - m) * v over this row's tokens
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[j][v] = 0.0f;
    }
    int bad = 0;

    const int niter = (t_end - t_begin + U - 1) / U;
    // Step order of this K/V head: logical step (it + rot) mod niter.
    const int rot = static_cast<int>((static_cast<int64_t>(hk) * niter) / num_kv_heads);
    auto rotated = [&](int it) { const int r = it + rot; return r >= niter ? r - niter : r; };

    auto load_step = [&](int it0, uint4 (&kr)[NL], uint4 (&vr)[NL]) {
        const int it = rotated(it0);
        const int tb = t_begin + it * U;
        const bool newest = APPEND && newest_here && it == niter - 1;  // wave-uniform
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            // Tokens past the partition re-read the last valid token (always
            // in bounds) and are masked out of the softmax.
            const int t = min(tb + i * TPL + row, t_end - 1);
            int b = s_blk[(t >> log2_bs) - j0];
            bad |= (b < 0);
            b = max(b, 0);
            const uint64_t e = static_cast<uint64_t>(static_cast<uint32_t>(b)) * blk_stride + lane_off +
                               static_cast<uint32_t>(t & bmask) * D;
            const bits* kp = kc + e;
            const bits* vp = vc + e;
            if (newest && t == ctx - 1) {
                kp = knew + kv_row + col * VEC;
                vp = vnew + kv_row + col * VEC;
            }
            kr[i] = load16<NT>(kp);
            vr[i] = load16<NT>(vp);
        }
    };

    auto compute_step = [&](int it0, const uint4 (&kr)[NL], const uint4 (&vr)[NL]) {
        const int it = rotated(it0);
        const int tb = t_begin + it * U;
        if constexpr (APPEND) {
            if (newest_here && it == niter - 1) {
                // The one row of lanes whose (unclamped) token is ctx-1 stores it.
                const int t = ctx - 1;
                const int b = s_blk[(t >> log2_bs) - j0];
                const uint64_t e = static_cast<uint64_t>(static_cast<uint32_t>(max(b, 0))) * blk_stride +
                                   lane_off + static_cast<uint32_t>(t & bmask) * D;
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    if (b >= 0 && tb + i * TPL + row == t) {
                        store16_nt(kc + e, kr[i]);
                        store16_nt(vc + e, vr[i]);
                    }
                }
            }
        }
        // Scores of this step's tokens for every query head of the group.
        float sc[G][NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            float kf[VEC];
            widen16<T>(kr[i], kf);
            const bool valid = tb + i * TPL + row < t_end;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float d = 0.0f;
#pragma unroll
                for (int v = 0; v < VEC; ++v) d = fmaf(qf[j][v], kf[v], d);
                d = group_reduce<1, LPR>(d, OpAdd{});
                sc[j][i] = valid ? d : -INFINITY;
            }
        }
        float p[G][NL];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = sc[j][0];
#pragma unroll
            for (int i = 1; i < NL; ++i) mx = fmaxf(mx, sc[j][i]);
            const float m_new = fmaxf(m[j], mx);
            // A row whose tokens so far are all masked keeps m = -inf; use 0
            // as its reference so no inf - inf appears (its weights stay 0).
            const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m[j] - m_ref);
            l[j] *= alpha;
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[j][v] *= alpha;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                p[j][i] = fast_exp2(sc[j][i] - m_ref);
                l[j] += p[j][i];
            }
            m[j] = m_new;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            float vf[VEC];
            widen16<T>(vr[i], vf);
#pragma unroll
            for (int j = 0; j < G; ++j) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] = fmaf(p[j][i], vf[v], acc[j][v]);
            }
        }
    };

    int it = wave;
    if constexpr (!Sh::PREFETCH) {
        for (; it < niter; it += kWgWaves) {
            uint4 ka[NL], va[NL];
            load_step(it, ka, va);
            compute_step(it, ka, va);
        }
    } else if (it < niter) {
        uint4 ka[NL], va[NL], kb[NL], vb[NL];
        load_step(it, ka, va);
        while (true) {
            int nx = it + kWgWaves;
            if (nx < niter) load_step(nx, kb, vb);
            compute_step(it, ka, va);
            if (nx >= niter) break;
            it = nx;
            nx = it + kWgWaves;
            if (nx < niter) load_step(nx, ka, va);
            compute_step(it, kb, vb);
            if (nx >= niter) break;
            it = nx;
        }
    }
    bad = __syncthreads_or(bad);

    const bool single = ctx <= part_tokens;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        // Merge the rows of each wavefront (rows hold disjoint tokens):
        // rescale every row to the wave maximum, then sum.
        const float mw = group_reduce<LPR, kWave>(m[j], OpMax{});
        const float fr = (m[j] == -INFINITY) ? 0.0f : fast_exp2(m[j] - mw);
        const float lw = group_reduce<LPR, kWave>(l[j] * fr, OpAdd{});
        float aw[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) aw[v] = xor_sum_from<LPR>(acc[j][v] * fr);
        if (row == 0) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) s_o[wave][col * VEC + v] = aw[v];
        }
        if (lane == 0) {
            s_m[wave] = mw;
            s_l[wave] = lw;
        }
        __syncthreads();

        // Merge the wavefronts.  Wave 0 always processed token t_begin.
        float M = s_m[0];
#pragma unroll
        for (int w = 1; w < kWgWaves; ++w) M = fmaxf(M, s_m[w]);
        float f[kWgWaves];
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWgWaves; ++w) {
            f[w] = (s_m[w] == -INFINITY) ? 0.0f : fast_exp2(s_m[w] - M);
            L = fmaf(f[w], s_l[w], L);
        }
        const int64_t sh = sh0 + j;
        for (int d = tid; d < D; d += kThreads) {
            float O = 0.0f;
#pragma unroll
            for (int w = 0; w < kWgWaves; ++w) O = fmaf(f[w], s_o[w][d], O);
            if (bad) O = __builtin_nanf("");
            if (single) {
                out[sh * D + d] = narrow<T>(O / L);
            } else {
                ws_o[(sh * max_parts + part) * D + d] = O;
            }
        }
        if (!single && tid == 0) {
            ws_m[sh * max_parts + part] = M;
            ws_l[sh * max_parts + part] = L;
        }
        if (G > 1) __syncthreads();  // s_o / s_m / s_l are reused by the next head
    }
}

// Merge the partitions of every (sequence, query head) whose context spans
// more than one partition: with M the largest partition maximum, each
// partition's sum and accumulator are rescaled by exp2(m_p - M) and added.
// Lane p reads partition p's statistics, so they arrive in one round trip.
template <class T, int D>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(
    typename T::bits* __restrict__ out, const float* __restrict__ ws_o, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const int32_t* __restrict__ context_lens, int num_heads, int max_context_len,
    int part_tokens, int max_parts, int num_kv_heads, const int32_t* __restrict__ meta) {
    __shared__ float s_w[kMergeMaxParts];
    const int h = blockIdx.x, s = blockIdx.y;
    const int ctx = context_lens[s];
    const int64_t sh = static_cast<int64_t>(s) * num_heads + h;
    const int lane = threadIdx.x;
    int np;
    if (part_tokens == 0) {
        // Sibling groups split over max_parts workgroups each: every
        // (sequence, head) has max_parts partials (empty ones weigh 0); the
        // sibling kernel skipped empty and impossible contexts.
        if (ctx <= 0 || ctx > max_context_len) {
            const float v = (ctx == 0) ? 0.0f : __builtin_nanf("");
            for (int d = lane; d < D; d += kWave) out[sh * D + d] = narrow<T>(v);
            return;
        }
        np = max_parts;
    } else if (meta) {
        // Balanced split: the decode kernel skipped empty and invalid
        // contexts, and wrote whole (sequence, K/V head) runs itself.
        if (ctx <= 0 || ctx > max_context_len) {
            const float v = (ctx == 0) ? 0.0f : __builtin_nanf("");
            for (int d = lane; d < D; d += kWave) out[sh * D + d] = narrow<T>(v);
            return;
        }
        const int C = meta[0];  // longest piece of the balanced split
        np = (ctx + C - 1) / C;
        if (np == 1) return;
    } else {
        if (ctx <= part_tokens || ctx > max_context_len) return;  // written by the partition kernel
        np = (ctx + part_tokens - 1) / part_tokens;
    }
    const float* wm = ws_m + sh * max_parts;
    const float* wl = ws_l + sh * max_parts;
    const float* wo = ws_o + sh * max_parts * D;
    // The accumulators of the first kMergePre partitions are loaded before
    // the statistics are reduced, so they arrive in the same memory round
    // trip as the maxima and sums (a split context usually has a few pieces).
    constexpr int DPL = (D + kWave - 1) / kWave;  // channels per lane
    float o_pre[kMergePre][DPL];
#pragma unroll
    for (int p = 0; p < kMergePre; ++p)
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const int d = lane + i * kWave;
            o_pre[p][i] = (p < np && d < D) ? wo[p * D + d] : 0.0f;
        }
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, wm[p]);
    M = group_reduce<1, kWave>(M, OpMax{});
    float L = 0.0f;
    for (int p = lane; p < np; p += kWave) {
        const float w = fast_exp2(wm[p] - M);
        if (p < kMergeMaxParts) s_w[p] = w;
        L = fmaf(w, wl[p], L);
    }
    L = group_reduce<1, kWave>(L, OpAdd{});
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
        const int d = lane + i * kWave;
        if (d >= D) break;
        float O = 0.0f;
#pragma unroll
        for (int p = 0; p < kMergePre; ++p)
            if (p < np) O = fmaf(s_w[p], o_pre[p][i], O);
        for (int p = kMergePre; p < np; ++p) {
            const float w = p < kMergeMaxParts ? s_w[p] : fast_exp2(wm[p] - M);
            O = fmaf(w, wo[p * D + d], O);
        }
        out[sh * D + d] = narrow<T>(O / L);
    }
}

#ifndef PA_MFMA_MIN_G
#define PA_MFMA_MIN_G 2  // smallest group size served by the matrix-core kernel
#endif

// The matrix-core kernel serves 16-bit caches with D in {64, 128, 256} when
// a K/V head has at least PA_MFMA_MIN_G query heads (measured 2-3x faster
// than the vector kernel at G = 4 and 8).
template <class T, int D, int G>
constexpr bool kUseMfma = sizeof(typename T::bits) == 2 && (D == 64 || D == 128 || D == 256) && G >= PA_MFMA_MIN_G;

// Its static LDS (per-wavefront K/V tiles) is ~44 KB for D = 64, ~77 KB for
// D = 128 and ~143 KB for D = 256; partitions staging more block ids than
// this (tiny blocks with very long partitions) take the vector kernel, so
// that static plus staged ids stay within the CU's 160 KB.
template <int D>
constexpr int kMfmaMaxStaged = D == 256 ? 4096 : 6144;

// Sibling-group decode: 16-bit caches, head_dim 64..256 (the group's members
// times the query heads of a K/V head take the matrix columns; the host
// checks that they fit 16).
template <class T, int D, int G>
constexpr bool kUseSiblings = sizeof(typename T::bits) == 2 && (D == 64 || D == 128 || D == 256);

template <class T, int D, int G, bool APPEND, bool NT>
hipError_t launch_decode_t(const DecodeArgs& a) {
    const int log2_bs = __builtin_ctz(static_cast<unsigned>(a.block_size));
    const float qscale = a.scale * 1.4426950408889634f;  // log2(e)
    using bits = typename T::bits;
    auto* out = static_cast<bits*>(a.out);
    float* ws_o = static_cast<float*>(a.workspace);
    const size_t n_sh = static_cast<size_t>(a.num_seqs) * a.num_heads * a.max_parts;
    float* ws_m = ws_o ? ws_o + n_sh * D : nullptr;
    float* ws_l = ws_o ? ws_m + n_sh : nullptr;
    int32_t* meta = ws_o ? reinterpret_cast<int32_t*>(ws_l + n_sh) : nullptr;
    dim3 grid(a.num_kv_heads, a.num_seqs, a.max_parts);
    const size_t lds = static_cast<size_t>(a.staged_blocks) * sizeof(int);
    if constexpr (kUseSiblings<T, D, G> && !APPEND) {
        if (a.siblings >= 2) {
            // One workgroup per (K/V head, sub-group of siblings), whole
            // contexts.
            const int64_t groups = (a.num_seqs + a.siblings - 1) / a.siblings;
            const int64_t per_group = (a.siblings + a.sibling_sub - 1) / a.sibling_sub;
            const unsigned rows = static_cast<unsigned>(groups * per_group);
            // Split tile lists: partials laid out with max_parts = parts.
            const int parts = a.sibling_parts;
            const size_t n_sp = static_cast<size_t>(a.num_seqs) * a.num_heads * parts;
            float* sp_o = parts > 1 ? static_cast<float*>(a.workspace) : nullptr;
            float* sp_m = parts > 1 ? sp_o + n_sp * D : nullptr;
            float* sp_l = parts > 1 ? sp_m + n_sp : nullptr;
            hipLaunchKernelGGL((decode_siblings_kernel<T, D, NT>), dim3(a.num_kv_heads, rows, parts),
                               dim3(kMfmaThreads), static_cast<size_t>(a.sibling_sub) * a.sibling_ids * sizeof(int),
                               a.stream, out, static_cast<const bits*>(a.query), static_cast<const bits*>(a.k_cache),
                               static_cast<const bits*>(a.v_cache), a.block_tables, a.context_lens, a.num_seqs,
                               a.num_kv_heads, G, a.siblings, a.sibling_sub, a.sibling_ids, log2_bs,
                               a.max_blocks_per_seq, a.max_context_len, a.num_blocks, qscale, parts, sp_o, sp_m,
                               sp_l);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess || parts <= 1) return err;
            hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.num_heads, a.num_seqs), dim3(kWave), 0, a.stream,
                               out, static_cast<const float*>(sp_o), static_cast<const float*>(sp_m),
                               static_cast<const float*>(sp_l), a.context_lens, a.num_heads, a.max_context_len, 0,
                               parts, a.num_kv_heads, static_cast<const int32_t*>(nullptr));
            return hipGetLastError();
        }
    }
    if constexpr (kUseMfma<T, D, G>) {
        if (a.balanced && a.staged_balanced <= kMfmaMaxStaged<D>) {
            const unsigned grid_b = static_cast<unsigned>(a.balanced_wgs + a.num_seqs * a.num_kv_heads);
            hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, APPEND, NT, true>), dim3(grid_b), dim3(kMfmaThreads),
                               static_cast<size_t>(a.staged_balanced) * sizeof(int), a.stream, out, ws_o, ws_m, ws_l,
                               static_cast<const bits*>(a.query), static_cast<bits*>(a.k_cache),
                               static_cast<bits*>(a.v_cache), static_cast<const bits*>(a.key_new),
                               static_cast<const bits*>(a.value_new), a.block_tables, a.context_lens, a.num_seqs,
                               a.num_kv_heads, log2_bs, a.max_blocks_per_seq, a.max_context_len, a.num_blocks,
                               a.part_tokens, a.max_parts, kPlanBalanced, a.balanced_wgs, meta, qscale);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.num_heads, a.num_seqs), dim3(kWave), 0, a.stream,
                               out, ws_o, ws_m, ws_l, a.context_lens, a.num_heads, a.max_context_len, a.part_tokens,
                               a.max_parts, a.num_kv_heads, static_cast<const int32_t*>(meta));
            return hipGetLastError();
        }
        // Otherwise (and for a balanced plan whose runs would stage too many
        // block ids): partitions of part_tokens.
        if (a.staged_blocks <= kMfmaMaxStaged<D>) {
            hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, APPEND, NT, false>), grid, dim3(kMfmaThreads), lds, a.stream,
                               out, ws_o, ws_m, ws_l, static_cast<const bits*>(a.query),
                               static_cast<bits*>(a.k_cache), static_cast<bits*>(a.v_cache),
                               static_cast<const bits*>(a.key_new), static_cast<const bits*>(a.value_new),
                               a.block_tables, a.context_lens, a.num_seqs, a.num_kv_heads, log2_bs,
                               a.max_blocks_per_seq, a.max_context_len, a.num_blocks, a.part_tokens, a.max_parts,
                               a.longest_first ? kPlanLongestFirst : kPlanPartitions,
                               a.longest_first ? a.pair_rows : 0, nullptr, qscale);
        } else {
            hipLaunchKernelGGL((decode_partition_kernel<T, D, G, APPEND, NT>), grid, dim3(kThreads), lds, a.stream,
                               out, ws_o, ws_m, ws_l, static_cast<const bits*>(a.query),
                               static_cast<bits*>(a.k_cache), static_cast<bits*>(a.v_cache),
                               static_cast<const bits*>(a.key_new), static_cast<const bits*>(a.value_new),
                               a.block_tables, a.context_lens, a.num_seqs, a.num_kv_heads, log2_bs,
                               a.max_blocks_per_seq, a.max_context_len, a.num_blocks, a.part_tokens, a.max_parts,
                               a.longest_first ? 1 : 0, qscale);
        }
    } else {
        hipLaunchKernelGGL((decode_partition_kernel<T, D, G, APPEND, NT>), grid, dim3(kThreads), lds, a.stream, out,
                           ws_o, ws_m, ws_l, static_cast<const bits*>(a.query), static_cast<bits*>(a.k_cache),
                           static_cast<bits*>(a.v_cache), static_cast<const bits*>(a.key_new),
                           static_cast<const bits*>(a.value_new), a.block_tables, a.context_lens, a.num_seqs,
                           a.num_kv_heads, log2_bs, a.max_blocks_per_seq, a.max_context_len, a.num_blocks,
                           a.part_tokens, a.max_parts, a.longest_first ? 1 : 0, qscale);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.max_parts <= 1) return err;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.num_heads, a.num_seqs), dim3(kWave), 0, a.stream, out,
                       ws_o, ws_m, ws_l, a.context_lens, a.num_heads, a.max_context_len, a.part_tokens,
                       a.max_parts, a.num_kv_heads, static_cast<const int32_t*>(nullptr));
    return hipGetLastError();
}

template <class T, int D, bool APPEND, bool NT>
hipError_t launch_decode_group(const DecodeArgs& a) {
    switch (a.num_heads / a.num_kv_heads) {
        case 1: return launch_decode_t<T, D, 1, APPEND, NT>(a);
        case 2: return launch_decode_t<T, D, 2, APPEND, NT>(a);
        case 4: return launch_decode_t<T, D, 4, APPEND, NT>(a);
        case 8: return launch_decode_t<T, D, 8, APPEND, NT>(a);
        default: return hipErrorInvalidValue;
    }
}

template <class T, bool APPEND, bool NT>
hipError_t launch_decode_dim(const DecodeArgs& a) {
    switch (a.head_dim) {
        case 8: return launch_decode_group<T, 8, APPEND, NT>(a);
        case 16: return launch_decode_group<T, 16, APPEND, NT>(a);
        case 32: return launch_decode_group<T, 32, APPEND, NT>(a);
        case 64: return launch_decode_group<T, 64, APPEND, NT>(a);
        case 128: return launch_decode_group<T, 128, APPEND, NT>(a);
        case 256: return launch_decode_group<T, 256, APPEND, NT>(a);
        default: return hipErrorInvalidValue;
    }
}

template <class T>
hipError_t launch_decode_type(const DecodeArgs& a) {
    if (a.key_new) return a.cached_loads ? launch_decode_dim<T, true, false>(a) : launch_decode_dim<T, true, true>(a);
    return a.cached_loads ? launch_decode_dim<T, false, false>(a) : launch_decode_dim<T, false, true>(a);
}

}  // namespace pa
