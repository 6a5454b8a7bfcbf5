// Decode of sibling sequences that share a prefix of physical blocks
// (forked samples of parallel sampling, beam candidates), on the gfx950
// matrix cores.
//
// Operation: as decode_partition_kernel (PagedAttention digest,
// irregular6612.github.io, section "Method"): for each sequence and head,
// softmax(scale * q K^T) V over the sequence's paged context.  Same digest,
// same section, and "vLLM PagedAttention and continuous batching
// architecture" (tech.blogsailing.com), section 2: the samples forked from
// one prompt keep pointing at the prompt's physical blocks (reference
// counted) and copy only a block they write.  Their contexts therefore begin
// with the same physical blocks, and reading those blocks once per sample
// moves the shared prompt through the memory system n times.
//
// Design: one workgroup per (group of n consecutive sequences, K/V head),
// or per (sub-group, K/V head) where the group has more members than the
// matrix columns hold: a group is then cut into consecutive sub-groups of
// `sub` members, each its own workgroup, so a shared block is read once per
// sub-group.  A workgroup's members' block-table rows are staged in LDS and
// compared entry by entry: the leading entries every member holds in common
// (the same physical block) cover the shared prefix, S = min(J * B,
// shortest context) tokens (J the common entries).  The prefix is read
// once: each 16-token K/V tile feeds the 16x16 matrix products of
// decode_mfma_kernel with the members' queries as the columns (where that
// kernel puts the G heads of a K/V head; member m takes columns
// m G .. m G + G - 1, members x G <= 16).  Each member's remaining tokens
// S .. ctx - 1 are then read from its own blocks with only its columns
// unmasked.  The grouping is a hint: nothing is assumed shared that the
// tables do not show (no common entries: every token is read privately,
// the same result), and the arithmetic is decode_mfma_kernel's (fp32
// products and softmax, probabilities split into hi and lo 16-bit parts).
// Each member's softmax state is per column; the 8 wavefronts split the
// tiles of the whole token list and merge through LDS.  A batch with few
// (sub-group, K/V head) pairs can also split each tile list over `parts`
// workgroups (grid z): workgroup z takes tiles [z n / parts, (z + 1) n /
// parts) of the n and writes, per member and query head, its unnormalised
// partial result (accumulator, maximum, sum) to the workspace, which
// decode_merge_kernel combines as it does the partitions of one context.
// The members' K/V values must be finite: a masked column still multiplies
// its zero probabilities with the tile's V rows, so a non-finite value in
// one member's own tokens can reach its siblings' results.
#pragma once

#include <math.h>

#include "pa_decode_mfma.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <class T, int D, bool NT>
__global__ __launch_bounds__(kMfmaThreads, mfma_waves_per_simd(D)) void decode_siblings_kernel(
    typename T::bits* __restrict__ out, const typename T::bits* __restrict__ q,
    const typename T::bits* __restrict__ kc, const typename T::bits* __restrict__ vc,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, int num_seqs,
    int num_kv_heads, int gq, int group, int sub, int ids_per_seq, int log2_bs, int max_blocks_per_seq,
    int max_context_len,
    int64_t num_blocks, float qscale, int parts, float* __restrict__ ws_o, float* __restrict__ ws_m,
    float* __restrict__ ws_l) {
    static_assert(sizeof(typename T::bits) == 2, "16-bit caches only");
    static_assert(D == 64 || D == 128 || D == 256, "head_dim");
    constexpr int KS = D / 32;  // q.k k-steps (8 channels per lane each)
    constexpr int E = D / 16;   // output tiles of 16 channels
    constexpr int DP = D + 4;   // padded LDS merge row
    constexpr int HC0 = kMfmaMergeFloats / (kMfmaWaves * DP);
    constexpr int HC = HC0 >= 16 ? 16 : (HC0 >= 8 ? 8 : (HC0 >= 4 ? 4 : (HC0 >= 2 ? 2 : 1)));  // columns per merge pass
    using Ops = MfmaOps<T>;

    constexpr int LDW = D + 16;                      // tile row pitch (16-bit elements)
    constexpr int TILE_ELEMS = 2 * kMfmaTile * LDW;  // K then V
    constexpr int RPI = kWave * 8 / D;               // token rows per 16-byte-per-lane load
    constexpr int NLD = kMfmaTile / RPI;             // loads per lane per tile, each of K and V
    static_assert(kMfmaTile % RPI == 0, "tile rows per load");
    constexpr size_t kTileBytes = sizeof(uint16_t) * TILE_ELEMS * kMfmaWaves;
    constexpr size_t kMergeBytes = sizeof(float) * kMfmaWaves * HC * DP;
    extern __shared__ int s_blk[];  // [sub][ids_per_seq]: the members' block ids (-1: unusable)
    __shared__ float s_m[kMfmaWaves][16], s_l[kMfmaWaves][16];
    __shared__ __align__(16) unsigned char s_raw[kTileBytes > kMergeBytes ? kTileBytes : kMergeBytes];
    __shared__ int s_ctx[kMaxSiblings];
    __shared__ int s_seg[kMaxSiblings + 2];  // first tile of each segment (shared, then members), then the total
    __shared__ int s_common, s_bad;
    auto s_o = reinterpret_cast<float (*)[HC][DP]>(s_raw);

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int c = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int hk = blockIdx.x;               // K/V head
    const int num_heads = num_kv_heads * gq;  // query heads (gq per K/V head)
    // Grid row y: sub-group y % per_group of group y / per_group; members
    // s0 .. s0 + n - 1 (a group's last sub-group, and the batch's last
    // group, may be smaller; a sub-group past the batch's end has none).
    const int per_group = (group + sub - 1) / sub;
    const int gi = blockIdx.y / per_group, si = blockIdx.y % per_group;
    const int s0 = gi * group + si * sub;
    const int n = min(min(sub, group - si * sub), num_seqs - s0);
    if (n <= 0) return;  // (workgroup-uniform)

    if (tid < n) s_ctx[tid] = context_lens[s0 + tid];
    if (tid == 0) s_bad = 0;
    __syncthreads();

    // Members with a usable context (1 .. max_context_len): their mask, the
    // first of them and the shortest context.
    int vmask = 0, m0 = 0, minctx = max_context_len;
    for (int m = n - 1; m >= 0; --m) {
        const int cm = s_ctx[m];
        if (cm > 0 && cm <= max_context_len) {
            vmask |= 1 << m;
            m0 = m;
            minctx = min(minctx, cm);
        }
    }
    const int nvalid = __builtin_popcount(vmask);
    // Matrix columns: member m's gq query heads take columns m gq .. m gq + gq - 1.
    const int ncols = n * gq;
    int vcols = 0;
    for (int m = 0; m < n; ++m)
        if ((vmask >> m) & 1) vcols |= ((1 << gq) - 1) << (m * gq);

    // Stage every usable member's block ids (entries past its context: -1).
    for (int i = tid; i < n * ids_per_seq; i += kMfmaThreads) {
        const int m = i / ids_per_seq, j = i - m * ids_per_seq;
        const int cm = s_ctx[m];
        int b = -1;
        if (((vmask >> m) & 1) && j <= ((cm - 1) >> log2_bs)) {
            b = block_tables[static_cast<int64_t>(s0 + m) * max_blocks_per_seq + j];
            b = (b >= 0 && b < num_blocks) ? b : -1;
        }
        s_blk[i] = b;
    }
    // Leading entries all usable members hold in common (only entries every
    // one of them needs: the shortest context's blocks).
    const int jmax = nvalid >= 2 ? ((minctx - 1) >> log2_bs) + 1 : 0;
    if (tid == 0) s_common = jmax;
    __syncthreads();  // ids staged, s_common initialised
    for (int j = tid; j < jmax; j += kMfmaThreads) {
        const int b0 = s_blk[m0 * ids_per_seq + j];
        bool same = true;
        for (int m = 0; m < n; ++m)
            if (((vmask >> m) & 1) && s_blk[m * ids_per_seq + j] != b0) same = false;
        if (!same) atomicMin(&s_common, j);
    }
    __syncthreads();
    const int common = __builtin_amdgcn_readfirstlane(s_common);
    const int shared_end = nvalid >= 2 ? min(common << log2_bs, minctx) : 0;  // tokens 0 .. shared_end - 1

    // Token segments: 0 = the shared prefix (every usable member's columns),
    // 1 + m = member m's tokens shared_end .. ctx_m - 1 (its columns only);
    // 16-token tiles numbered segment after segment.
    if (tid == 0) {
        int t = (shared_end + kMfmaTile - 1) / kMfmaTile;
        s_seg[0] = 0;
        for (int m = 0; m < n; ++m) {
            s_seg[1 + m] = t;
            if ((vmask >> m) & 1) t += (s_ctx[m] - shared_end + kMfmaTile - 1) / kMfmaTile;
        }
        s_seg[n + 1] = t;
    }

    // B operand of q.k: column c's query, member c / gq's query head
    // hk gq + c % gq (zero for columns past the group).
    const int64_t q_row = static_cast<int64_t>(s0 + c / gq) * num_heads + hk * gq + c % gq;
    u32x4 qv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qv[ks] = (c < ncols) ? as_u32x4(load16(q + q_row * D + 32 * ks + 8 * g)) : u32x4{0u, 0u, 0u, 0u};
    __syncthreads();  // s_seg published
    const int ntile = __builtin_amdgcn_readfirstlane(s_seg[n + 1]);
    // This workgroup's tiles [it_begin, it_end) of the list.
    const int part = blockIdx.z;
    const int it_begin = static_cast<int>(static_cast<int64_t>(ntile) * part / parts);
    const int it_end = static_cast<int>(static_cast<int64_t>(ntile) * (part + 1) / parts);

    const uint32_t blk_stride = static_cast<uint32_t>(num_kv_heads << log2_bs) * D;
    const uint32_t head_off = (static_cast<uint32_t>(hk) << log2_bs) * D;
    const int bmask = (1 << log2_bs) - 1;

    // Tile `it`: its segment, first token, end token, the member whose ids
    // address it and its column mask (all wave-uniform).
    struct TileInfo {
        int seg, tb, tend, ids, cols;
    };
    auto tile_info = [&](int it) {
        int seg = 0;
        while (seg < n && s_seg[seg + 1] <= it) ++seg;
        TileInfo ti;
        ti.seg = __builtin_amdgcn_readfirstlane(seg);
        const int first = __builtin_amdgcn_readfirstlane(s_seg[ti.seg]);
        if (ti.seg == 0) {
            ti.tb = (it - first) * kMfmaTile;
            ti.tend = shared_end;
            ti.ids = m0 * ids_per_seq;
            ti.cols = vcols;
        } else {
            const int m = ti.seg - 1;
            ti.tb = shared_end + (it - first) * kMfmaTile;
            ti.tend = __builtin_amdgcn_readfirstlane(s_ctx[m]);
            ti.ids = m * ids_per_seq;
            ti.cols = ((1 << gq) - 1) << (m * gq);
        }
        return ti;
    };

    f32x4 acc[E];
#pragma unroll
    for (int t = 0; t < E; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY;  // running maximum of column c's base-2 scores (same in the 4 lane groups)
    float l = 0.0f;       // running sum of exp2(score - m) over this lane's tokens
    uint32_t bad = 0;     // bit 0: the shared prefix, bit 1 + m: member m's own tokens

    uint16_t* const sK = reinterpret_cast<uint16_t*>(s_raw) + wave * TILE_ELEMS;
    uint16_t* const sV = sK + kMfmaTile * LDW;

    // Coalesced global loads of a tile: load i of lane L reads 16 bytes
    // (chunk L % (D / 8)) of token row RPI i + L / (D / 8), for K and V.
    // Tokens past the segment re-read its last token (masked out).  A row in
    // a block with an unusable id is not read: it is zero, so the columns
    // masked out of this tile add 0 * 0 (the product of a masked column's
    // zero probabilities with whatever such a row held could be NaN), and
    // the segment is flagged so its columns come out NaN.
    const int ld_row = lane / (D / 8), ld_ch = lane % (D / 8);
    uint4 kreg[NLD], vreg[NLD];
    auto load_tile = [&](const TileInfo& ti) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int t = min(ti.tb + RPI * i + ld_row, ti.tend - 1);
            const int b = s_blk[ti.ids + (t >> log2_bs)];
            if (b < 0) {
                bad |= 1u << ti.seg;
                kreg[i] = vreg[i] = uint4{0u, 0u, 0u, 0u};
            } else {
                const uint64_t e = static_cast<uint64_t>(static_cast<uint32_t>(b)) * blk_stride + head_off +
                                   static_cast<uint32_t>(t & bmask) * D + 8 * ld_ch;
                kreg[i] = load16<NT>(kc + e);
                vreg[i] = load16<NT>(vc + e);
            }
        }
    };
    auto store_tile = [&]() {
        // This wavefront's LDS accesses run in order; keep the compiler from
        // moving these stores above the previous tile's reads.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            *reinterpret_cast<uint4*>(sK + (RPI * i + ld_row) * LDW + 8 * ld_ch) = kreg[i];
            *reinterpret_cast<uint4*>(sV + (RPI * i + ld_row) * LDW + 8 * ld_ch) = vreg[i];
        }
        asm volatile("" ::: "memory");
    };
    auto compute_tile = [&](const TileInfo& ti) {
        // Scores S^T: lane (c, g) gets tokens tb + 4 g + j of column c.
        f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sc = Ops::qk(as_u32x4(*reinterpret_cast<const uint4*>(sK + c * LDW + 32 * ks + 8 * g)), qv[ks], sc);
        const bool col_on = (ti.cols >> c) & 1;
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = (col_on && ti.tb + 4 * g + j < ti.tend) ? sc[j] * qscale : -INFINITY;
            mx = fmaxf(mx, x[j]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // A column masked on every tile so far keeps m = -inf: its
        // probabilities are 0 and nothing is rescaled (no -inf - -inf).
        const float m_new = fmaxf(m, mx);
        if (__builtin_amdgcn_ballot_w64(m_new > m)) {
            const float alpha = (m_new > m) ? fast_exp2(m - m_new) : 1.0f;  // 0 when m was -inf
            l *= alpha;
#pragma unroll
            for (int t = 0; t < E; ++t) acc[t] *= alpha;
        }
        m = m_new;
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = (x[j] == -INFINITY) ? 0.0f : fast_exp2(x[j] - m);
            l += p[j];
        }
        uint32_t ph0, pl0, ph1, pl1;
        Ops::split(p[0], p[1], ph0, pl0);
        Ops::split(p[2], p[3], ph1, pl1);
        const u32x2 bh = u32x2{ph0, ph1}, bl = u32x2{pl0, pl1};
        // O^T += V^T P^T through transposing LDS reads (as decode_mfma_kernel).
        const uint16_t* vt = sV + (4 * g + (c >> 2)) * LDW + 4 * (c & 3);
#pragma unroll
        for (int t = 0; t < E; ++t) {
            const u32x2 a = lds_read_tr16_b64(vt + 16 * t);
            acc[t] = Ops::pv(a, bh, acc[t]);
            acc[t] = Ops::pv(a, bl, acc[t]);
        }
    };

    // Software pipeline: the next tile's loads in flight while the current
    // one is computed.
    int it = it_begin + wave;
    if (it < it_end) {
        TileInfo cur = tile_info(it);
        load_tile(cur);
        while (true) {
            store_tile();
            const int nx = it + kMfmaWaves;
            TileInfo nxt = cur;
            if (nx < it_end) {
                nxt = tile_info(nx);
                load_tile(nxt);
            }
            compute_tile(cur);
            if (nx >= it_end) break;
            it = nx;
            cur = nxt;
        }
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (bad) atomicOr(&s_bad, static_cast<int>(bad));
    __syncthreads();  // every wavefront is done with its tiles (s_o aliases them)
    const uint32_t bad_all = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(s_bad));

    // Merge the wavefronts through LDS, HC columns per pass; one output row
    // per member, or (parts > 1) one partial per member and query head: the
    // empty and impossible members' rows are then the merge kernel's, and a
    // flagged segment makes the partial NaN (sum and accumulator), which the
    // merge carries into the row whatever the partial's weight.
    if (g == 0) {
        s_m[wave][c] = m;
        s_l[wave][c] = l;
    }
    for (int c0 = 0; c0 < ncols; c0 += HC) {
        if (c >= c0 && c < c0 + HC) {
#pragma unroll
            for (int t = 0; t < E; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) s_o[wave][c - c0][16 * t + 4 * g + j] = acc[t][j];
        }
        __syncthreads();
        for (int idx = tid; idx < HC * D; idx += kMfmaThreads) {
            const int hl = idx / D, d = idx % D, col = c0 + hl;
            if (col >= ncols) continue;
            const int mem = col / gq;
            const int cm = s_ctx[mem];
            if (parts > 1) {
                if (!((vmask >> mem) & 1)) continue;
                float M = s_m[0][col];
#pragma unroll
                for (int w = 1; w < kMfmaWaves; ++w) M = fmaxf(M, s_m[w][col]);
                float L = 0.0f, O = 0.0f;
#pragma unroll
                for (int w = 0; w < kMfmaWaves; ++w) {
                    const float f = (s_m[w][col] == -INFINITY) ? 0.0f : fast_exp2(s_m[w][col] - M);
                    L = fmaf(f, s_l[w][col], L);
                    O = fmaf(f, s_o[w][hl][d], O);
                }
                if ((bad_all & 1u) || ((bad_all >> (mem + 1)) & 1u)) L = O = __builtin_nanf("");
                const int64_t slot = (static_cast<int64_t>(s0 + mem) * num_heads + hk * gq + col % gq) * parts + part;
                ws_o[slot * D + d] = O;
                if (d == 0) {
                    ws_m[slot] = M;
                    ws_l[slot] = L;
                }
                continue;
            }
            float v;
            if (cm == 0) {
                v = 0.0f;
            } else if (!((vmask >> mem) & 1) || (bad_all & 1u) || ((bad_all >> (mem + 1)) & 1u)) {
                v = __builtin_nanf("");
            } else {
                float M = s_m[0][col];
#pragma unroll
                for (int w = 1; w < kMfmaWaves; ++w) M = fmaxf(M, s_m[w][col]);
                float L = 0.0f, O = 0.0f;
#pragma unroll
                for (int w = 0; w < kMfmaWaves; ++w) {
                    const float f = (s_m[w][col] == -INFINITY) ? 0.0f : fast_exp2(s_m[w][col] - M);
                    L = fmaf(f, s_l[w][col], L);
                    O = fmaf(f, s_o[w][hl][d], O);
                }
                v = O / L;
            }
            out[(static_cast<int64_t>(s0 + mem) * num_heads + hk * gq + col % gq) * D + d] = narrow<T>(v);
        }
        __syncthreads();  // s_o is reused by the next pass
    }
}

}  // namespace pa
