// Paged prefill attention on the gfx950 matrix cores (prompt and chunked
// prefill).  Host side: pa_prefill in pa_api.hip.
//
// Operation: page "vLLM PagedAttention and continuous batching architecture"
// (tech.blogsailing.com), sections 3 and 5, and page "KV cache and
// PagedAttention" (allinfo.ai.kr), key insights: newly arrived prompts are
// prefilled, possibly in fixed-size chunks, against the paged KV cache.  A
// call takes, per sequence s, a chunk of n_s query rows whose K/V rows are
// already in the cache at positions ctx_s - n_s .. ctx_s - 1; row i attends
// causally to positions 0 .. ctx_s - n_s + i:
//
//   out[row, h] = softmax_t(scale * <q[row, h], K_s[t, h/G]>) V_s[t, h/G],  t <= ctx_s - n_s + i
//
// Unlike decode, this is a real matrix product: a tile of M query rows
// against N keys is M*N*D multiply-adds for (M + N)*D loaded elements, so the
// kernel is matrix-core bound.  Design (one workgroup = 4 wavefronts = 128
// query rows of one sequence and one query head; a wavefront owns two blocks
// of 16 rows, so every K and V operand it reads from LDS feeds two products;
// at head_dim 256 one block, 64 rows per workgroup, as the accumulators and
// query operands per row are twice as large):
//
//   * the K and V rows of a 32-key tile are gathered through the block table
//     (ids staged in LDS once) into double-buffered LDS, the next tile's
//     global loads in flight while the current one is computed;
//   * scores as S^T[key][row] = K[key] . Q[row] on v_mfma_f32_16x16x32
//     (two 16-key halves, D/32 k-steps; the query rows are the B operand,
//     kept in registers);
//   * the score layout (lane L = 16g + c holds keys 4g..4g+3 of row c) is the
//     B-operand layout of the second product, so probabilities never move
//     between lanes: O^T[d][row] += V^T[d][key] . P^T[key][row] on
//     v_mfma_f32_16x16x32 with the tile's 32 keys as the contraction index.
//     The V^T operand comes straight out of the row-major V tile through
//     gfx950's transposing LDS read (ds_read_b64_tr_b16): two per output
//     tile, no register shuffles;
//   * fp16 probabilities are one round-to-nearest fp16 operand (relative
//     error <= 2^-11 each); bf16 ones are split into a truncated hi part and
//     the remainder, both accumulated, so they keep ~16 bits (the product of
//     two 16-bit values is exact in the fp32 accumulator);
//   * online softmax per row in base 2; the tile maximum is shared across
//     the four lane groups of a row with two gfx950 half-wave / row swaps
//     (v_permlane32_swap, v_permlane16_swap); the reference maximum moves
//     (and the accumulators are rescaled) only when a tile exceeds it by more
//     than 2^8, so the rescale is rare; the score scale is one fused
//     multiply-add;
//   * wavefront priority raised while a wavefront issues its products
//     (s_setprio), so the other wavefronts' softmax work fills in under them;
//   * register budget for 3 wavefronts per SIMD (<= 168 VGPRs, 3 workgroups
//     per CU), accumulators in VGPRs (MFMA with VGPR C/D); LDS rows padded
//     by 32 bytes;
//   * causal masking per element; a wavefront skips tiles entirely past its
//     rows;
//   * XCD-aware dispatch: the hardware hands workgroups to the 8 XCDs
//     round-robin by linear id, each XCD with its own L2.  Every workgroup of
//     one (sequence, K/V head) unit gets a linear id congruent to the unit
//     mod 8, so the unit's G query heads and query tiles read its K/V through
//     one L2.  Three orders per XCD:
//       - unit-major (most launched tiles hold rows: chunked prefill): the
//         units in decreasing context length (sequences ranked in LDS), and
//         all tiles and heads of a unit adjacent, last tile first, so they
//         run together and share each K/V tile through the L2 instead of
//         re-reading it from memory;
//       - packed (mixed whole prompts, where most of a padded grid's tiles
//         would be empty; at most 64 sequences): the last query tile (most
//         keys) of every chunk first, then the second last, and so on,
//         chunks in decreasing length within a level, the G heads of a unit
//         and tile adjacent: longest work first, and only tiles holding
//         rows are enumerated (each workgroup finds its tile from the chunk
//         lengths in LDS);
//       - tile-major (more sequences than can be ranked): the same level
//         order over every unit's padded tiles; empty tiles exit at once.
#include <math.h>

#include <algorithm>

#include "pa_decode_mfma.h"  // MfmaOps, vector types
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
// 16-row blocks per wavefront: two up to head_dim 128, so every K/V operand
// read from LDS feeds two products; one at head_dim 256, whose accumulators
// and query operands are twice as large per row.
constexpr int pf_blocks(int D) { return D <= 128 ? 2 : 1; }
constexpr int pf_rows(int D) { return 16 * pf_blocks(D) * kPfWaves; }  // query rows per workgroup
constexpr int kPfKeys = 32;                         // keys per tile
constexpr int kXcds = 8;                            // MI355X: XCDs, each with its own L2
constexpr int kPfPad = 16;                          // LDS row padding (elements): 32 bytes
// The running maximum used as the softmax reference moves only when a tile's
// maximum exceeds it by more than this (log2 units), so the accumulators are
// rescaled rarely; probabilities stay below 2^8 (no overflow in f16/bf16 or
// fp32).
constexpr float kPfRescaleSlack = 8.0f;
constexpr int kPfMaxRankedSeqs = 64;  // the ranked orders rank at most this many sequences
static_assert(kPfMaxRankedSeqs <= kPfThreads, "one thread ranks one sequence");

template <int D>
struct PfShape {
    static constexpr int KS = D / 32;                 // q.k k-steps
    static constexpr int E = D / 16;                  // channels per lane of a V row = output tiles
    static constexpr int LD = D + kPfPad;             // LDS row pitch (elements)
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int CHUNKS = kPfKeys * CPR;      // 16-byte chunks per tile (each of K and V)
    static constexpr int CPT = CHUNKS / kPfThreads;   // chunks per thread per tile
    static_assert(CHUNKS % kPfThreads == 0 && CPR % CPT == 0, "tile chunks must divide over the workgroup");
};

// Maximum over the four lanes c, c + 16, c + 32, c + 48 (the lane groups g
// holding one score row), with the gfx950 cross-row swaps instead of LDS
// permutes.  v_permlane32_swap(a, b) exchanges the upper half-wave of a with
// the lower half-wave of b; applied to two copies of x, the two results hold
// x of the lower and of the upper half-wave in every lane, so their maximum
// is the maximum over lanes i and i ^ 32.  v_permlane16_swap does the same
// for rows of 16 lanes (i and i ^ 16).  (The results are copied to scalars
// before the bit cast: a bit cast applied directly to an element of the
// returned pair reads element 0 with this compiler.)
__device__ __forceinline__ float swap_max(float x, bool rows32) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = rows32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                          : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

__device__ __forceinline__ float max_over_groups(float x) {
    return swap_max(swap_max(x, true), false);
}

// fp16 probabilities go to the matrix cores as one round-to-nearest fp16
// operand (11 significant bits, relative error <= 2^-11 per probability);
// bf16 ones as a truncated hi part plus the remainder (8 + 8 bits).
template <class T>
constexpr bool kPfSingleP = false;
template <>
constexpr bool kPfSingleP<F16> = true;

__device__ __forceinline__ uint32_t pack_f16_rne(float p0, float p1) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{p0, p1}), f16x2_t));
}

// acc + x.lo + x.hi for a packed pair of fp16 values x (v_dot2_f32_f16
// against (1, 1)): one instruction for two terms of a row sum.
__device__ __forceinline__ float dot2_f16_ones(uint32_t x, float acc) {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    const f16x2_t one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), one, acc, false);
}

// Register budget: <= 168 VGPRs for 3 workgroups per CU up to head_dim 128;
// at 256 the tiles' 70 KB of LDS allow two workgroups per CU, so <= 256.
constexpr int pf_waves_per_simd(int D) { return D <= 128 ? 3 : 2; }

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  In each group of 16
// lanes, lanes 4r .. 4r + 3 each point at 4 consecutive 16-bit elements, the
// four together a 16-element row segment r (r = 0..3); lane i of the group
// receives column i of the 4 x 16 block, i.e. element i of segments 0..3.
// p must be 8-byte aligned and point into LDS.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p));
    return __builtin_bit_cast(u32x2, v);
}

// Dispatch orders of the prefill grid (chosen on the host).
constexpr int kPfOrderTileMajor = 0;  // query tiles last first, every unit's tiles launched (padded)
constexpr int kPfOrderUnitMajor = 1;  // units by decreasing context, all of a unit's tiles adjacent
constexpr int kPfOrderPacked = 2;     // tile levels last first, only tiles that hold rows
constexpr int kPfMaxLevels = 64;      // packed order: at most this many row tiles per chunk
static_assert(kPfMaxLevels <= kPfThreads, "one thread counts one tile level");

// Rows of sequence s whose chunk lies inside the call's rows [0, num_tokens):
// n >= 1, or 0 for an empty chunk or one outside the call's rows (skipped).
__device__ __forceinline__ int chunk_rows(const int32_t* __restrict__ query_start, int s, int num_tokens) {
    const int q0 = query_start[s], q1 = query_start[s + 1];
    return (q0 >= 0 && q1 > q0 && q1 <= num_tokens) ? q1 - q0 : 0;
}

template <class T, int D>
__global__ __launch_bounds__(kPfThreads, pf_waves_per_simd(D)) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start, int num_heads,
    int num_kv_heads, int log2_bs, int max_blocks_per_seq, int64_t num_blocks, int max_context_len, int n_qtiles,
    int num_units, int num_tokens, int max_query_len, int order, float qscale) {
    using Sh = PfShape<D>;
    constexpr int KS = Sh::KS, E = Sh::E, LD = Sh::LD, CPR = Sh::CPR, CPT = Sh::CPT;
    constexpr int RB = pf_blocks(D);
    constexpr int kPfRows = pf_rows(D);
    using Ops = MfmaOps<T>;

    extern __shared__ int s_ids[];  // block ids of keys 0 .. kv_end - 1 (dynamic size)
    __shared__ __align__(16) uint16_t sK[2][kPfKeys][LD];
    __shared__ __align__(16) uint16_t sV[2][kPfKeys][LD];

    // Linear id -> (query tile, unit, head).  A unit is a (sequence, K/V
    // head); unit u runs on XCD u % 8, and per XCD the ids r8 = lin / 8 run
    //   tile-major: through the query tiles last first, within a tile
    //     through the XCD's units and, within a unit, its G query heads;
    //     unit u is (sequence u / Hk, K/V head u % Hk).  The grid holds
    //     ceil(units / 8) * 8 * G * n_qtiles workgroups; those of padding
    //     units and of tiles past a chunk return at once;
    //   unit-major: through the XCD's units, within a unit through its query
    //     tiles last first and, within a tile, its G query heads; unit u is
    //     (sequence of rank u / Hk in decreasing context length, K/V head
    //     u % Hk).  Same grid;
    //   packed: as tile-major (query tiles last first), but through only
    //     the units whose chunk reaches the tile: unit u is (sequence of
    //     rank u / Hk in decreasing chunk length, K/V head u % Hk), so tile
    //     qt is held by the first c_qt * Hk units, c_qt the number of chunks
    //     longer than 128 qt rows.  Only tiles holding rows are enumerated;
    //     the grid is an upper bound and the ids past the last tile return
    //     at once.
    // Ranks break ties by sequence index (num_seqs <= kPfMaxRankedSeqs:
    // host check for both ranked orders).
    const int G = num_heads / num_kv_heads;
    const int lin = static_cast<int>(blockIdx.x);
    const int xcd = lin % kXcds, r8 = lin / kXcds;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int num_seqs = num_units / num_kv_heads;
    int qt, s, hk, h;
    if (order == kPfOrderTileMajor) {
        const int per_tile = static_cast<int>(gridDim.x) / (kXcds * n_qtiles);  // units per XCD x G
        qt = n_qtiles - 1 - r8 / per_tile;
        const int unit = ((r8 % per_tile) / G) * kXcds + xcd;
        if (unit >= num_units) return;
        s = unit / num_kv_heads;
        hk = unit % num_kv_heads;
        h = hk * G + r8 % G;
    } else {
        __shared__ int s_key[kPfMaxRankedSeqs];
        __shared__ int s_lvl[kPfMaxLevels];
        __shared__ int s_pick, s_level, s_off;
        int rank, level = 0;
        if (order == kPfOrderUnitMajor) {
            const int per_unit = n_qtiles * G;
            qt = n_qtiles - 1 - (r8 % per_unit) / G;
            const int unit = (r8 / per_unit) * kXcds + xcd;
            if (unit >= num_units) return;
            rank = unit / num_kv_heads;
            hk = unit % num_kv_heads;
            h = hk * G + r8 % G;
            if (tid < num_seqs) s_key[tid] = context_lens[tid];
            __syncthreads();
        } else {
            // Rank key: the chunk's rows (0 when skipped), capped at the
            // launched tiles.  Tiles of sequence i: ceil(key / 128).
            if (tid < num_seqs) s_key[tid] = min(chunk_rows(query_start, tid, num_tokens), n_qtiles * kPfRows);
            __syncthreads();
            if (tid < n_qtiles) {
                // Level tid: query tile n_qtiles - 1 - tid (tiles with the
                // most keys first), held by the chunks longer than its start.
                int cnt = 0;
                for (int i = 0; i < num_seqs; ++i) cnt += s_key[i] > (n_qtiles - 1 - tid) * kPfRows;
                const int units_j = cnt * num_kv_heads;
                s_lvl[tid] = units_j > xcd ? (units_j - xcd + kXcds - 1) / kXcds * G : 0;
            }
            __syncthreads();
            if (tid == 0) {
                int base = 0, j = 0;
                while (j < n_qtiles && r8 >= base + s_lvl[j]) base += s_lvl[j++];
                s_level = j;
                s_off = r8 - base;
            }
            __syncthreads();
            level = __builtin_amdgcn_readfirstlane(s_level);
            if (level >= n_qtiles) return;  // past the last level (uniform)
            const int off = __builtin_amdgcn_readfirstlane(s_off);
            const int unit = (off / G) * kXcds + xcd;
            rank = unit / num_kv_heads;
            hk = unit % num_kv_heads;
            h = hk * G + off % G;
        }
        if (tid < num_seqs) {
            const int c0 = s_key[tid];
            int r = 0;
            for (int j = 0; j < num_seqs; ++j) {
                const int cj = s_key[j];
                r += (cj > c0) || (cj == c0 && j < tid);
            }
            if (r == rank) s_pick = tid;
        }
        __syncthreads();
        s = __builtin_amdgcn_readfirstlane(s_pick);
        if (order == kPfOrderPacked) qt = n_qtiles - 1 - level;
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = lane & 15, g = lane >> 4;

    // Guards on the device-side row bounds: a chunk whose rows are not inside
    // [0, num_tokens) (query_start falling, negative or past num_tokens) is
    // skipped, nothing read or written.
    const int q0 = __builtin_amdgcn_readfirstlane(query_start[s]);
    const int q1 = __builtin_amdgcn_readfirstlane(query_start[s + 1]);
    if (q0 < 0 || q1 <= q0 || q1 > num_tokens) return;
    const int n = q1 - q0;
    const int r0 = qt * kPfRows;  // first row of this workgroup within the chunk
    if (r0 >= n) return;
    const int ctx = __builtin_amdgcn_readfirstlane(context_lens[s]);
    const int wr0 = r0 + 16 * RB * wave;  // first row of this wavefront
    if (ctx < n || ctx > max_context_len || n > max_query_len) {
        // Impossible lengths: NaN rows, nothing read.  A chunk longer than
        // max_query_len has tiles only up to n_qtiles; the last of them
        // writes every row past its start.
        const int row_end = (n > max_query_len && qt == n_qtiles - 1) ? n : min(r0 + kPfRows, n);
        const uint16_t nan_bits = narrow<T>(__builtin_nanf(""));
        for (int row = r0 + tid / (D / 2); row < row_end; row += kPfThreads / (D / 2)) {
            uint32_t* op = reinterpret_cast<uint32_t*>(out + (static_cast<int64_t>(q0 + row) * num_heads + h) * D);
            op[tid % (D / 2)] = nan_bits * 0x10001u;
        }
        return;
    }
    const int first_pos = ctx - n;                      // position of chunk row 0
    const int last_row = min(r0 + kPfRows, n) - 1;      // last valid row of the workgroup
    const int kv_end = first_pos + last_row + 1;        // keys 0 .. kv_end - 1 are needed (<= ctx)
    const int ntiles = (kv_end + kPfKeys - 1) / kPfKeys;
    const int bmask = (1 << log2_bs) - 1;
    const int nids = ((kv_end - 1) >> log2_bs) + 1;

    const int32_t* bt = block_tables + static_cast<int64_t>(s) * max_blocks_per_seq;
    for (int i = tid; i < nids; i += kPfThreads) {
        const int b = bt[i];
        s_ids[i] = (b >= 0 && b < num_blocks) ? b : -1;
    }

    // B operands of q.k: query rows wr0 + 16 rb + c (rows past the chunk
    // re-read its last row; they are never written).  A negative scale is
    // folded into the query by flipping its sign bits (exact), so the scale
    // applied to the scores is >= 0 and the maximum commutes with it.
    const uint32_t sign = qscale < 0.0f ? 0x80008000u : 0u;
    const float sc_mul = fabsf(qscale);
    u32x4 qv[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int qrow = min(wr0 + 16 * rb + c, n - 1);
        const uint16_t* qp = q + (static_cast<int64_t>(q0 + qrow) * num_heads + h) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qv[rb][ks] = as_u32x4(load16(qp + 32 * ks)) ^ sign;
    }
    __syncthreads();  // s_ids staged

    const uint32_t blk_stride = static_cast<uint32_t>(num_kv_heads << log2_bs) * D;
    const uint32_t head_off = (static_cast<uint32_t>(hk) << log2_bs) * D;
    int bad = 0;

    uint4 kreg[CPT], vreg[CPT];
    // Thread tid moves CPT 16-byte chunks of one key row (one block-table
    // lookup per tile): row tid / (CPR / CPT), chunks tid % (CPR / CPT) +
    // u CPR / CPT, so each LDS store instruction writes whole row halves
    // (no bank conflicts).
    const int ld_row = tid / (CPR / CPT), ld_chunk = tid % (CPR / CPT);
    auto load_tile = [&](int kt) {
        // Keys past kv_end (the last tile's tail) re-read key kv_end - 1:
        // they are masked out of every row, and the value row read is a real
        // one (finite, as 0 * V must be).
        const int kp = min(kt * kPfKeys + ld_row, kv_end - 1);
        const int b = s_ids[kp >> log2_bs];
        bad |= (b < 0);
        const uint64_t e = static_cast<uint64_t>(static_cast<uint32_t>(max(b, 0))) * blk_stride + head_off +
                           static_cast<uint32_t>(kp & bmask) * D + 8 * ld_chunk;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            kreg[u] = load16(kc + e + 8 * (CPR / CPT) * u);
            vreg[u] = load16(vc + e + 8 * (CPR / CPT) * u);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            *reinterpret_cast<uint4*>(&sK[buf][ld_row][8 * (ld_chunk + (CPR / CPT) * u)]) = kreg[u];
            *reinterpret_cast<uint4*>(&sV[buf][ld_row][8 * (ld_chunk + (CPR / CPT) * u)]) = vreg[u];
        }
    };

    f32x4 acc[RB][E];
    float m[RB], l[RB];  // per row c: softmax reference (same in the 4 lane groups), this lane's sum
    int pos[RB];         // position of this lane's row in each block (padding rows clamped)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int t = 0; t < E; ++t) acc[rb][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        m[rb] = -INFINITY;
        l[rb] = 0.0f;
        pos[rb] = min(first_pos + wr0 + 16 * rb + c, ctx - 1);
    }
    const int wpos0 = first_pos + wr0;                        // position of the wavefront's first row
    const int wave_last_key = min(wpos0 + 16 * RB - 1, ctx - 1);  // wave-uniform

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ntiles) load_tile(kt + 1);
        const int k0 = kt * kPfKeys;
        if (wr0 < n && k0 <= wave_last_key) {
            // Scores S^T: lane (c, g) gets keys k0 + 16 sub + 4 g + j of row
            // wr0 + 16 rb + c.  Each key operand serves both row blocks.
            f32x4 sc[RB][2];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) sc[rb][sub] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            // Issue priority: a wavefront issuing matrix-core products goes
            // first, so other wavefronts' softmax instructions fill the
            // cycles under its products instead of delaying them.
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    const u32x4 kop = as_u32x4(*reinterpret_cast<const uint4*>(&sK[buf][16 * sub + c][8 * g + 32 * ks]));
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) sc[rb][sub] = Ops::qk(kop, qv[rb][ks], sc[rb][sub]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            u32x4 bh[RB], bl[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                float raw[8];
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int j = 0; j < 4; ++j) raw[4 * sub + j] = sc[rb][sub][j];
                // Exponent arguments against the current reference m.
                float t[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = fmaf(raw[i], sc_mul, -m[rb]);
                // Keys above the diagonal exist only in tiles reaching past
                // the block's first row (wave-uniform test).  Key k0 + 16 sub
                // + 4 g + j is visible to this lane's row iff 16 sub + j <=
                // pos - k0 - 4 g; a hidden key gets exponent -inf (p = 0),
                // whatever the scale (also 0).
                const bool full = k0 + kPfKeys - 1 <= wpos0 + 16 * rb;
                if (!full) {
                    // (The empty asm keeps this a branch around the tile
                    // instead of selects executed on every tile.)
                    asm volatile("");
                    const int lim = pos[rb] - k0 - 4 * g;
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (16 * sub + j > lim) t[4 * sub + j] = -INFINITY;
                }
                float tmax = t[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, t[i]);
                // The reference moves only when some key of the wavefront's
                // rows exceeds it by more than the slack (always on the
                // first tile, where m = -inf); then the row maximum over
                // the visible keys becomes the reference.
                if (__builtin_amdgcn_ballot_w64(tmax > kPfRescaleSlack)) {
                    // Visible keys are those whose exponent argument is not
                    // -inf (finite scores give a finite or +inf argument).
                    float mr = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (t[i] > -INFINITY) mr = fmaxf(mr, raw[i]);
                    // Every row sees key 0 on tile 0, so m is finite from then on.
                    const float m_new = fmaxf(m[rb], max_over_groups(mr) * sc_mul);
                    const float alpha = fast_exp2(m[rb] - m_new);  // 0 on the first tile (m = -inf)
                    l[rb] *= alpha;
#pragma unroll
                    for (int t2 = 0; t2 < E; ++t2) acc[rb][t2] *= alpha;
                    m[rb] = m_new;
#pragma unroll
                    for (int i = 0; i < 8; ++i) t[i] = t[i] > -INFINITY ? fmaf(raw[i], sc_mul, -m_new) : -INFINITY;
                }
                float p[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) p[i] = fast_exp2(t[i]);  // <= 2^slack
                uint32_t ph[4], pl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (kPfSingleP<T>) {
                        // The row sum takes the rounded fp16 probabilities the
                        // product uses, two per dot instruction.
                        ph[i] = pack_f16_rne(p[2 * i], p[2 * i + 1]);
                        l[rb] = dot2_f16_ones(ph[i], l[rb]);
                    } else {
                        Ops::split(p[2 * i], p[2 * i + 1], ph[i], pl[i]);
                        l[rb] += p[2 * i] + p[2 * i + 1];
                    }
                }
                bh[rb] = u32x4{ph[0], ph[1], ph[2], ph[3]};
                if constexpr (!kPfSingleP<T>) bl[rb] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            }

            // A operand of output tile t (channels 16 t .. 16 t + 15): lane
            // (c, g) needs channel 16 t + c of keys 4 g + j and 16 + 4 g + j
            // (j = 0..3, the contraction order of the probabilities); two
            // transposing reads, lanes 4 r + q of a group pointing at key
            // row 4 g + r (+ 16), channels 16 t + 4 q .. 16 t + 4 q + 3.
            const int tr_row = 4 * g + (c >> 2), tr_col = 4 * (c & 3);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int t = 0; t < E; ++t) {
                const u32x2 lo4 = lds_read_tr16(&sV[buf][tr_row][16 * t + tr_col]);
                const u32x2 hi4 = lds_read_tr16(&sV[buf][16 + tr_row][16 * t + tr_col]);
                const u32x4 a = u32x4{lo4.x, lo4.y, hi4.x, hi4.y};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    acc[rb][t] = Ops::qk(a, bh[rb], acc[rb][t]);
                    if constexpr (!kPfSingleP<T>) acc[rb][t] = Ops::qk(a, bl[rb], acc[rb][t]);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if (kt + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }
    bad = __syncthreads_or(bad);

    // Lane (c, g) holds row wr0 + 16 rb + c: acc[rb][t][j] is channel
    // 16 t + 4 g + j (transposing reads) or D/4 g + E j + t (row reads).
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float lt = l[rb];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int row = wr0 + 16 * rb + c;
        if (row < n) {
            const float inv = bad ? __builtin_nanf("") : 1.0f / lt;
            uint16_t* op = out + (static_cast<int64_t>(q0 + row) * num_heads + h) * D + 4 * g;
#pragma unroll
            for (int t = 0; t < E; ++t) {
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = narrow<T>(acc[rb][t][j] * inv);
                const uint32_t w0 = w[0] | (w[1] << 16), w1 = w[2] | (w[3] << 16);
                *reinterpret_cast<uint2*>(op + 16 * t) = uint2{w0, w1};
            }
        }
    }
}

template <class T, int D>
hipError_t launch_prefill_t(const PrefillArgs& a) {
    constexpr int kPfRows = pf_rows(D);
    const int log2_bs = __builtin_ctz(static_cast<unsigned>(a.block_size));
    const float qscale = a.scale * 1.4426950408889634f;  // log2(e)
    const int n_qtiles = (a.max_query_len + kPfRows - 1) / kPfRows;
    const int num_units = a.num_seqs * a.num_kv_heads;
    const int G = a.num_heads / a.num_kv_heads;
    const int64_t groups = (num_units + kXcds - 1) / kXcds;
    const int64_t padded = groups * kXcds * G * n_qtiles;  // every unit's n_qtiles tiles
    // Unit-major order when at least half of the launched query tiles hold
    // rows (the chunks fill their tiles); otherwise the packed order, which
    // launches only tiles holding rows, when the sequences can be ranked;
    // tile-major beyond that.
    const bool rankable = a.num_seqs <= kPfMaxRankedSeqs;
    int order = kPfOrderTileMajor;
    int64_t wgs = padded;
    if (rankable && 2 * static_cast<int64_t>(a.num_tokens) >= static_cast<int64_t>(a.num_seqs) * n_qtiles * kPfRows) {
        order = kPfOrderUnitMajor;
    } else if (rankable && n_qtiles <= kPfMaxLevels) {
        // Chunks inside [0, num_tokens) hold at most (num_tokens + 127 S) /
        // 128 tiles in all; an XCD's share of level j is at most
        // ceil(c_j Hk / 8) units, so per XCD at most that total * Hk / 8 +
        // n_qtiles units (G workgroups each).
        order = kPfOrderPacked;
        const int64_t tiles = (static_cast<int64_t>(a.num_tokens) + (kPfRows - 1) * int64_t{a.num_seqs}) / kPfRows;
        const int64_t per_xcd = (tiles * a.num_kv_heads + kXcds - 1) / kXcds + n_qtiles;
        wgs = std::min(padded, per_xcd * kXcds * G);
    }
    dim3 grid(static_cast<unsigned>(wgs));
    const size_t lds = static_cast<size_t>(a.staged_ids) * sizeof(int);
    hipLaunchKernelGGL((prefill_kernel<T, D>), grid, dim3(kPfThreads), lds, a.stream, static_cast<uint16_t*>(a.out),
                       static_cast<const uint16_t*>(a.query), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.block_tables, a.context_lens, a.query_start,
                       a.num_heads, a.num_kv_heads, log2_bs, a.max_blocks_per_seq, a.num_blocks, a.max_context_len,
                       n_qtiles, num_units, a.num_tokens, a.max_query_len, order, qscale);
    return hipGetLastError();
}

template <class T>
hipError_t launch_prefill_dim(const PrefillArgs& a) {
    switch (a.head_dim) {
        case 64: return launch_prefill_t<T, 64>(a);
        case 128: return launch_prefill_t<T, 128>(a);
        case 256: return launch_prefill_t<T, 256>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
    return a.dtype == 1 ? launch_prefill_dim<F16>(a) : launch_prefill_dim<BF16>(a);
}

}  // namespace pa
