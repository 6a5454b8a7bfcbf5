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
// of 16 rows, so every K and V operand it reads from LDS feeds two products):
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
//     Lane (c, g) reads D/16 channels of each of its 8 value rows from LDS
//     (16 lanes cover a row: conflict-free) and one v_perm per register
//     builds the A operand of each output tile;
//   * probabilities are split into hi + lo 16-bit parts (truncation), both
//     accumulated, so the weights keep ~16 bits (the product of two 16-bit
//     values is exact in the fp32 accumulator);
//   * online softmax per row in base 2, tile maximum shared across the four
//     lane groups of a row with two cross-row exchanges; the reference
//     maximum moves (and the accumulators are rescaled) only when a tile
//     exceeds it by more than 2^8, so the rescale is rare; the score scale is
//     one fused multiply-add;
//   * at most 2 wavefronts per SIMD (launch bound): the compiler then keeps
//     the accumulators in VGPRs (MFMA with VGPR C/D) instead of shuttling
//     them through AGPRs;
//   * causal masking per element; a wavefront skips tiles entirely past its
//     rows; workgroups are dispatched last query tile first (they have the
//     most keys).
#include <math.h>

#include "pa_decode_mfma.h"  // MfmaOps, vector types
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfBlocks = 2;                        // 16-row blocks per wavefront
constexpr int kPfRows = 16 * kPfBlocks * kPfWaves;  // query rows per workgroup
constexpr int kPfKeys = 32;                         // keys per tile
// The running maximum used as the softmax reference moves only when a tile's
// maximum exceeds it by more than this (log2 units), so the accumulators are
// rescaled rarely; probabilities stay below 2^8 (no overflow in f16/bf16 or
// fp32; the hi + lo split keeps their relative precision).
constexpr float kPfRescaleSlack = 8.0f;

template <int D>
struct PfShape {
    static constexpr int KS = D / 32;                 // q.k k-steps
    static constexpr int E = D / 16;                  // channels per lane of a V row = output tiles
    static constexpr int NW = E / 2;                  // 32-bit words per lane of a V row
    static constexpr int LD = D + 8;                  // LDS row pitch (elements): 16-byte pad
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int CHUNKS = kPfKeys * CPR;      // 16-byte chunks per tile (each of K and V)
    static constexpr int CPT = CHUNKS / kPfThreads;   // chunks per thread per tile
    static_assert(CHUNKS % kPfThreads == 0, "tile chunks must divide over the workgroup");
};

template <int NW>
__device__ __forceinline__ void lds_read_words(const uint16_t* p, uint32_t (&w)[NW]) {
    if constexpr (NW == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x;
        w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const uint4 v = reinterpret_cast<const uint4*>(p)[i];
            w[4 * i + 0] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    }
}

template <class T, int D>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start, int num_heads,
    int num_kv_heads, int log2_bs, int max_blocks_per_seq, int64_t num_blocks, int max_context_len, int n_qtiles,
    float qscale) {
    using Sh = PfShape<D>;
    constexpr int KS = Sh::KS, E = Sh::E, NW = Sh::NW, LD = Sh::LD, CPR = Sh::CPR, CPT = Sh::CPT;
    constexpr int RB = kPfBlocks;
    using Ops = MfmaOps<T>;

    extern __shared__ int s_ids[];  // block ids of keys 0 .. kv_end - 1 (dynamic size)
    __shared__ __align__(16) uint16_t sK[2][kPfKeys][LD];
    __shared__ __align__(16) uint16_t sV[2][kPfKeys][LD];

    const int h = blockIdx.x, s = blockIdx.y, qt = n_qtiles - 1 - static_cast<int>(blockIdx.z);
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = lane & 15, g = lane >> 4;

    const int q0 = __builtin_amdgcn_readfirstlane(query_start[s]);
    const int n = __builtin_amdgcn_readfirstlane(query_start[s + 1]) - q0;
    const int r0 = qt * kPfRows;  // first row of this workgroup within the chunk
    if (n <= 0 || r0 >= n) return;
    const int ctx = __builtin_amdgcn_readfirstlane(context_lens[s]);
    const int wr0 = r0 + 16 * RB * wave;  // first row of this wavefront
    if (ctx < n || ctx > max_context_len) {
        // Impossible lengths: NaN rows, nothing read.
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int row = wr0 + 16 * rb + c;
            if (row < n) {
                for (int d = g; d < D; d += 4)
                    out[(static_cast<int64_t>(q0 + row) * num_heads + h) * D + d] = narrow<T>(__builtin_nanf(""));
            }
        }
        return;
    }
    const int first_pos = ctx - n;                      // position of chunk row 0
    const int last_row = min(r0 + kPfRows, n) - 1;      // last valid row of the workgroup
    const int kv_end = first_pos + last_row + 1;        // keys 0 .. kv_end - 1 are needed (<= ctx)
    const int ntiles = (kv_end + kPfKeys - 1) / kPfKeys;
    const int G = num_heads / num_kv_heads;
    const int hk = h / G;
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
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int ci = tid + u * kPfThreads;
            const int kk = ci / CPR, cc = ci % CPR;
            const int kp = kt * kPfKeys + kk;
            if (kp < kv_end) {
                const int b = s_ids[kp >> log2_bs];
                bad |= (b < 0);
                const uint64_t e = static_cast<uint64_t>(static_cast<uint32_t>(max(b, 0))) * blk_stride + head_off +
                                   static_cast<uint32_t>(kp & bmask) * D + 8 * cc;
                kreg[u] = load16(kc + e);
                vreg[u] = load16(vc + e);
            } else {
                // Keys past the context: zeros (masked out; V must be finite).
                kreg[u] = uint4{0u, 0u, 0u, 0u};
                vreg[u] = uint4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int ci = tid + u * kPfThreads;
            const int kk = ci / CPR, cc = ci % CPR;
            *reinterpret_cast<uint4*>(&sK[buf][kk][8 * cc]) = kreg[u];
            *reinterpret_cast<uint4*>(&sV[buf][kk][8 * cc]) = vreg[u];
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
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    const u32x4 kop = as_u32x4(*reinterpret_cast<const uint4*>(&sK[buf][16 * sub + c][8 * g + 32 * ks]));
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) sc[rb][sub] = Ops::qk(kop, qv[rb][ks], sc[rb][sub]);
                }
            }
            u32x4 bh[RB], bl[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                // Keys above the diagonal exist only in tiles reaching past
                // the block's first row (wave-uniform test).
                const bool full = k0 + kPfKeys - 1 <= wpos0 + 16 * rb;
                float raw[8];
                float mx = -INFINITY;
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float v = sc[rb][sub][j];
                        if (!full) v = (k0 + 16 * sub + 4 * g + j <= pos[rb]) ? v : -INFINITY;
                        raw[4 * sub + j] = v;
                        mx = fmaxf(mx, v);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                mx *= sc_mul;  // every row has a valid key here: finite (tile 0 holds key 0)
                if (__builtin_amdgcn_ballot_w64(mx > m[rb] + kPfRescaleSlack)) {
                    const float m_new = fmaxf(m[rb], mx);
                    const float alpha = fast_exp2(m[rb] - m_new);  // 0 on the first tile (m = -inf)
                    l[rb] *= alpha;
#pragma unroll
                    for (int t = 0; t < E; ++t) acc[rb][t] *= alpha;
                    m[rb] = m_new;
                }
                float p[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    p[i] = fast_exp2(fmaf(raw[i], sc_mul, -m[rb]));  // masked: exp2(-inf) = 0
                    l[rb] += p[i];
                }
                uint32_t ph[4], pl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) Ops::split(p[2 * i], p[2 * i + 1], ph[i], pl[i]);
                bh[rb] = u32x4{ph[0], ph[1], ph[2], ph[3]};
                bl[rb] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            }

            // Value rows of keys 16 sub + 4 g + j, channels E c .. E c + E - 1.
            uint32_t vr[8][NW];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int j = 0; j < 4; ++j) lds_read_words<NW>(&sV[buf][16 * sub + 4 * g + j][E * c], vr[4 * sub + j]);
#pragma unroll
            for (int t = 0; t < E; ++t) {
                const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
                const int w = t / 2;
                const u32x4 a = u32x4{__builtin_amdgcn_perm(vr[1][w], vr[0][w], sel),
                                      __builtin_amdgcn_perm(vr[3][w], vr[2][w], sel),
                                      __builtin_amdgcn_perm(vr[5][w], vr[4][w], sel),
                                      __builtin_amdgcn_perm(vr[7][w], vr[6][w], sel)};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    acc[rb][t] = Ops::qk(a, bh[rb], acc[rb][t]);
                    acc[rb][t] = Ops::qk(a, bl[rb], acc[rb][t]);
                }
            }
        }
        if (kt + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }
    bad = __syncthreads_or(bad);

    // Lane (c, g) holds row wr0 + 16 rb + c, channels D/4 g .. D/4 g + D/4 - 1.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float lt = l[rb];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int row = wr0 + 16 * rb + c;
        if (row < n) {
            const float inv = bad ? __builtin_nanf("") : 1.0f / lt;
            uint16_t* op = out + (static_cast<int64_t>(q0 + row) * num_heads + h) * D + (D / 4) * g;
            uint32_t packed[D / 8];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < E; t += 2) {
                    const uint32_t lo = narrow<T>(acc[rb][t][j] * inv), hi = narrow<T>(acc[rb][t + 1][j] * inv);
                    packed[(E * j + t) / 2] = lo | (hi << 16);
                }
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
                reinterpret_cast<uint4*>(op)[i] =
                    uint4{packed[4 * i + 0], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]};
        }
    }
}

template <class T, int D>
hipError_t launch_prefill_t(const PrefillArgs& a) {
    const int log2_bs = __builtin_ctz(static_cast<unsigned>(a.block_size));
    const float qscale = a.scale * 1.4426950408889634f;  // log2(e)
    const int n_qtiles = (a.max_query_len + kPfRows - 1) / kPfRows;
    dim3 grid(a.num_heads, a.num_seqs, n_qtiles);
    const size_t lds = static_cast<size_t>(a.staged_ids) * sizeof(int);
    hipLaunchKernelGGL((prefill_kernel<T, D>), grid, dim3(kPfThreads), lds, a.stream, static_cast<uint16_t*>(a.out),
                       static_cast<const uint16_t*>(a.query), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.block_tables, a.context_lens, a.query_start,
                       a.num_heads, a.num_kv_heads, log2_bs, a.max_blocks_per_seq, a.num_blocks, a.max_context_len,
                       n_qtiles, qscale);
    return hipGetLastError();
}

template <class T>
hipError_t launch_prefill_dim(const PrefillArgs& a) {
    switch (a.head_dim) {
        case 64: return launch_prefill_t<T, 64>(a);
        case 128: return launch_prefill_t<T, 128>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
    return a.dtype == 1 ? launch_prefill_dim<F16>(a) : launch_prefill_dim<BF16>(a);
}

}  // namespace pa
