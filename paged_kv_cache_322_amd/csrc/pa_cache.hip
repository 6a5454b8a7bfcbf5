// KV-cache updates for gfx950: slot-mapped append and copy-on-write block
// copies.  Both are pure data movement in 16-byte units (bit-exact), bound by
// HBM bandwidth.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kCopyThreads = 256;

// Append (velog "LLM Inference 8: PagedAttention", how PagedAttention works:
// a new token's K/V goes into the current block of its sequence).  One
// workgroup per token copies the token's H rows of K and of V, each row
// `row_units` 16-byte units long, to block slot / B, offset slot % B.
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ kc,
    uint4* __restrict__ vc, const int64_t* __restrict__ slot_mapping, int num_heads, int row_units,
    int log2_bs, int64_t num_slots) {
    const int i = blockIdx.x;
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t blk = slot >> log2_bs;
    const int64_t off = slot & ((int64_t{1} << log2_bs) - 1);
    const int n = num_heads * row_units;
    for (int c = threadIdx.x; c < n; c += kCopyThreads) {
        const int h = c / row_units;
        const int u = c - h * row_units;
        const int64_t src = (static_cast<int64_t>(i) * num_heads + h) * row_units + u;
        const int64_t dst = ((((blk * num_heads + h) << log2_bs) + off) * row_units) + u;
        kc[dst] = key[src];
        vc[dst] = value[src];
    }
}

// Whole-block copies between two pools (which may be the same pool), used by
// copy-on-write (PagedAttention digest, "Method": only the shared block that
// is written at a branch point is copied) and by swapping (same digest,
// scheduling and glossary: a preempted request's blocks move to CPU RAM and
// back).  grid.y = pair, grid.x = chunk of kCopyUnits 16-byte units of the
// block.  Either pool may be pinned host memory: the loads or stores then
// cross the host link, and one launch keeps every block of every pair in
// flight instead of one DMA transfer per block.
constexpr int kCopyUnits = kCopyThreads * 4;

__global__ __launch_bounds__(kCopyThreads) void copy_pool_blocks_kernel(
    uint4* dk, uint4* dv, const uint4* sk, const uint4* sv, const int64_t* __restrict__ pairs,
    int64_t units_per_block, int64_t src_num_blocks, int64_t dst_num_blocks) {
    const int p = blockIdx.y;
    const int64_t src = pairs[2 * static_cast<int64_t>(p)];
    const int64_t dst = pairs[2 * static_cast<int64_t>(p) + 1];
    if (src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks) return;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kCopyUnits;
    const int64_t hi = min(lo + kCopyUnits, units_per_block);
    const uint4* ks = sk + src * units_per_block;
    const uint4* vs = sv + src * units_per_block;
    uint4* kd = dk + dst * units_per_block;
    uint4* vd = dv + dst * units_per_block;
    for (int64_t u = lo + threadIdx.x; u < hi; u += kCopyThreads) {
        const uint4 a = ks[u], b = vs[u];
        kd[u] = a;
        vd[u] = b;
    }
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_heads,
                                    int row_bytes, int block_size, int64_t num_blocks,
                                    hipStream_t stream) {
    const int log2_bs = __builtin_ctz(static_cast<unsigned>(block_size));
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(kCopyThreads), 0, stream,
                       static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping,
                       num_heads, row_bytes / 16, log2_bs, num_blocks * block_size);
    return hipGetLastError();
}

hipError_t launch_copy_pool_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                                   const int64_t* block_pairs, int num_pairs, int64_t block_bytes,
                                   int64_t src_num_blocks, int64_t dst_num_blocks, hipStream_t stream) {
    const int64_t units = block_bytes / 16;
    const unsigned chunks = static_cast<unsigned>((units + kCopyUnits - 1) / kCopyUnits);
    hipLaunchKernelGGL(copy_pool_blocks_kernel, dim3(chunks, num_pairs), dim3(kCopyThreads), 0, stream,
                       static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), static_cast<const uint4*>(src_k),
                       static_cast<const uint4*>(src_v), block_pairs, units, src_num_blocks, dst_num_blocks);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream) {
    return launch_copy_pool_blocks(k_cache, v_cache, k_cache, v_cache, block_pairs, num_pairs, block_bytes,
                                   num_blocks, num_blocks, stream);
}

}  // namespace pa
