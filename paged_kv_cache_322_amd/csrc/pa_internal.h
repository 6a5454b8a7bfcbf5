// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Largest number of physical blocks one KV partition may touch (its block
// ids are staged in LDS: at most 32 KB).
constexpr int kMaxPartitionBlocks = 8192;

// Default KV partition: the largest power of two in [256, 4096] tokens (and
// not above the next power of two of the longest context) that still yields
// at least kTargetWorkItems (sequence, head, partition) work items, so that
// the 256 compute units stay busy to the end of the grid.
constexpr int kMinDefaultPartition = 256;
constexpr int kMaxDefaultPartition = 4096;
constexpr int64_t kTargetWorkItems = 8192;

inline int default_partition_tokens(int64_t num_seqs, int64_t num_heads, int64_t max_context_len) {
    int part = kMinDefaultPartition;
    while (part < kMaxDefaultPartition && part < max_context_len) part *= 2;
    const int64_t pairs = num_seqs * num_heads;
    while (part > kMinDefaultPartition && pairs * ((max_context_len + part - 1) / part) < kTargetWorkItems)
        part /= 2;
    return part;
}

// Blocks a partition of `part` tokens can touch when it starts mid-block.
inline int64_t partition_blocks(int64_t part, int64_t block_size) {
    return (part + block_size - 1) / block_size + 1;
}

struct DecodeArgs {
    void* out;
    const void* query;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int num_seqs, num_heads, head_dim, block_size;
    int max_blocks_per_seq, max_context_len;
    int64_t num_blocks;
    float scale;
    int dtype;
    int part_tokens, max_parts;
    int staged_blocks;  // LDS entries for a partition's block ids
    void* workspace;  // float [S*H*max_parts*D] then [S*H*max_parts] x 2; NULL when max_parts == 1
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_heads,
                                    int row_bytes, int block_size, int64_t num_blocks,
                                    hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream);

}  // namespace pa
