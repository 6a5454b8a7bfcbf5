// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Largest number of physical blocks one KV partition may touch; bounds the
// LDS array that stages a partition's block ids.
constexpr int kMaxPartitionBlocks = 512;
constexpr int kDefaultPartitionTokens = 512;

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
