// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Largest number of physical blocks one KV partition may touch (its block
// ids are staged in LDS: at most 32 KB).
constexpr int kMaxPartitionBlocks = 8192;

// Launch plan of pa_decode.
//
// Work items are (sequence, K/V head, KV partition).  The hardware
// dispatches workgroups in grid order, so the order of the items decides how
// evenly the 256 compute units finish.
//  * Grouped heads (G >= 2, the matrix-core kernel), fewer pairs than the
//    longest-first threshold (512), no caller-given partition length:
//    balanced split.  One workgroup per resident slot (kBalancedWgsPerCu per
//    CU); each takes an equal share (at least kBalancedMinChunk tokens) of
//    the flat (sequence, K/V head, token) work, whatever the length mix, and
//    a merge launch combines the heads split across workgroups.
//  * Many (sequence, K/V head) pairs (>= kManyPairs): whole contexts up to
//    4096 tokens per item, in batch order (the items are many and short
//    enough).
//  * Fewer pairs but at least the longest-first threshold, and at most
//    kMaxLptSeqs sequences: whole contexts, dispatched longest first (each
//    workgroup finds the sequence of its rank; longest-processing-time-first
//    list scheduling).  No split means no merge launch.
//  * Otherwise: split contexts into the largest power-of-two partition in
//    [minimum, 4096] that still gives >= kManyPairs items, in batch order.
// The longest-first threshold and the minimum partition depend on the group
// size G (query heads per K/V head), because G >= 2 runs the matrix-core
// kernel, whose workgroups carry less per-token work and more fixed cost:
//   G = 1:  longest first from 1024 pairs, partitions of at least 256 tokens;
//   G >= 2: longest first from 512 pairs, partitions of at least 512 tokens
// (measured on MI355X: LLaMA-3-8B-shaped GQA batch 72 -> 64 us, a one-K/V-head
// 128-sequence batch 49 -> 46 us; for multi-head batches the G = 1 values
// measured best).  A caller-given partition length overrides the length
// choice.  Longest-first order is used only when no context is split: with
// splits, the empty partitions of short sequences would pay for the ranking
// before exiting.
#ifndef PA_LPT_PAIRS
#define PA_LPT_PAIRS 1024
#endif
#ifndef PA_MIN_PART
#define PA_MIN_PART 256
#endif
constexpr int kMinDefaultPartition = PA_MIN_PART;
constexpr int kMinGroupedPartition = 512;
constexpr int kMaxDefaultPartition = 4096;
constexpr int64_t kManyPairs = 8192;
constexpr int64_t kLptPairs = PA_LPT_PAIRS;
constexpr int64_t kLptGroupedPairs = 512;
constexpr int kMaxLptSeqs = 512;

// Work decompositions of the decode kernels.
constexpr int kPlanPartitions = 0;    // one workgroup per (K/V head, sequence, partition)
constexpr int kPlanLongestFirst = 1;  // whole contexts, longest sequences dispatched first
constexpr int kPlanBalanced = 2;      // equal shares of the flat (sequence, K/V head, token) work

#ifndef PA_BALANCED_WGS_PER_CU
#define PA_BALANCED_WGS_PER_CU 2  // resident matrix-core decode workgroups per CU (8 waves, <= 128 VGPRs)
#endif
constexpr int kBalancedWgsPerCu = PA_BALANCED_WGS_PER_CU;
constexpr int kBalancedMinChunk = 256;  // fewest tokens a balanced-split workgroup takes

struct DecodePlan {
    int part_tokens;
    bool longest_first;
    bool balanced;  // the matrix-core kernel splits the flat work evenly (part_tokens = smallest share)
};

inline DecodePlan plan_decode(int64_t num_seqs, int64_t num_kv_heads, int64_t group, int64_t max_context_len,
                              int partition_size) {
    const int64_t pairs = num_seqs * num_kv_heads;
    const int min_part = group >= 2 ? kMinGroupedPartition : kMinDefaultPartition;
    const int64_t lpt_pairs = group >= 2 ? kLptGroupedPairs : kLptPairs;
    int whole = min_part;
    while (whole < kMaxDefaultPartition && whole < max_context_len) whole *= 2;
    DecodePlan p{whole, false, false};
    const bool can_sort = num_seqs <= kMaxLptSeqs;
    // Grouped heads (the matrix-core kernel) with few (sequence, K/V head)
    // pairs: split the flat work evenly over the resident workgroups.  The
    // flat index must fit 31 bits.
    if (group >= 2 && partition_size == 0 && pairs < lpt_pairs && can_sort &&
        pairs * max_context_len < (int64_t{1} << 31)) {
        p.part_tokens = kBalancedMinChunk;
        p.balanced = true;
        return p;
    }
    if (pairs >= kManyPairs) {
        p.part_tokens = whole;
    } else if (pairs >= lpt_pairs && can_sort) {
        p.part_tokens = whole;
        p.longest_first = true;
    } else {
        int part = whole;
        while (part > min_part && pairs * ((max_context_len + part - 1) / part) < kManyPairs) part /= 2;
        p.part_tokens = part;
    }
    if (partition_size > 0) p.part_tokens = partition_size;
    if (p.part_tokens < max_context_len) p.longest_first = false;
    return p;
}

// Blocks a partition of `part` tokens can touch when it starts mid-block.
inline int64_t partition_blocks(int64_t part, int64_t block_size) {
    return (part + block_size - 1) / block_size + 1;
}

struct DecodeArgs {
    void* out;
    const void* query;
    void* k_cache;  // written only when key_new is set
    void* v_cache;
    const void* key_new;    // [S, H, D] newest token's K (append mode) or NULL
    const void* value_new;  // [S, H, D] newest token's V (append mode) or NULL
    const int32_t* block_tables;
    const int32_t* context_lens;
    int num_seqs, num_heads, num_kv_heads, head_dim, block_size;  // num_heads = G * num_kv_heads
    int max_blocks_per_seq, max_context_len;
    int64_t num_blocks;
    float scale;
    int dtype;
    int part_tokens, max_parts;
    int staged_blocks;  // LDS entries for a partition's block ids
    bool longest_first; // map grid rows to sequences in decreasing context length
    int pair_rows;      // matrix-core longest-first: grid rows per round of one workgroup per CU (0 = none)
    bool balanced;      // balanced split (matrix-core kernel); else partitions of part_tokens
    int balanced_wgs;   // workgroups of the balanced split
    int staged_balanced;  // LDS entries for a balanced-split run's block ids
    bool cached_loads;  // ordinary (cached) K/V loads instead of non-temporal ones
    // Sibling groups (pa_decode with PA_DECODE_SIBLINGS(n)): consecutive
    // groups of `siblings` sequences read their common leading blocks once;
    // 0 = no grouping.  sibling_ids: block ids staged per member.
    int siblings;
    int sibling_sub;  // members per workgroup: min(siblings, 16 / G)
    int sibling_ids;
    // > 1: a sub-group's tiles are split over this many workgroups, whose
    // partial results (workspace laid out as below with max_parts =
    // sibling_parts) decode_merge_kernel combines; 1: whole tile lists.
    int sibling_parts;
    // float [S*H*max_parts*D] then [S*H*max_parts] x 2, then (balanced plan)
    // int32 [S + 2]; NULL when max_parts == 1
    void* workspace;
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_decode_f32(const DecodeArgs& a);
hipError_t launch_decode_f16(const DecodeArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a);

// Sibling-group decode: at most this many members per group (the columns of
// one 16x16 matrix product) and staged block ids per workgroup.
constexpr int kMaxSiblings = 16;
constexpr int kMaxSiblingIds = 4096;
constexpr int kMaxSiblingParts = 64;  // workgroups one sub-group's tiles are split over, at most

// Query heads per K/V head with built kernels.
inline bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Prefill (pa_prefill): causal attention of packed query chunks over the
// paged context.  16-bit caches, head_dim 64, 128 or 256.
constexpr int kMaxPrefillIds = 4096;  // block ids of one context staged in LDS (16 KB)

struct PrefillArgs {
    void* out;
    const void* query;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* query_start;
    int num_seqs, num_heads, num_kv_heads, head_dim, block_size;
    int max_blocks_per_seq, max_query_len, max_context_len;
    int num_tokens;  // query rows of the call (sum of the chunk lengths)
    int64_t num_blocks;
    float scale;
    int dtype;
    int staged_ids;  // LDS entries for a context's block ids
    hipStream_t stream;
};

hipError_t launch_prefill(const PrefillArgs& a);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_heads,
                                    int row_bytes, int block_size, int64_t num_blocks,
                                    hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream);

hipError_t launch_copy_pool_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                                   const int64_t* block_pairs, int num_pairs, int64_t block_bytes,
                                   int64_t src_num_blocks, int64_t dst_num_blocks, hipStream_t stream);

}  // namespace pa
