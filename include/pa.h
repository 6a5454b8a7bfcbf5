/*
 * pa.h - C ABI of libpa, paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * Three operations on a KV cache that is cut into fixed-size physical blocks
 * of B tokens and addressed through per-sequence block tables:
 *
 *   pa_decode             single-query (decode) attention over the blocks
 *   pa_reshape_and_cache  write new tokens' K/V rows into slot-mapped blocks
 *   pa_copy_blocks        copy-on-write duplication of whole blocks
 *   pa_append_decode      pa_reshape_and_cache of each sequence's newest
 *                         token fused with pa_decode (one launch)
 *   pa_prefill            causal attention of new prompt tokens (chunks)
 *                         over the paged context
 *   pa_swap_blocks        whole blocks between the device caches and a
 *                         pinned host pool (preemption by swapping)
 *
 * Memory layout (every array dense, row-major, no padding):
 *   query, out          [num_seqs, num_heads, head_dim]              element type `dtype`
 *   k_cache, v_cache    [num_blocks, num_heads, block_size, head_dim] element type `dtype`
 *   block_tables        int32 [num_seqs, max_blocks_per_seq]; entry j of row s
 *                       is the physical block holding tokens j*B .. j*B+B-1 of
 *                       sequence s; entries at j >= ceil(ctx_s / B) are never read
 *   context_lens        int32 [num_seqs]
 *   slot_mapping        int64 [num_tokens]; slot = block * B + offset, < 0 = skip
 *   block_pairs         int64 [num_pairs, 2]; (src, dst) physical block ids
 * bf16 is the upper half of an IEEE binary32; f16 is IEEE binary16.
 *
 * Ownership and execution: every pointer argument other than the scalars is
 * device memory owned by the caller (query, caches, tables, lengths, slot
 * mapping, pairs, out, workspace); pa_swap_blocks also takes pinned host
 * memory.  The library allocates nothing, frees
 * nothing and never synchronises: each call validates its arguments on the
 * host, enqueues its kernels on `stream` (a hipStream_t; NULL is the null
 * stream) and returns.  Apart from the scratch array of pa_decode_static
 * (one per GPU, see there) the library keeps no global state, so calls are
 * re-entrant; calls on one stream execute in order.
 *
 * Errors: the return value is a pa_status.  Argument errors are detected on
 * the host before anything is enqueued.  PA_ERR_HIP reports a failed launch.
 * Contents of device memory are the caller's contract and are not checked on
 * the host (the kernels guard their own reads and writes, see each call).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_F32 = 0,  /* IEEE binary32 */
    PA_F16 = 1,  /* IEEE binary16 */
    PA_BF16 = 2  /* bfloat16 */
} pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,        /* a required pointer is NULL */
    PA_ERR_UNSUPPORTED = 2, /* dtype, head_dim or block_size outside the built kernels */
    PA_ERR_INVALID = 3,     /* sizes, alignment, scale or workspace out of range */
    PA_ERR_HIP = 4,         /* the HIP runtime rejected a launch */
    PA_ERR_OUT_OF_BLOCKS = 5, /* block manager: not enough free blocks (nothing changed) */
    PA_ERR_SCRATCH = 6        /* pa_decode_static: more scratch needed than PA_STATIC_SCRATCH_BYTES */
} pa_status;

/* pa_decode / pa_append_decode flags. */
#define PA_DECODE_SHARED_BLOCKS 1u /* some blocks are read by several sequences of the batch
                                      (forked samples, shared prefixes): load K/V through the
                                      caches so sibling sequences hit in L2.  Without it, K/V
                                      are streamed with non-temporal loads, the faster choice
                                      when every block is read once.  Results are identical. */
#define PA_DECODE_SIBLINGS(n) ((uint32_t)(n) << 8)
                                   /* pa_decode: consecutive groups of n (2 .. 16) sequences are
                                      siblings (samples forked from one prompt, beam candidates):
                                      sequences n*k .. n*k+n-1 form group k (the last group may be
                                      smaller).  The library compares the members' block tables and
                                      reads the leading blocks they all hold (the same physical ids)
                                      once per group and head, for all members together; each
                                      member's other tokens are read from its own blocks.  A hint:
                                      nothing is assumed that the tables do not show.  One
                                      workgroup per (group, K/V head) takes up to 16 / G members
                                      (G = num_heads / num_kv_heads): a larger group is cut into
                                      consecutive sub-groups of u = min(n, floor(16 / G)) members,
                                      each reading the blocks its members share once.  Taken for
                                      16-bit caches, head_dim 64, 128 or 256, u >= 2 (G <= 8) and
                                      u * ceil(max_context_len / B) <= 4096, over whole contexts
                                      (partition_size is then not used).  Where its workgroups
                                      (sub-groups x num_kv_heads) are fewer than half the GPU's
                                      compute units and max_context_len >= 1024, one round of
                                      them would leave most of the GPU idle: each sub-group's
                                      tiles are then split over several workgroups (about one
                                      per compute unit), whose partial results a second kernel
                                      merges, as many as the workspace the call needs without
                                      the hint (pa_decode_workspace_size) holds; with room for
                                      fewer than two the hint is declined.  Not taken, the hint
                                      still makes K/V load through the caches, as
                                      PA_DECODE_SHARED_BLOCKS does (the results do not depend on
                                      the load policy).  Taken, the arithmetic (fp32
                                      products and softmax, probabilities as hi and lo 16-bit
                                      parts) differs from the multi-head kernel's only by fp32
                                      rounding.  Each block shared within a group is then
                                      read once per (sub-group, head): PA_DECODE_SHARED_BLOCKS is not
                                      needed for it (the streaming loads are faster).  n = 0 or 1:
                                      no grouping; n > 16: PA_ERR_INVALID.  Ignored by
                                      pa_append_decode. */

/* Supported shapes: head_dim in {8, 16, 32, 64, 128, 256}; block_size a power
 * of two in [1, 256]; num_seqs and num_heads at most 65535. */

/*
 * pa_decode_partition_tokens - KV partition length pa_decode will use.
 *
 * Each (sequence, K/V head) context is split into partitions of this many
 * tokens, one workgroup each (serving all query heads of that K/V head);
 * workgroups are dispatched in grid order.  A positive `partition_size` is
 * returned unchanged.  0 selects the default, from the number of
 * (sequence, K/V head) pairs R = num_seqs * num_kv_heads and the group size
 * G = num_heads / num_kv_heads.
 *
 * Balanced split (G >= 2, R < 512, R * max_context_len < 2^31): returns
 * 256, the smallest piece.  The matrix-core kernel then cuts each (sequence,
 * K/V head) context into n = ceil(ctx / C) equal pieces, with C (>= 256)
 * chosen on the device from the batch's total so that the pieces about fill
 * the resident workgroups (2 per compute unit, 1 for head_dim 256),
 * whatever the mix of context lengths; heads cut into several pieces are
 * merged by a second launch.  (For caches the matrix-core kernel does not serve, fp32 or
 * head_dim below 64, and when a share would stage more than 6144 block ids,
 * pa_decode uses partitions of 256 tokens instead.)
 *
 * Otherwise, with Pmin = 256 and Rlpt = 1024 for G = 1, Pmin = 512 and
 * Rlpt = 512 for G >= 2:
 *   R >= 8192:  the whole context (next power of two of max_context_len,
 *               clamped to [Pmin, 4096]) per workgroup, in batch order;
 *   Rlpt <= R < 8192 and num_seqs <= 512:  whole contexts as above,
 *               dispatched longest context first (no split, no merge launch);
 *               with G >= 2 the second round of one workgroup per compute
 *               unit takes its sequences in increasing length, so each
 *               unit's two slots pair a long and a short context;
 *   otherwise:  the largest power of two in [Pmin, 4096] (not above the
 *               next power of two of max_context_len) that still gives
 *               R * ceil(max_context_len / P) >= 8192 work items, in batch
 *               order.
 * Longest-first order applies only when no context is split.
 * Returns 0 for invalid sizes (num_heads not a multiple of num_kv_heads
 * included).
 */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode_workspace_size - bytes of device scratch pa_decode needs.
 *
 * When a context spans several partitions, each partition's unnormalised
 * partial result (fp32 accumulator, maximum, sum) goes to the workspace and a
 * second kernel merges them.  Under a balanced split the workspace holds
 * ceil(max_context_len / 256) + 1 partials per query head and one int32
 * (the piece length).  Returns 0 when no sequence can span two
 * partitions (then pa_decode accepts a NULL workspace), and 0 for invalid
 * sizes.  `partition_size` as for pa_decode_partition_tokens.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode - paged single-query attention.
 *
 * Defined by the page "PagedAttention - Efficient Memory Management for LLM
 * Serving with vLLM" (irregular6612.github.io), section "Method": the KV cache
 * is split into fixed-size blocks of B tokens, attention follows the block
 * table to gather a sequence's non-contiguous blocks and evaluates
 * softmax(Q K^T) V.  For every sequence s and head h:
 *
 *   out[s,h,:] = sum_t softmax_t( scale * <query[s,h,:], K_s[t,h,:]> ) * V_s[t,h,:]
 *
 * over t = 0 .. context_lens[s]-1, where token t of sequence s is stored in
 * physical block block_tables[s][t / B] at offset t % B.  With
 * num_kv_heads < num_heads (grouped-query attention, which the digest's
 * related work names as an orthogonal way to shrink the cache) the caches
 * hold num_kv_heads heads and query head h reads K/V head h / G,
 * G = num_heads / num_kv_heads in {1, 2, 4, 8}.  Arithmetic is fp32
 * (fp32 accumulation of products of widened inputs); out is rounded to
 * `dtype` with round-to-nearest-even.
 *
 *   out            [S, H, D] written
 *   query          [S, H, D] read
 *   k_cache, v_cache  [N, Hk, B, D] read, Hk = num_kv_heads
 *   block_tables   int32 [S, max_blocks_per_seq] read
 *   context_lens   int32 [S] read
 *   max_context_len  host upper bound of context_lens (sizes the grid without
 *                  a device-to-host copy); must be <= max_blocks_per_seq * B
 *   num_blocks     N, the number of physical blocks in each cache
 *   scale          finite softmax scale (1/sqrt(D) for standard attention)
 *   partition_size tokens per KV partition, 0 = default (see
 *                  pa_decode_partition_tokens); ceil(P / B) + 1 <= 8192
 *   flags          PA_DECODE_SHARED_BLOCKS and/or PA_DECODE_SIBLINGS(n) (other bits:
 *                  PA_ERR_INVALID)
 *   workspace      device scratch of at least pa_decode_workspace_size(...)
 *                  bytes, 4-byte aligned; contents need no initialisation
 *
 * query, out and both caches must be 16-byte aligned, and one block of one
 * cache (num_kv_heads * block_size * head_dim elements) below 2^31 elements.
 * num_heads must be a multiple of num_kv_heads (else PA_ERR_INVALID) with a
 * built group size (else PA_ERR_UNSUPPORTED).
 * Device-side guards:
 * a context length of 0 yields zeros; a context length below 0 or above
 * max_context_len, or a needed block id outside [0, N), yields NaN for that
 * (sequence, head) without reading outside the caches.
 */
int pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens,
              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
              float scale, int32_t dtype, int32_t partition_size, uint32_t flags,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_append_decode - one decode step: store every sequence's newest K/V row,
 * then attend over the whole context, in a single launch.
 *
 * The same result as pa_reshape_and_cache with
 *   slot_mapping[s] = block_tables[s][(ctx_s - 1) / B] * B + (ctx_s - 1) % B
 * followed by pa_decode (the newest token of a sequence is its last context
 * token; a new block is taken only when the current one is full, Velog "LLM
 * Inference 8: PagedAttention", how PagedAttention works).  key and value
 * are [S, Hk, D] in `dtype`, 16-byte aligned: row s is token ctx_s - 1 of
 * sequence s.  The workgroup whose KV partition holds that token writes the
 * rows into both caches and reads them from key/value directly.  A sequence
 * with context length 0 (or an impossible one, see pa_decode) stores
 * nothing.  Other arguments, errors and guards as for pa_decode; the block
 * holding a newest token must not be shared with another sequence (copy it
 * first with pa_copy_blocks).
 */
int pa_append_decode(void* out, const void* query, const void* key, const void* value,
                     void* k_cache, void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                     int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype,
                     int32_t partition_size, uint32_t flags, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * pa_decode_static - pa_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that must not call the allocator, harnesses that forbid it).
 *
 * Same arguments (minus workspace and workspace_bytes), results, guards and
 * errors as pa_decode; it runs the same kernels.  When the call's plan splits
 * contexts, the partial results go to a scratch buffer the library holds in
 * device memory: a file-scope array of PA_STATIC_SCRATCH_BYTES, one copy per
 * GPU the library runs on, kept until the process ends (the copy of the GPU
 * that `stream` belongs to, or of the current GPU for the null stream).
 * Nothing is allocated or freed by the call.  A call whose plan needs more than
 * PA_STATIC_SCRATCH_BYTES (pa_decode_workspace_size of the same arguments)
 * returns PA_ERR_SCRATCH before anything is enqueued.  The scratch needs no
 * initialisation (every partial is written before it is read).
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (different streams, or host threads racing) race on it and give
 * undefined results; calls on one stream are ordered and safe.
 */
#define PA_STATIC_SCRATCH_BYTES (32u << 20) /* 32 MiB per GPU */
int pa_decode_static(void* out, const void* query, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks, float scale,
                     int32_t dtype, int32_t partition_size, uint32_t flags, void* stream);

/*
 * pa_reshape_and_cache - store new tokens' keys and values in their slots.
 *
 * Page "LLM Inference 8: PagedAttention" (velog.io), section on how
 * PagedAttention works: each new token's key and value go into the
 * sequence's current physical block, and a fresh block is taken only when
 * that block is full (the caller's allocator does this and encodes the
 * result as the slot mapping).  For every i with slot = slot_mapping[i] >= 0:
 *
 *   k_cache[slot / B, h, slot % B, :] = key[i, h, :]    for every head h
 *   v_cache[slot / B, h, slot % B, :] = value[i, h, :]
 *
 * A bit-exact copy (no arithmetic).  key, value [num_tokens, H, D] read,
 * H the caches' head count (num_kv_heads for grouped-query attention);
 * caches written in place.  key, value and the caches must be 16-byte
 * aligned.  Slots must be distinct (duplicates race); a slot at or beyond
 * num_blocks * B is skipped by the kernel.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         int32_t dtype, void* stream);

/*
 * pa_copy_blocks - copy-on-write block duplication.
 *
 * PagedAttention digest (irregular6612.github.io), section "Method": samples
 * of parallel sampling or beam search share the prompt's physical blocks,
 * and when a shared block is written at the branch point only that block is
 * copied.  For every pair (src, dst) in block_pairs:
 *
 *   k_cache[dst] = k_cache[src];  v_cache[dst] = v_cache[src]
 *
 * whole blocks (all heads, slots and channels), bit-exact.  Destinations must
 * be distinct and disjoint from the sources (otherwise the result depends on
 * execution order); a pair with an id outside [0, num_blocks) is skipped by
 * the kernel.  The caches must be 16-byte aligned.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int32_t num_pairs,
                   int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int32_t dtype, void* stream);

/*
 * pa_prefill - causal attention of new prompt tokens over the paged context
 * (whole-prompt and chunked prefill).
 *
 * Page "vLLM PagedAttention and continuous batching architecture"
 * (tech.blogsailing.com), sections 3 and 5, and page "KV cache and
 * PagedAttention: LLM inference speed and GPU throughput" (allinfo.ai.kr),
 * key insights: newly arrived prompts are prefilled against the paged KV
 * cache, with chunked prefill in fixed-size chunks after the prompt's
 * earlier chunks (or a cached shared prefix).  Each sequence s brings a
 * chunk of n_s query rows whose K/V rows are already stored (e.g. by
 * pa_reshape_and_cache) at positions ctx_s - n_s .. ctx_s - 1 of its
 * context.  Row i of the chunk attends causally to positions
 * 0 .. ctx_s - n_s + i:
 *
 *   out[r, h, :] = sum_t softmax_t( scale * <query[r,h,:], K_s[t, h/G, :]> ) * V_s[t, h/G, :]
 *
 * with r = query_start[s] + i, t over 0 .. ctx_s - n_s + i, and token t at
 * block block_tables[s][t / B], offset t % B.  G = num_heads / num_kv_heads
 * (any divisor).  Arithmetic: q.k products of the stored 16-bit values
 * accumulated in fp32; softmax in fp32 (base 2); the probabilities enter
 * the p.v products as 16-bit matrix-core operands, accumulated in fp32:
 *   - bf16: each probability p as a truncated bf16 hi part plus the bf16
 *     rounding of the remainder (about 16 significant bits);
 *   - f16: each probability as one round-to-nearest-even fp16 value p~
 *     (relative error <= 2^-11, or 2^-25 absolute where p~ is subnormal),
 *     and the row sum adds the same rounded values, so the output is the
 *     exact softmax average under perturbed weights: its error is at most
 *     2^-11 * sum_t w_t |V_t - out| + 2^-25 * sum_t |V_t - out| (w the
 *     softmax weights) plus fp32 accumulation and the final rounding.
 *     With N(0,1) values that is far below 2e-3; where V rows are large and
 *     cancel (e.g. +-64) it can exceed 2e-3 (pa_decode keeps fp32
 *     probabilities there).
 * out is rounded to `dtype` (nearest-even).
 *
 *   out, query     [num_tokens, num_heads, head_dim], packed by sequence
 *   query_start    int32 [num_seqs + 1], device: rising from 0 to num_tokens;
 *                  sequence s owns rows query_start[s] .. query_start[s+1]-1
 *   context_lens   int32 [num_seqs], device: ctx_s, the chunk included
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_dim] read
 *   block_tables   int32 [num_seqs, max_blocks_per_seq]
 *   max_query_len  host upper bound of every n_s (sizes the grid)
 *   max_context_len  host upper bound of every ctx_s; <= max_blocks_per_seq *
 *                  block_size and ceil(max_context_len / block_size) <= 4096
 *
 * Built for dtype PA_F16 and PA_BF16 with head_dim 64, 128 or 256 (others:
 * PA_ERR_UNSUPPORTED).  query, out and the caches 16-byte aligned.  Ownership,
 * streams and host-side errors as for pa_decode.  Device-side guards (the
 * kernel checks what it reads from device memory, nothing faults):
 *   - a chunk whose rows are not inside [0, num_tokens) (query_start[s] < 0,
 *     query_start[s+1] <= query_start[s], or query_start[s+1] > num_tokens)
 *     is skipped: nothing read or written for it (an empty chunk, n_s = 0,
 *     is the ordinary case of this);
 *   - n_s > ctx_s, ctx_s > max_context_len or n_s > max_query_len gives NaN
 *     in every row of that chunk;
 *   - a needed block id outside [0, num_blocks) gives NaN for the rows of
 *     that (row tile, head) without reading outside the caches (tiles of
 *     128 rows, 64 at head_dim 256).
 * Chunks of a query_start that is not non-decreasing may overlap; their
 * rows are then undefined (some may be left unwritten).
 */
int pa_prefill(void* out, const void* query, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
               int32_t num_seqs, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t max_query_len,
               int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype, void* stream);

/*
 * pa_swap_blocks - move whole blocks between two pools (swapping).
 *
 * PagedAttention digest (irregular6612.github.io), section "Method"
 * (scheduling) and its glossary: when memory runs short a preempted
 * request's KV blocks are moved to CPU RAM, and moved back when it resumes;
 * the page "vLLM PagedAttention and continuous batching architecture"
 * (tech.blogsailing.com), section 3, names the same swap space.  For every
 * pair (src, dst) in block_pairs:
 *
 *   dst_k[dst] = src_k[src];  dst_v[dst] = src_v[src]
 *
 * whole blocks (all heads, slots and channels), bit-exact.  Swap-out passes
 * the device caches as src and a host pool as dst; swap-in the reverse.
 * The two pools have the same [*, num_heads, block_size, head_dim] block
 * shape and their own block counts.  Every pool, and block_pairs (int64
 * [num_pairs, 2]), must be device memory or pinned, mapped host memory
 * (hipHostMalloc; torch's pin_memory=True): pageable host memory is
 * rejected with PA_ERR_INVALID before anything is enqueued, as are
 * pointers the HIP runtime does not know.  The pools must be 16-byte
 * aligned.  Destinations must be distinct (and, within one pool, disjoint
 * from the sources); a pair with an id outside its pool is skipped by the
 * kernel.  One kernel launch on `stream` moves every pair (the host-side
 * loads or stores cross the host link); ownership and errors otherwise as
 * for pa_copy_blocks.
 */
int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int64_t* block_pairs,
                   int32_t num_pairs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                   int64_t src_num_blocks, int64_t dst_num_blocks, int32_t dtype, void* stream);

/* Human-readable name of a pa_status value (static storage; never NULL). */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
