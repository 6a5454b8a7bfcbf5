/*
 * pa_block_manager.h - host-side KV-cache block manager of libpa (C ABI).
 *
 * The bookkeeping that decides where every token's K/V row lives, so that a
 * serving loop can drive pa_reshape_and_cache / pa_prefill / pa_decode /
 * pa_copy_blocks / pa_swap_blocks without keeping its own tables.  From the
 * pages:
 *  - PagedAttention digest (irregular6612.github.io), "Method", core
 *    components: the block manager keeps the free list of physical blocks,
 *    per-block reference counts and the copy-on-write trigger; blocks are
 *    taken only as tokens arrive; its flowchart: two sequences share a
 *    physical block and a write to it copies the block first;
 *  - "vLLM PagedAttention and continuous batching architecture"
 *    (tech.blogsailing.com), sections 2 and 4: forked samples share the
 *    prompt's blocks by reference count; a sequence of n tokens holds
 *    ceil(n / B) blocks; finished sequences return their blocks;
 *  - "KV cache and PagedAttention" (allinfo.ai.kr), key insights: with
 *    prefix caching, requests sharing a prefix point at the same physical
 *    blocks and skip that part of the prefill;
 *  - the digest's scheduling and glossary: a preempted request's blocks are
 *    swapped to CPU RAM and back.
 *
 * Policies where the pages are silent:
 *  - the free list is first-in first-out, starting from a given order;
 *  - an append first checks that every block it needs is available (new
 *    blocks, plus one private copy when the partly filled last block is
 *    shared) and changes nothing when it is not (PA_ERR_OUT_OF_BLOCKS);
 *  - prefix caching identifies a full block by the whole token prefix up to
 *    its end; the first full block with a given prefix is the cached one; a
 *    new sequence takes over the cached blocks of its prompt's longest
 *    cached prefix of whole blocks, always leaving >= 1 token to compute;
 *    cached blocks whose count drops to zero stay cached and evictable;
 *    allocation takes plain free blocks first, then evicts the least
 *    recently released cached block;
 *  - freeing releases a sequence's blocks from first to last;
 *  - swap-out moves every block of a sequence to a host manager (pairs in
 *    table order) and releases them; swap-in is the reverse onto freshly
 *    allocated blocks (a swapped-in sequence owns private blocks).
 *
 * Slots: token t of a sequence lives at slot table[t / B] * B + t % B.
 * Copy pairs and swap pairs are (src, dst) int64 pairs, ready for
 * pa_copy_blocks / pa_swap_blocks.  All arrays here are host memory.
 * A manager is not thread-safe: one caller at a time.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;

/* New manager of num_blocks blocks of block_size tokens.  free_order: NULL
 * (0, 1, 2, ...) or a permutation of the block ids, the initial free-list
 * order.  prefix_cache: nonzero to identify and share full blocks by their
 * token prefix (appends then need the token ids).  Returns NULL on invalid
 * arguments (num_blocks outside [1, 2^31), block_size outside [1, 65536],
 * free_order not a permutation). */
pa_bm* pa_bm_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order, int32_t prefix_cache);
void pa_bm_destroy(pa_bm* bm);

/* Register sequence `seq` (any id not in use).  With prefix caching and a
 * prompt (prompt_len tokens), its longest cached whole-block prefix (at
 * most prompt_len - 1 tokens) is taken over: *cached_tokens (may be NULL)
 * receives the number of prompt tokens it covers; the caller appends the
 * rest.  PA_ERR_INVALID if `seq` exists. */
int pa_bm_add_seq(pa_bm* bm, int64_t seq, const int32_t* prompt, int32_t prompt_len, int32_t* cached_tokens);

/* Reserve slots for n new tokens of `seq`: slots (int64 [n]) receives each
 * token's slot; pair (int64 [2]) receives the copy-on-write pair when the
 * partly filled last block was shared (at most one per call), and
 * *num_pairs (0 or 1) says whether it did.  tokens (int32 [n]) are required
 * with prefix caching and ignored otherwise.  PA_ERR_OUT_OF_BLOCKS (nothing
 * changed) when the blocks needed are not available. */
int pa_bm_append(pa_bm* bm, int64_t seq, int32_t n, const int32_t* tokens, int64_t* slots, int64_t* pair,
                 int32_t* num_pairs);

/* One token for each of n_seqs sequences, in order (a decode step):
 * slots int64 [n_seqs]; pairs int64 [n_seqs, 2] receives the copy pairs,
 * *num_pairs their count; tokens int32 [n_seqs] (prefix caching) or NULL.
 * Stops at the first sequence that cannot get its block: returns
 * PA_ERR_OUT_OF_BLOCKS with *done (may be NULL) the number of sequences
 * appended before it. */
int pa_bm_append_batch(pa_bm* bm, const int64_t* seqs, int32_t n_seqs, const int32_t* tokens, int64_t* slots,
                       int64_t* pairs, int32_t* num_pairs, int32_t* done);

/* `child` (a new id) shares every block of `parent` (reference counts + 1). */
int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* Release every block of `seq` and forget it. */
int pa_bm_free_seq(pa_bm* bm, int64_t seq);

/* Swap-out: move `seq` from `bm` to the host manager `host` (same block
 * size): pairs (int64 [capacity, 2]) receives the (device, host) block
 * pairs in table order, *num_pairs their count.  PA_ERR_OUT_OF_BLOCKS when
 * the host manager lacks free blocks, PA_ERR_INVALID when capacity is too
 * small; nothing changes in either case. */
int pa_bm_swap_out(pa_bm* bm, pa_bm* host, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* num_pairs);

/* Swap-in: move `seq` back from `host` onto freshly allocated blocks of
 * `bm`; pairs receives (host, device) pairs.  Errors as for swap-out. */
int pa_bm_swap_in(pa_bm* bm, pa_bm* host, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* num_pairs);

/* Block tables of n_seqs sequences: tables int32 [n_seqs, width] padded
 * with -1, lens int32 [n_seqs] (may be NULL).  PA_ERR_INVALID for an
 * unknown sequence or a table wider than width. */
int pa_bm_block_tables(const pa_bm* bm, const int64_t* seqs, int32_t n_seqs, int32_t width, int32_t* tables,
                       int32_t* lens);

/* Queries: -1 for an unknown sequence or block. */
int64_t pa_bm_num_free(const pa_bm* bm);                           /* plain free + evictable cached */
int64_t pa_bm_seq_len(const pa_bm* bm, int64_t seq);
int32_t pa_bm_num_blocks_held(const pa_bm* bm, int64_t seq);        /* table length */
int32_t pa_bm_blocks_needed(const pa_bm* bm, int64_t seq, int32_t n);
int32_t pa_bm_ref_count(const pa_bm* bm, int32_t block);
int64_t pa_bm_num_cached(const pa_bm* bm);                         /* blocks identified by a prefix */

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
