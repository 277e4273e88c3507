/*
 * pkv_block_manager.h -- host-side KV block manager of libpkv.so (C ABI).
 *
 * The bookkeeping that feeds the kernels of pkv.h: which physical block holds which
 * tokens of which sequence. It produces block-table rows, the slot of every new token
 * (pkv_reshape_and_cache), copy-on-write pairs (pkv_copy_blocks) and swap pairs
 * (pkv_swap_blocks). It touches no GPU memory and makes no HIP call.
 *
 * What it does follows the pages:
 * - a global pool of fixed-size physical blocks with a free list; blocks are handed out
 *   on demand and taken back when a sequence ends ("vLLM推理引擎PagedAttention原理与性能优化
 *   实战", §2.2 and §四; "vLLM 推理优化技术深度调研报告", 维度一.4);
 * - a new block is taken only when the sequence's current block is full ("vLLM 是什么…", §二);
 * - forked sequences (beams) share blocks, counted by reference; a shared block is read-only
 *   and the first write into it takes a fresh block and records a (src, dst) copy; the last
 *   holder writes in place ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.2);
 * - under memory pressure a sequence's blocks move to a host pool and back (swap; "vLLM 是
 *   什么…", §五 误解三; the scheduler reclaims preempted requests' blocks, same page as above §四);
 * - prefix caching, which the pages recommend turning on in production (same page, §5.1):
 *   a full block is known by its tokens and everything before them; a new sequence whose
 *   prompt starts with known full blocks shares them instead of recomputing them. Blocks of
 *   ended sequences stay known until their memory is needed (least recently freed first).
 *
 * Conventions: every pointer here is a HOST pointer. Sequence ids are caller-chosen int64.
 * A call that fails returns a negative status (pkv.h's codes and the three below) and leaves
 * the manager unchanged. A manager is not thread-safe: one thread at a time.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ERR_NO_BLOCKS (-8)   /* not enough free blocks (GPU or host pool) */
#define PKV_ERR_SEQ (-9)         /* unknown sequence id, id already in use, or the sequence is in the wrong place */
#define PKV_ERR_CAPACITY (-10)   /* an output array is too small */

typedef struct pkv_block_manager pkv_block_manager;

/*
 * A manager of num_gpu_blocks GPU blocks (ids 0 .. num_gpu_blocks - 1) and num_host_blocks
 * host blocks (0 = no swapping), block_size tokens each. Free blocks are handed out lowest id
 * first, freed ones are queued at the back. enable_prefix_caching: 0 or 1.
 */
int pkv_bm_create(int num_gpu_blocks, int num_host_blocks, int block_size, int enable_prefix_caching,
                  pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/*
 * A new sequence seq_id with a prompt of num_tokens tokens (token ids in tokens; may be NULL
 * when prefix caching is off), blocks taken for all of them. slots_out[num_tokens] receives
 * every prompt token's slot (block * block_size + offset). With prefix caching, leading full
 * blocks whose content is known are shared; *num_cached_tokens (may be NULL) receives how
 * many leading tokens' K/V are therefore already in the cache: a multiple of block_size,
 * always less than num_tokens (a prompt known to its last token still recomputes its last
 * block, whose K/V the caller writes). num_tokens >= 0.
 */
int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int num_tokens,
                        int64_t* slots_out, int* num_cached_tokens);

/*
 * Room for n more tokens of seq_id (on the GPU). slots_out[n] receives their slots. When the
 * sequence's partial last block is shared, a fresh block replaces it and the pair
 * (old, fresh) is written to cow_pairs[2 * k], [2 * k + 1] (cow_cap pairs of room); *num_cow
 * receives the count (at most 1 per call). tokens (may be NULL) are the new tokens' ids,
 * used to make blocks they fill known to the prefix cache.
 */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int n, int64_t* slots_out,
                  int64_t* cow_pairs, int cow_cap, int* num_cow);

/*
 * One decode step's appends in one call: one new token for each of the n sequences in
 * seq_ids (distinct, all on the GPU), in order; as n calls of pkv_bm_append with one token
 * each. tokens (may be NULL) holds one token id per sequence. slots_out[n] receives the
 * slots; copy-on-write pairs go to cow_pairs (cow_cap pairs of room), their count to *num_cow.
 */
int pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seq_ids, int n, const int32_t* tokens,
                        int64_t* slots_out, int64_t* cow_pairs, int cow_cap, int* num_cow);

/*
 * pkv_bm_append_batch for pkv_decode_step's fused copy-on-write: the same appends, with
 * sequence i's copy-on-write source in cow_src_out[i] (int32; the pair's `old` block, whose
 * copy is the block its new token lands in; -1 when it needs no copy) in place of a pair list.
 */
int pkv_bm_append_step(pkv_block_manager* bm, const int64_t* seq_ids, int n, const int32_t* tokens,
                       int64_t* slots_out, int32_t* cow_src_out);

/* child_id shares every block of parent_id (which must be on the GPU). */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Ends seq_id (on the GPU or swapped out): its blocks go back or, known to the prefix cache, wait to be reused. */
int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id);

/*
 * Block-table rows and context lengths of n sequences (all on the GPU): tables[n][max_blocks]
 * int32, padded with pad_block; context_lens[n] int32 (may be NULL).
 */
int pkv_bm_block_tables(pkv_block_manager* bm, const int64_t* seq_ids, int n, int32_t* tables, int max_blocks,
                        int32_t pad_block, int32_t* context_lens);

/*
 * Moves seq_id's blocks to the host pool: pairs[2 * k] = GPU block, [2 * k + 1] = host block
 * for each of its blocks, in logical order (cap pairs of room); *num_pairs receives the
 * count. Run pkv_swap_blocks with these pairs before the GPU blocks are reused. A block the
 * sequence shares with others gets its own host copy.
 */
int pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int64_t* pairs, int cap, int* num_pairs);

/* Brings a swapped-out seq_id back into fresh GPU blocks: pairs (host block, GPU block), as above. */
int pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int64_t* pairs, int cap, int* num_pairs);

/*
 * Counts: free GPU blocks (not counting known blocks waiting for reuse), known blocks
 * waiting for reuse, free host blocks. Any pointer may be NULL.
 */
int pkv_bm_num_free(const pkv_block_manager* bm, int* gpu_free, int* gpu_cached, int* host_free);

/* Holders of GPU block `block` (0 when free or only known to the cache). */
int pkv_bm_refcount(const pkv_block_manager* bm, int block, int* count);

/* Tokens and GPU blocks of seq_id; *on_gpu = 0 while it is swapped out. Any output may be NULL. */
int pkv_bm_sequence_info(const pkv_block_manager* bm, int64_t seq_id, int* num_tokens, int* num_blocks, int* on_gpu);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
