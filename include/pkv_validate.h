/*
 * pkv_validate.h -- debug checks of the values inside the index buffers of libpkv.so.
 *
 * The attention, cache-write and block-copy calls check their arguments on the host, but
 * they cannot see the values inside device buffers: block ids, context lengths, slots and
 * copy pairs. Their kernels stay inside every buffer whatever those values are (an
 * out-of-range block id reads zeros, an out-of-range slot or pair is skipped), but the
 * results of a sequence that hits such a value are unspecified. These calls check the
 * values against what the method assumes of them, for debugging a caller:
 *
 * - a sequence's context is found through its block table: token t of sequence s lies in
 *   physical block block_tables[s][t / block_size] at offset t % block_size, for
 *   t < context_lens[s] ("vLLM推理引擎PagedAttention原理与性能优化实战", §2.2), so every
 *   table entry that holds context must name a block of the pool, and a context cannot be
 *   longer than its table row;
 * - a new token's K/V row is written into one slot of its sequence's current block
 *   ("vLLM 推理优化技术深度调研报告", 维度一.2), one token per slot;
 * - copy-on-write copies a shared block into a freshly taken block before a sequence
 *   writes to it ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.2), so the blocks
 *   written by one pkv_copy_blocks call are distinct and are not read by the same call;
 * - pkv_decode_step writes sequence s's new token into the slot of its last position,
 *   context_lens[s] - 1, in a block that no other sequence of the batch reads (a shared
 *   block is copied first);
 * - with cow_src, pkv_decode_step first makes that block a copy of block cow_src[s] (the
 *   same section's copy-on-write, done inside the step), so the source is a block of the
 *   pool, the sequence has a last block to copy into, and no other sequence reads that
 *   block in the step, neither through its table nor as its own copy's source; the copy
 *   reads its source in the same launch, so another sequence's new token may land there
 *   only in the row of the copying sequence's own new token, which the copy does not take.
 *
 * Both calls are synchronous and meant for debugging, not for the hot path. They allocate
 * host memory only. The result names the first failed check in the order of pkv_check.
 */
#ifndef PKV_VALIDATE_H
#define PKV_VALIDATE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_check {
  PKV_CHECK_OK = 0,
  PKV_CHECK_CONTEXT_LEN = 1,        /* context_lens[s] < 0 or > max_blocks_per_seq * block_size; index = s */
  PKV_CHECK_BLOCK_ID = 2,           /* a table entry that holds context is outside [0, num_blocks);
                                       index = s * max_blocks_per_seq + column */
  PKV_CHECK_SLOT_RANGE = 3,         /* slot_mapping[t] >= num_blocks * block_size; index = t */
  PKV_CHECK_SLOT_DUPLICATE = 4,     /* a slot already taken by an earlier token; index = the later token */
  PKV_CHECK_SLOT_NOT_LAST = 5,      /* decode step: slot of sequence s is not the slot of its position
                                       context_lens[s] - 1; index = s */
  PKV_CHECK_SLOT_SHARED_BLOCK = 6,  /* decode step: the new token's block holds context of another sequence;
                                       index = s, value = the other sequence */
  PKV_CHECK_PAIR_RANGE = 7,         /* a copy pair's src or dst is outside [0, num_blocks); index = pair */
  PKV_CHECK_PAIR_DUPLICATE_DST = 8, /* a dst already written by an earlier pair; index = the later pair */
  PKV_CHECK_PAIR_DST_IS_SRC = 9,    /* a dst that is also the src of another pair; index = the pair writing it */
  PKV_CHECK_COW_RANGE = 10,         /* decode step: cow_src[s] < -1 or >= num_blocks; index = s */
  PKV_CHECK_COW_NO_CONTEXT = 11,    /* decode step: cow_src[s] >= 0 for a sequence with no context (no block
                                       to copy into); index = s, value = cow_src[s] */
  PKV_CHECK_COW_SHARED_DST = 12,    /* decode step: the block that sequence s's copy writes holds context of
                                       another sequence; index = s, value = the other sequence */
  PKV_CHECK_COW_DST_IS_SRC = 13,    /* decode step: the block that sequence s's copy writes is the copy
                                       source of another sequence; index = s, value = the other sequence */
  PKV_CHECK_COW_SRC_WRITTEN = 14    /* decode step: another sequence's new token lands in sequence s's copy
                                       source at a row the copy takes (any row but that of s's own new
                                       token); index = s, value = the other sequence */
} pkv_check;

typedef struct pkv_validation {
  int32_t check;   /* a pkv_check value */
  int32_t reserved;
  int64_t index;   /* where the failed check looked (see pkv_check), -1 when check == 0 */
  int64_t value;   /* the offending value (block id, slot, context length or block), 0 when check == 0 */
} pkv_validation;

/*
 * Checks host copies of the index buffers.
 *
 *   block_tables   [num_seqs, max_blocks_per_seq] int32, or NULL (with context_lens)
 *   context_lens   [num_seqs] int32, or NULL (with block_tables)
 *   slot_mapping   [num_tokens] int64 (negative = no write), or NULL
 *   decode_step    nonzero: slot_mapping is pkv_decode_step's (num_tokens == num_seqs,
 *                  token s belongs to sequence s; needs block_tables and context_lens)
 *   cow_src        [num_seqs] int32 as for pkv_decode_step (-1: no copy), or NULL; needs
 *                  decode_step. A source equal to its destination is a no-op and passes.
 *   src_dst_pairs  [num_pairs, 2] int64 (src, dst) as for pkv_copy_blocks, or NULL
 *   block_size     16, 32 or 64
 *   result         written with the first failed check, or PKV_CHECK_OK
 *
 * Returns PKV_OK when the checks ran (the verdict is in *result), a negative pkv_status
 * when the arguments themselves are inconsistent (NULL result, negative sizes, one of
 * block_tables / context_lens without the other, decode_step without them or with
 * num_tokens != num_seqs: PKV_ERR_NULL or PKV_ERR_SHAPE; cow_src without decode_step:
 * PKV_ERR_SHAPE).
 */
int pkv_validate_inputs_host(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                             int max_blocks_per_seq, int block_size, int64_t num_blocks,
                             const int64_t* slot_mapping, int num_tokens, int decode_step,
                             const int32_t* cow_src, const int64_t* src_dst_pairs, int num_pairs,
                             pkv_validation* result);

/*
 * The same checks on device buffers: copies them to host memory on `stream` (a
 * hipStream_t as void*, NULL = the default stream), waits for the copies, then checks as
 * pkv_validate_inputs_host does. Device pointers: block_tables, context_lens,
 * slot_mapping, cow_src, src_dst_pairs; result is a host pointer. PKV_ERR_HIP when a copy
 * fails.
 */
int pkv_validate_inputs(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                        int max_blocks_per_seq, int block_size, int64_t num_blocks,
                        const int64_t* slot_mapping, int num_tokens, int decode_step,
                        const int32_t* cow_src, const int64_t* src_dst_pairs, int num_pairs, void* stream,
                        pkv_validation* result);

#ifdef __cplusplus
}
#endif

#endif /* PKV_VALIDATE_H */
