/*
 * pkv.h -- paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.so. Three operations, all enqueued asynchronously on the caller's
 * HIP stream:
 *
 *   pkv_paged_attention_decode  one decode step of attention over a paged KV cache
 *   pkv_reshape_and_cache       write each new token's K/V row into its cache slot
 *   pkv_copy_blocks             copy-on-write copies of whole KV blocks
 *   pkv_decode_step             cache write + attention of one decode step, one launch
 *   pkv_decode_step_no_alloc    the same step without a workspace, for callers that cannot allocate
 *   pkv_paged_attention_prefill causal attention of prefill chunks over the paged cache
 *   pkv_swap_blocks             move whole blocks between a GPU pool and a pinned host pool
 *   pkv_gather_probe            measurement aid: the decode read pattern with no arithmetic
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *_cache, q, out, key, value, block_tables, context_lens,
 *   query_start_loc, slot_mapping, src_dst_pairs, workspace and sink are DEVICE pointers; every other
 *   pointer is a host pointer. All tensors are dense, row-major, in the shapes
 *   given below, and 16-byte aligned.
 * - The caller allocates and owns every buffer, including the workspace. The
 *   library allocates no device memory and keeps no pointer after a call returns;
 *   its one device buffer is the fixed scratch array of pkv_decode_step_no_alloc,
 *   part of its device image. Buffers must stay alive until the stream has passed
 *   the enqueued work.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 * - Arguments are checked on the host before anything is enqueued; a violation
 *   returns a negative pkv_status and enqueues nothing. No call aborts or throws.
 *   PKV_ERR_HIP means the HIP runtime refused a launch.
 * - Values inside device buffers (block ids, slots, context lengths) cannot be
 *   checked on the host. The kernels never touch memory outside the buffers for any
 *   such value: an out-of-range block id is read as zeros, an out-of-range slot or
 *   copy pair is skipped, a context length is clamped to the block-table row.
 *   The results of a sequence that hits one of these cases are unspecified.
 *   pkv_validate_inputs (pkv_validate.h) checks these values, for debugging.
 * - Calls are reentrant. The only global state is the per-GPU address of that scratch
 *   array, looked up once; calls of pkv_decode_step_no_alloc that overlap in time on one
 *   GPU share the array itself.
 *
 * Cache layout (chosen for gfx950): k_cache and v_cache are separate tensors of
 * shape [num_blocks, num_kv_heads, block_size, head_dim] with block_size 16 (the
 * default of the pages), 32 or 64, so one kv head's slice of one block is a contiguous
 * run of 16-token tiles that a wavefront reads with 16-byte loads. A slot is the flat
 * index block * block_size + offset. ("vLLM 推理优化技术深度调研报告", 维度四.5 weighs
 * bigger blocks; on MI355X 16 is both the fastest and the least wasteful.)
 *
 * The method follows the pages on PagedAttention: the KV cache is cut into blocks
 * of 16 token slots, placed anywhere in a shared pool and found through a
 * per-sequence block table ("vLLM推理引擎PagedAttention原理与性能优化实战", §2.2;
 * "vLLM 是什么…", §二); attention itself is the standard Softmax(Q K^T / sqrt(d)) V
 * over the gathered K and V ("vLLM 推理优化技术深度调研报告", 维度一.1 误解二 and
 * 维度一.3 公式 3-4).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: pkv_decode_step and pkv_decode_step_no_alloc take cow_src.
 * 3: pkv_validate_inputs and pkv_validate_inputs_host take cow_src (pkv_validate.h).
 * 4: pkv_decode_partition_tokens takes num_q_heads. */
#define PKV_API_VERSION 4

/* Element types. */
typedef enum pkv_dtype {
  PKV_F16 = 1,       /* IEEE binary16 */
  PKV_BF16 = 2,      /* bfloat16 */
  PKV_FP8_E4M3 = 3   /* OCP E4M3FN codes (cache only), read as code value * per-tensor fp32 scale */
} pkv_dtype;

/* Status codes: 0 on success, negative on error. */
typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,         /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,        /* a size is out of range or sizes disagree */
  PKV_ERR_DTYPE = -3,        /* unknown dtype, or a dtype combination that is not allowed */
  PKV_ERR_UNSUPPORTED = -4,  /* valid request outside what the kernels implement (e.g. head_dim) */
  PKV_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
  PKV_ERR_ALIGN = -6,        /* a device pointer or stride breaks 16-byte alignment */
  PKV_ERR_HIP = -7           /* the HIP runtime reported an error at launch */
} pkv_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* pkv_status_string(int status);

/* PKV_API_VERSION of the library. */
int pkv_api_version(void);

/*
 * Context-partition length, in tokens, that pkv_paged_attention_decode (and
 * pkv_decode_step) will use for these sizes. partition_size > 0 is validated and returned
 * as is (it must be a multiple of 16); 0 asks the library to choose. It aims at 1024
 * (sequence, kv head, partition) work items for grouped query heads (num_q_heads >
 * num_kv_heads, the matrix-core kernel) and at 2048 for one query head per kv head (the
 * vector-ALU kernel): one partition per sequence when num_seqs * num_kv_heads reaches
 * that, otherwise the shortest multiple of 64 tokens that gives at most about that many
 * items (the whole context when that is longer). Returns a negative pkv_status on bad
 * input.
 */
int pkv_decode_partition_tokens(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len,
                                int partition_size);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for these sizes (0 when
 * every sequence fits one partition). The workspace holds fp32 partial results
 * [num_seqs, num_q_heads, num_partitions, head_dim + 2]. Returns 0 on bad input.
 */
size_t pkv_paged_attention_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                          int max_context_len, int partition_size);

/*
 * Decode-step attention over a paged KV cache. A sequence's K and V live in fixed-size
 * blocks found through its block table, logical position t in block t / block_size at
 * offset t % block_size ("vLLM推理引擎PagedAttention原理与性能优化实战", §2.2;
 * "vLLM 推理优化技术深度调研报告", 维度一.3 公式 3, whose body is lost: this is the plain
 * O(1) reading). Attention over the gathered K and V is ordinary softmax attention,
 * equal to attention over the contiguous sequence ("vLLM 推理优化技术深度调研报告",
 * 维度一.1 误解二 and 维度一.3 公式 4). The pages never mention grouped query heads;
 * query heads map onto kv heads in consecutive groups.
 *
 * For every sequence s and query head h (kv head g = h / (num_q_heads / num_kv_heads)):
 *   K_s[t] = k_cache[block_tables[s][t / 16], g, t % 16, :]  for t < context_lens[s]
 *   (V_s likewise; an fp8 cache is read as code value * k_scale / v_scale)
 *   out[s, h, :] = softmax(scale * K_s q[s, h]) V_s
 * accumulated in fp32 and rounded (nearest even) to q's dtype. A sequence with
 * context length 0 gets zeros. context_lens counts the newest token, so the caller
 * runs pkv_reshape_and_cache for it first.
 *
 *   out            [num_seqs, num_q_heads, head_dim]          q_dtype (written)
 *   q              [num_seqs, num_q_heads, head_dim]          q_dtype; sequence stride
 *                  q_seq_stride elements (0 = num_q_heads * head_dim)
 *   k_cache/v_cache[num_blocks, num_kv_heads, block_size, head_dim]   kv_dtype
 *   block_tables   [num_seqs, max_blocks_per_seq] int32       physical block ids
 *   context_lens   [num_seqs] int32                            tokens to attend, <= max_context_len
 *   q_dtype        PKV_F16 or PKV_BF16
 *   kv_dtype       q_dtype, or PKV_FP8_E4M3
 *   scale          logit scale (1/sqrt(head_dim) for standard attention)
 *   k_scale/v_scale fp8 cache scales (ignored for 16-bit caches)
 *   max_context_len upper bound of context_lens; sets the grid (host-side hint)
 *   partition_size tokens per context partition, multiple of 16, or 0 (see
 *                  pkv_decode_partition_tokens); more than one partition per
 *                  sequence runs a second, merging kernel
 *   workspace      device buffer of pkv_paged_attention_workspace_size() bytes
 *                  (may be NULL when that size is 0)
 *
 * Supported: head_dim 64 or 128; num_q_heads a multiple of num_kv_heads with group
 * size 1..16; block_size 16, 32 or 64. Group size 1 runs on the vector ALUs, larger
 * groups on the matrix cores.
 */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                               int64_t num_blocks, int max_blocks_per_seq, int max_context_len,
                               int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                               int64_t q_seq_stride, int partition_size,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * One whole decode step in one launch: the cache write of every sequence's new token
 * followed by attention over the paged cache that now includes it. The results (caches
 * and out) are those of
 *   pkv_reshape_and_cache(key, value, slot_mapping, k_cache, v_cache, num_tokens = num_seqs, ...)
 *   pkv_paged_attention_decode(out, q, k_cache, v_cache, ...)
 * on the same stream, bit for bit. The work item that attends over a sequence's last
 * position writes that sequence's new token first (the pages' memory flow: a new token's
 * KV is registered in its block, then attention reads the blocks; "vLLM 推理优化技术深度
 * 调研报告", 维度一.2).
 *
 *   key/value      [num_seqs, num_kv_heads, head_dim] q_dtype: the new token of each
 *                  sequence; token strides key_stride / value_stride elements (0 = dense)
 *   slot_mapping   [num_seqs] int64: slot of sequence s's new token, which must be the slot
 *                  of its logical position context_lens[s] - 1 in its own (unshared)
 *                  blocks; a negative slot is skipped
 *   cow_src        [num_seqs] int32 or NULL: copy-on-write ("vLLM推理引擎PagedAttention原理
 *                  与性能优化实战", §3.2: the first write into a block that several
 *                  sequences share goes to a private copy). cow_src[s] >= 0 makes the block
 *                  that holds sequence s's last position (its block-table entry, private to
 *                  s) a copy of block cow_src[s], for this cache's K and V, before s's new
 *                  token is written into it: the results are those of
 *                  pkv_copy_blocks(pairs (cow_src[s], that block)) followed by the two calls
 *                  above, bit for bit. -1 (or an id outside the pool) copies nothing. No
 *                  other sequence may read the destination block in the same step, and
 *                  another sequence's new token may land in the source only in the row of
 *                  s's own new token (the one row the copy does not take; beams that share
 *                  a partial block hold the same tokens in it, so theirs share that row).
 *   k_cache/v_cache written (copies, new tokens converted as pkv_reshape_and_cache does, fp8
 *                  with k_scale / v_scale) and read
 * Every other argument is as for pkv_paged_attention_decode, whose checks also apply.
 * Returns PKV_ERR_ALIGN for a cow_src that is not 4-byte aligned.
 */
int pkv_decode_step(void* out, const void* q, void* k_cache, void* v_cache,
                    const void* key, const void* value, const int64_t* slot_mapping, const int32_t* cow_src,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                    int64_t num_blocks, int max_blocks_per_seq, int max_context_len,
                    int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                    int64_t q_seq_stride, int64_t key_stride, int64_t value_stride, int partition_size,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device scratch array that pkv_decode_step_no_alloc uses in place of a
 * workspace: one array per GPU, held from the library's load on that GPU until the process
 * ends. */
#define PKV_NO_ALLOC_SCRATCH_BYTES (32u << 20)

/*
 * pkv_decode_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, checks
 * and results as pkv_decode_step, without the workspace: the split-context partials
 * [num_seqs, num_q_heads, num_partitions, head_dim + 2] fp32 go to a scratch array inside
 * the library (PKV_NO_ALLOC_SCRATCH_BYTES on each GPU). The call allocates and frees
 * nothing; its first call on a GPU looks up the address of that GPU's array.
 *
 * Returns PKV_ERR_WORKSPACE, before any launch, when the partials would need more than
 * PKV_NO_ALLOC_SCRATCH_BYTES (pkv_paged_attention_workspace_size gives their size; the
 * library's own choice of partitions, partition_size = 0, needs at most about 17 MiB).
 * The array keeps whatever the last call left in it; every call writes the partials it
 * reads, so nothing needs clearing.
 *
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or unordered calls from several threads) race and give unspecified
 * outputs. Calls ordered on one stream are safe. The work runs on the device of `stream`
 * (the current device for NULL).
 */
int pkv_decode_step_no_alloc(void* out, const void* q, void* k_cache, void* v_cache,
                             const void* key, const void* value, const int64_t* slot_mapping, const int32_t* cow_src,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             int64_t num_blocks, int max_blocks_per_seq, int max_context_len,
                             int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                             int64_t q_seq_stride, int64_t key_stride, int64_t value_stride, int partition_size,
                             void* stream);

/*
 * Attention of prefill chunks over a paged KV cache. Long prompts are cut into chunks
 * that run between decode steps ("vLLM推理引擎PagedAttention原理与性能优化实战", §六);
 * the pages give no formula for a chunk, and this library takes the plain reading: a
 * chunk of n_s new tokens is the last n_s positions of sequence s's context, its K/V are
 * already in the cache (the caller runs pkv_reshape_and_cache for the chunk's
 * num_tokens rows first), and new token i, at position p = context_lens[s] - n_s + i,
 * attends causally to positions 0 .. p:
 *   out[r, h, :] = softmax(scale * K_s[0..p] q[r, h]) V_s[0..p],   r = query_start_loc[s] + i
 * with K_s, V_s and the kv head of h as for pkv_paged_attention_decode, accumulated in
 * fp32 and rounded (nearest even) to q's dtype. With n_s = 1 for every sequence this is
 * a decode step.
 *
 *   out            [num_tokens, num_q_heads, head_dim]        q_dtype, dense (written)
 *   q              [num_tokens, num_q_heads, head_dim]        q_dtype; token stride
 *                  q_token_stride elements (0 = num_q_heads * head_dim)
 *   query_start_loc[num_seqs + 1] int32: sequence s owns rows [qsl[s], qsl[s+1]) of q
 *                  and out; non-decreasing, qsl[num_seqs] <= num_tokens
 *   context_lens   [num_seqs] int32: context length after the chunk (chunk included),
 *                  at least n_s and at most max_blocks_per_seq * block_size
 *   max_query_len  upper bound of every n_s (host-side hint; sets the grid)
 *   scale          logit scale, finite and > 0
 * Every other argument is as for pkv_paged_attention_decode. No workspace is needed.
 *
 * Rows outside every sequence's range are not written. A sequence whose offsets fall
 * outside [0, num_tokens] is skipped; a chunk longer than max_query_len or than its
 * context is cut to the shorter, and only its first rows are written.
 * Supported: head_dim 64 or 128; any group size; block_size 16, 32 or 64; matrix cores
 * throughout.
 */
int pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_start_loc,
                                int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int64_t num_blocks, int max_blocks_per_seq, int max_query_len,
                                int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                                int64_t q_token_stride, void* stream);

/*
 * Write the K and V rows of num_tokens new tokens into their cache slots
 * ("vLLM 是什么…", §二: a token goes into the current block, a new block is taken only
 * when that one is full; the slot numbers come from the caller's block manager).
 *
 *   key/value      [num_tokens, num_kv_heads, head_dim] in_dtype; token strides
 *                  key_stride / value_stride elements (0 = num_kv_heads * head_dim)
 *   slot_mapping   [num_tokens] int64; slot = block * block_size + offset; a negative slot is skipped
 *   k_cache/v_cache[num_blocks, num_kv_heads, block_size, head_dim] kv_dtype (one layer)
 *   in_dtype       PKV_F16 or PKV_BF16
 *   kv_dtype       in_dtype (the row is copied bit for bit) or PKV_FP8_E4M3, where every
 *                  element is stored as E4M3FN(fl32(x / scale)): IEEE fp32 division,
 *                  round to nearest even, saturating to +-448, NaN kept
 *                  ("vLLM推理引擎PagedAttention原理与性能优化实战", §5.2 names FP8 caches;
 *                  the format and rounding are this library's reading)
 *   k_scale/v_scale fp8 scales, finite and > 0 (ignored for 16-bit caches)
 *
 * Two tokens mapped to one slot in one call is a caller error (the winner is unspecified).
 */
int pkv_reshape_and_cache(const void* key, const void* value, const int64_t* slot_mapping,
                          void* k_cache, void* v_cache,
                          int num_tokens, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                          int in_dtype, int kv_dtype, float k_scale, float v_scale,
                          int64_t key_stride, int64_t value_stride, void* stream);

/*
 * Copy-on-write block copies ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.2:
 * a block shared by several sequences is read-only; the first write into it takes a
 * fresh block and copies the old contents there). For every pair (src, dst) and every
 * layer l: k_caches[l][dst] = k_caches[l][src] and v_caches[l][dst] = v_caches[l][src],
 * whole blocks, byte for byte.
 *
 *   k_caches/v_caches host arrays of num_layers device pointers, each a cache of
 *                  num_blocks blocks of block_bytes bytes
 *   src_dst_pairs  device [num_pairs, 2] int64
 *   block_bytes    bytes of one block of one layer's K (= V) cache:
 *                  num_kv_heads * block_size * head_dim * element size; a multiple of 16
 *
 * Every dst must be distinct and must not be a src in the same call (a copy goes to a
 * freshly taken block); num_pairs = 0 is a no-op.
 */
int pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int num_layers,
                    const int64_t* src_dst_pairs, int num_pairs, int64_t block_bytes, int64_t num_blocks,
                    void* stream);

/*
 * Swapping blocks between the GPU pool and host memory ("vLLM 是什么…", §五 误解三: when
 * physical memory runs out, blocks are moved to CPU memory; the scheduler reclaims the
 * blocks of preempted requests, "vLLM推理引擎PagedAttention原理与性能优化实战", §四). For
 * every pair (src, dst) and every layer l:
 *   dst_k_caches[l][dst] = src_k_caches[l][src] and dst_v_caches[l][dst] = src_v_caches[l][src],
 * whole blocks, byte for byte. Swapping out: the sources are GPU pools and the
 * destinations host pools; swapping in: the other way round. The copy runs as one kernel
 * whose loads and stores cross the host link directly, so scattered blocks cost no more
 * than contiguous ones.
 *
 *   src_*_caches / dst_*_caches host arrays of num_layers pointers, each a pool of
 *                  num_src_blocks / num_dst_blocks blocks of block_bytes bytes. Every pool
 *                  must be addressable by the GPU: device memory, or host memory allocated
 *                  pinned through the HIP runtime (hipHostMalloc; torch pin_memory=True),
 *                  which is mapped for the device at the same address. Memory pinned after
 *                  the fact by registration is not supported.
 *   src_dst_pairs  [num_pairs, 2] int64 (src block, dst block), GPU-addressable (device or
 *                  pinned host memory); a pair with an id out of range is skipped
 *   block_bytes    bytes of one block of one layer's K (= V) pool; a multiple of 16
 *
 * Every dst must be distinct. The source and destination pools are different
 * allocations (blocks within one pool are copied with pkv_copy_blocks). Host pools are
 * read or written by the GPU until the stream passes the call. num_pairs = 0 is a no-op.
 */
int pkv_swap_blocks(const void* const* src_k_caches, const void* const* src_v_caches, void* const* dst_k_caches,
                    void* const* dst_v_caches, int num_layers, const int64_t* src_dst_pairs, int num_pairs,
                    int64_t block_bytes, int64_t num_src_blocks, int64_t num_dst_blocks, void* stream);

/*
 * Measurement aid, not part of the attention path. Decode attention is bound by reading the
 * cache ("vLLM 推理优化技术深度调研报告", 维度一.3 公式5), and what it can reach is set by
 * the gather of 16-token tiles through the block tables ("vLLM推理引擎PagedAttention原理与
 * 性能优化实战", §2.2). This call reads exactly the bytes a decode step over the same batch
 * reads: for every sequence s and kv head g, the K and V bytes of g in the 16-token tiles
 * that hold tokens 0 .. context_lens[s] - 1 (whole tiles), found through block_tables as
 * pkv_paged_attention_decode finds them, with the decode kernels' loads. It computes
 * nothing but the XOR of every 32-bit word it reads, which it XORs into sink[s *
 * num_kv_heads + g]; its rate is the ceiling of this access pattern on the device. Each
 * wavefront reads a run of up to 32 tiles of one (sequence, kv head); runs are shortened
 * (to 16, 8 or 4 tiles) when a small batch would otherwise give the device fewer than
 * 4096 wavefronts.
 *
 *   k_cache, v_cache, block_tables, context_lens, num_seqs, num_kv_heads, head_dim,
 *   block_size, num_blocks, max_blocks_per_seq, max_context_len, kv_dtype
 *                  as for pkv_paged_attention_decode (max_context_len: the largest
 *                  context_lens entry; longer contexts are read only up to it)
 *   sink           [num_seqs, num_kv_heads] uint32, device, 4-byte aligned; XORed into,
 *                  so zero it first for the XOR of this call alone
 *
 * Block ids outside the pool read as zeros (they contribute nothing to the XOR).
 */
int pkv_gather_probe(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, int num_seqs, int num_kv_heads, int head_dim, int block_size,
                     int64_t num_blocks, int max_blocks_per_seq, int max_context_len, int kv_dtype, uint32_t* sink,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
