// Launch-side structs and entry points of the kernels (host and device share these).
#pragma once

#include "decode_common.h"

namespace pkv {

struct ReduceArgs {
  void* out;                    // [S, Hq, D] q dtype
  const float* part_ml;         // [S, Hq, num_parts, 2]
  const float* part_o;          // [S, Hq, num_parts, D]
  const int32_t* context_lens;  // [S]
  int num_seqs, num_q_heads, num_parts, part_tokens, max_tokens;
  float v_scale;
};

struct CacheWriteArgs {
  const void* key;            // [T, Hkv, D] in dtype, token stride key_stride elements
  const void* value;
  const int64_t* slot_mapping;
  void* k_cache;              // [NB, Hkv, 16, D]
  void* v_cache;
  int64_t key_stride, value_stride;
  int64_t num_slots;          // NB * block size
  int num_tokens, num_kv_heads, head_dim;
  int block_shift;            // block size = 16 << block_shift
  float k_scale, v_scale;
};

// Workgroups of the matrix-core decode kernel hold up to this many sequences (one
// wavefront each).
constexpr int kMaxSeqsPerGroup = 4;
// Small LDS area of a group-mode workgroup: per-sequence context ends, the new tokens'
// positions and the per-wave (max, sum) of every column for the final merge.
constexpr int kDecodeSmallLds = 2048;
// Largest number of group-mode tile-list entries (sequences x partition blocks) a
// workgroup stages in LDS.
constexpr int kMaxGroupListEntries = 2048;

// Per sequence in a fused step: the LDS copy of its new token (K row then V row, storage
// format, up to 512 bytes) and, at byte kCowSlot (decode_common.h), its copy-on-write block
// and source.
constexpr int kTokenRowsLds = kCowSlot + 16;

// Entries reserved per wavefront for its group-mode tile list: a wave lists every B-th
// logical block of the partition, each with up to B distinct physical blocks, so at most
// B * ceil(part_blocks / B) < part_blocks + kMaxSeqsPerGroup entries.
__host__ __device__ inline int group_list_stride(int part_blocks) { return part_blocks + kMaxSeqsPerGroup; }

// Dynamic LDS bytes of one matrix-core decode workgroup: per-wave K/V tile staging,
// per-wave new-token rows, per-wave block-table slices, and in group mode the small area
// and the per-wave tile lists (ids and packed metadata).
inline size_t mfma_decode_lds_bytes(int head_dim, int seqs_per_group, int part_blocks, bool group_mode) {
  const size_t tile = (size_t)2 * 16 * head_dim * 2;
  return seqs_per_group * (tile + kTokenRowsLds) + (size_t)seqs_per_group * part_blocks * 4 +
         (group_mode ? kDecodeSmallLds + (size_t)2 * seqs_per_group * group_list_stride(part_blocks) * 4 : 0);
}

// One launch of the prefill-chunk kernel. Work item = (kv head, sequence, tile of
// kPrefillRows query rows); the rows of a sequence and kv head are its new tokens x the
// G query heads of the group, token-major.
struct PrefillArgs {
  void* out;                      // [T, Hq, D] q dtype, contiguous
  const void* q;                  // [T, Hq, D] q dtype, token stride q_token_stride elements
  const void* k_cache;            // [NB, Hkv, 16, D]
  const void* v_cache;            // [NB, Hkv, 16, D]
  const int32_t* block_tables;    // [S, max_blocks]
  const int32_t* context_lens;    // [S], after the chunk
  int block_shift;                // a cache block holds 16 << block_shift tokens
  const int32_t* query_start_loc; // [S + 1]
  int64_t q_token_stride;
  int64_t num_blocks;
  int num_seqs, num_tokens, num_q_heads, num_kv_heads, group;
  int max_blocks;                 // block-table row length
  int max_query_len;              // longest chunk the launch covers
  int row_tiles;                  // ceil(max_query_len * group / kPrefillRows)
  int num_items;                  // num_kv_heads * num_seqs * row_tiles
  float qk_scale_log2;            // scale * log2(e) (* k_scale for an fp8 cache)
  float v_scale;                  // 1, or v_scale for an fp8 cache
};

// Prefill workgroup: 4 wavefronts x 32 query rows. The fp8-cache kernel takes keys 64
// (four 16-token tiles) at a time through registers; the 16-bit-cache kernel takes 32 at
// a time straight into LDS.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillCols = 32;
constexpr int kPrefillRows = kPrefillWaves * kPrefillCols;
constexpr int kPrefillKeys = 64;

hipError_t launch_prefill_mfma(const PrefillArgs& a, int q_type, int kv_type, int head_dim, hipStream_t s);   // fp8 cache
hipError_t launch_prefill_lds(const PrefillArgs& a, int q_type, int head_dim, hipStream_t s);                 // 16-bit cache
hipError_t launch_decode_mfma(const DecodeArgs& a, int q_type, int kv_type, int head_dim, hipStream_t s);
hipError_t launch_decode_valu(const DecodeArgs& a, int q_type, int kv_type, int head_dim, hipStream_t s);
hipError_t launch_decode_reduce(const ReduceArgs& a, int q_type, int head_dim, hipStream_t s);
hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, int in_type, int kv_type, hipStream_t s);
// Copy-on-write (src pools = dst pools) and swapping (a GPU pool and a host pool) move whole
// blocks with the same kernel.
hipError_t launch_move_blocks(const void* const* src_k, const void* const* src_v, void* const* dst_k,
                              void* const* dst_v, int num_layers, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_src_blocks, int64_t num_dst_blocks, hipStream_t s);

}  // namespace pkv
