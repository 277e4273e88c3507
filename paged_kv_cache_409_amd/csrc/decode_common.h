// Parameters and helpers shared by the paged decode-attention kernels.
#pragma once

#include "pkv_device.h"

namespace pkv {

// One launch of the decode main kernel. Work item = (sequence, kv head, context
// partition); one wavefront per item.
struct DecodeArgs {
  void* out;                      // [S, Hq, D] q dtype (written when num_parts == 1)
  const void* q;                  // [S, Hq, D] q dtype, sequence stride q_seq_stride elements
  const void* k_cache;            // [NB, Hkv, 16, D]
  const void* v_cache;            // [NB, Hkv, 16, D]
  const int32_t* block_tables;    // [S, max_blocks]
  const int32_t* context_lens;    // [S]
  float* part_ml;                 // [S, Hq, num_parts, 2]: running max (log2 units), sum
  float* part_o;                  // [S, Hq, num_parts, D]: unnormalised weighted sums
  int64_t q_seq_stride;
  int64_t num_blocks;
  int num_seqs, num_q_heads, num_kv_heads, group;
  int max_blocks;                 // block-table row length
  int num_parts;                  // partitions per sequence (grid dimension)
  int part_blocks;                // KV blocks per partition
  int num_items;                  // workgroups with work: num_seq_groups * num_kv_heads * num_parts
  int seqs_per_group;             // sequences (one wavefront each) per workgroup; 1 for the VALU kernel
  int num_seq_groups;             // ceil(num_seqs / seqs_per_group)
  int group_mode_ok;              // the workgroup's LDS holds a tile list for sharing groups
  float qk_scale_log2;            // scale * log2(e) (* k_scale for an fp8 cache)
  float v_scale;                  // 1, or v_scale for an fp8 cache
};

// Workgroup -> work item. Workgroups are dealt to the 8 XCDs round-robin; this map
// gives each run of 4 consecutive items (neighbouring sequences, or sequence groups)
// to a single XCD, so blocks they share stay in that XCD's L2. The grid is padded to a
// multiple of 32; ids past num_items do nothing.
__device__ __forceinline__ int item_of_workgroup(int w) {
  const int xcd = w & 7, k = w >> 3;
  return (((k >> 2) << 3) + xcd) * 4 + (k & 3);
}

struct Item {
  int s, g, p;
};

// Items are ordered (kv head, partition, sequence group) with the group fastest; it.s is
// the group's first sequence (groups of one sequence for the VALU kernel).
__device__ __forceinline__ Item decode_item(int j, const DecodeArgs& a) {
  Item it;
  it.s = (j % a.num_seq_groups) * a.seqs_per_group;
  const int r = j / a.num_seq_groups;
  it.p = r % a.num_parts;
  it.g = r / a.num_parts;
  return it;
}

// Orders a wavefront's own LDS writes before its later LDS reads of other lanes' data
// (what a workgroup barrier does for a one-wave workgroup), without involving the
// other wavefronts of the workgroup.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache-policy operand of a buffer load: 0 is the default (allocate in L2), bit 1 is
// "nt" (non-temporal, streaming).
constexpr int kPolicyCached = 0;
constexpr int kPolicyStream = 2;

// 16-byte load of KV cache bytes. A block that only one sequence reads is read once per
// decode step, so its loads are marked non-temporal: they do not displace other lines in
// L2, and on gfx950 a random gather of whole blocks runs about 9% faster this way. Blocks
// that several sequences share keep the default policy so that the other readers hit L2.
template <int POLICY>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, POLICY));
}

// True when block `idx` of sequence s's table is also the block at the same logical
// index of the previous or next sequence in the batch. That is the layout of beams (or
// parallel samples) forked from one prompt: they share its blocks and sit next to each
// other in the batch. idx must be < max_blocks.
__device__ __forceinline__ bool neighbour_shares_block(const DecodeArgs& a, int s, int idx) {
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks + idx;
  const int mine = bt[0];
  bool shared = false;
  if (s > 0) shared = shared || bt[-a.max_blocks] == mine;
  if (s + 1 < a.num_seqs) shared = shared || bt[a.max_blocks] == mine;
  return shared;
}

// Two waves share each SIMD and the older one wins instruction arbitration, so without
// help it runs ahead and finishes long before its neighbour, leaving the memory system
// under-fed at the end of the launch. A wave that streams private blocks therefore
// lowers its issue priority as it works through them (3 in the first quarter ... 0 in
// the last), which lets a lagging wave catch up. (Waves reading shared blocks do better
// in step with each other, so they keep the default priority.)
__device__ __forceinline__ void progress_priority(int done, int total) {
  const int level = ((total - done) * 4 - 1) / total;   // 3 .. 0 while done < total
  if (level >= 3) __builtin_amdgcn_s_setprio(3);
  else if (level == 2) __builtin_amdgcn_s_setprio(2);
  else if (level == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

}  // namespace pkv
