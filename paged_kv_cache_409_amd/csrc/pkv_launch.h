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
  int64_t num_slots;          // NB * 16
  int num_tokens, num_kv_heads, head_dim;
  float k_scale, v_scale;
};

hipError_t launch_decode_mfma(const DecodeArgs& a, int q_type, int kv_type, int head_dim, hipStream_t s);
hipError_t launch_decode_valu(const DecodeArgs& a, int q_type, int kv_type, int head_dim, hipStream_t s);
hipError_t launch_decode_reduce(const ReduceArgs& a, int q_type, int head_dim, hipStream_t s);
hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, int in_type, int kv_type, hipStream_t s);
hipError_t launch_copy_blocks(void* const* k, void* const* v, int num_layers, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t s);

}  // namespace pkv
