// The decode read pattern alone, a measurement aid (gather_probe.hip, pkv_gather_probe).
#pragma once

#include "pkv_launch.h"

namespace pkv {

// The decode read pattern alone (gather_probe.hip): each wavefront reads up to kProbeChunk
// 16-token tiles of one (sequence, kv head) and XORs what it read into sink[s * Hkv + g].
constexpr int kProbeChunk = 32;
struct ProbeArgs {
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint32_t* sink;
  int64_t num_blocks;
  int num_seqs, num_kv_heads, max_blocks, block_shift;
  int num_chunks;   // ceil(max tiles of a context / kProbeChunk)
};
hipError_t launch_gather_probe(const ProbeArgs& a, int tile_bytes, hipStream_t s);

}  // namespace pkv
