// The decode read pattern alone, a measurement aid (gather_probe.hip, pkv_gather_probe).
#pragma once

#include "pkv_launch.h"

namespace pkv {

// The decode read pattern alone (gather_probe.hip): each wavefront reads up to `chunk`
// 16-token tiles of one (sequence, kv head) and XORs what it read into sink[s * Hkv + g].
// The host takes 32-tile chunks unless that leaves fewer than kProbeMinWaves wavefronts,
// then the largest of 16, 8 and 4 that gives that many (4 at the least): a small batch
// read in 32-tile chunks leaves most of the chip idle and would understate its ceiling.
constexpr int kProbeChunkMax = 32;
constexpr int kProbeChunkMin = 4;
constexpr long long kProbeMinWaves = 4096;
struct ProbeArgs {
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint32_t* sink;
  int64_t num_blocks;
  int num_seqs, num_kv_heads, max_blocks, block_shift;
  int chunk;        // tiles per wavefront, kProbeChunkMin .. kProbeChunkMax
  int num_chunks;   // ceil(max tiles of a context / chunk)
};
hipError_t launch_gather_probe(const ProbeArgs& a, int tile_bytes, hipStream_t s);

}  // namespace pkv
