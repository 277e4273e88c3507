// The decode access pattern without the decode: a measurement aid.
//
// Decode attention is bound by reading the paged cache ("vLLM 推理优化技术深度调研报告",
// 维度一.3 公式5). What a kernel can reach is then set by the access pattern itself:
// 16-token tiles of one kv head (a few KiB each) gathered through block tables from
// blocks scattered over the pool ("vLLM推理引擎PagedAttention原理与性能优化实战", §2.2).
// This kernel reads exactly those bytes with the decode kernels' loads (16-byte buffer
// loads, streaming cache policy, whole rows per instruction) and does nothing with them
// but an XOR, so that its rate is the ceiling of the pattern on the device it runs on;
// the decode rate divided by it says how much of the achievable the decode kernels reach.
// Each wavefront takes up to `chunk` tiles of one (sequence, kv head), so that short and
// long contexts alike give the device thousands of wavefronts.
#include "gather_probe.h"

namespace pkv {

constexpr int kProbeWaves = 4;       // wavefronts per workgroup
constexpr int kProbeInFlight = 2;    // tiles whose loads a wavefront keeps in flight

template <int TB>   // bytes of one kv head's 16-token tile
__global__ __launch_bounds__(kWave * kProbeWaves) void gather_probe_kernel(const ProbeArgs a) {
  constexpr int L = TB / (16 * kWave);   // 16-byte loads per lane per tile, K or V
  static_assert(L >= 1 && TB % (16 * kWave) == 0, "whole rows per load instruction");
  static_assert(kProbeChunkMax <= kWave, "one tile name per lane");
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  // Items (chunk, sequence, kv head), the kv head fastest, as the decode kernels order theirs.
  const long long item = (long long)blockIdx.x * kProbeWaves + w;
  if (item >= (long long)a.num_seqs * a.num_kv_heads * a.num_chunks) return;   // no barrier below
  const int g = (int)(item % a.num_kv_heads);
  const long long rest = item / a.num_kv_heads;
  const int s = (int)(rest % a.num_seqs), c = (int)(rest / a.num_seqs);
  const int shift = a.block_shift;
  const int ctx = min(max(a.context_lens[s], 0), (a.max_blocks * kBlock) << shift);
  const int t0 = c * a.chunk;
  const int cn = min(a.chunk, (ctx + kBlock - 1) / kBlock - t0);   // tiles of this wavefront
  if (cn <= 0) return;
  const int64_t head_stride = (int64_t)TB << shift;
  const int64_t block_stride = (int64_t)a.num_kv_heads * head_stride;
  const uint8_t* kbase = (const uint8_t*)a.k_cache + (int64_t)g * head_stride;
  const uint8_t* vbase = (const uint8_t*)a.v_cache + (int64_t)g * head_stride;
  // lane i holds the name of tile t0 + i
  const int my_name = lane < cn ? tile_name(a.block_tables + (int64_t)s * a.max_blocks, t0 + lane, shift, a.num_blocks) : -1;
  uint32_t acc = 0;
  for (int b0 = 0; b0 < cn; b0 += kProbeInFlight) {
    u32x4 k[kProbeInFlight][L], v[kProbeInFlight][L];
#pragma unroll
    for (int b = 0; b < kProbeInFlight; ++b) {
      const int id = readfirstlane(__shfl(my_name, b0 + b, kWave));   // -1 past cn
      const bool live = id >= 0;
      const int64_t off = live ? tile_offset(id, shift, block_stride, TB) : 0;
      const auto rk = make_rsrc(kbase + off, live ? (uint32_t)TB : 0u);
      const auto rv = make_rsrc(vbase + off, live ? (uint32_t)TB : 0u);
#pragma unroll
      for (int u = 0; u < L; ++u) k[b][u] = buf_load16<kPolicyStream>(rk, (uint32_t)((u * kWave + lane) * 16));
#pragma unroll
      for (int u = 0; u < L; ++u) v[b][u] = buf_load16<kPolicyStream>(rv, (uint32_t)((u * kWave + lane) * 16));
    }
#pragma unroll
    for (int b = 0; b < kProbeInFlight; ++b)
#pragma unroll
      for (int u = 0; u < L; ++u)
        acc ^= k[b][u][0] ^ k[b][u][1] ^ k[b][u][2] ^ k[b][u][3] ^ v[b][u][0] ^ v[b][u][1] ^ v[b][u][2] ^ v[b][u][3];
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, kWave);
  if (lane == 0) atomicXor(a.sink + (int64_t)s * a.num_kv_heads + g, acc);
}

hipError_t launch_gather_probe(const ProbeArgs& a, int tile_bytes, hipStream_t stream) {
  const long long items = (long long)a.num_seqs * a.num_kv_heads * a.num_chunks;
  if (items == 0) return hipSuccess;
  const dim3 grid((unsigned)((items + kProbeWaves - 1) / kProbeWaves));
  switch (tile_bytes) {
    case 4096: hipLaunchKernelGGL((gather_probe_kernel<4096>), grid, dim3(kWave * kProbeWaves), 0, stream, a); break;
    case 2048: hipLaunchKernelGGL((gather_probe_kernel<2048>), grid, dim3(kWave * kProbeWaves), 0, stream, a); break;
    case 1024: hipLaunchKernelGGL((gather_probe_kernel<1024>), grid, dim3(kWave * kProbeWaves), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
