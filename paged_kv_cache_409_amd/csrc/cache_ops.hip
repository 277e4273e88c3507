// Writing new tokens into their cache slots, and copy-on-write block copies.
//
// * A decoded token's K and V rows go into the slot the block manager assigned it
//   (a fresh block is taken only when the current one is full: "vLLM 是什么…", §二).
//   The slot is the flat index block * block_size + offset; a negative slot is skipped.
//   For an fp8 cache each value is quantised on the way in:
//   code = E4M3FN(fl32(x / scale)), round to nearest even, saturating at +-448, NaN
//   kept (the pages only say FP8 halves KV memory, "vLLM推理引擎PagedAttention原理与
//   性能优化实战", §5.2; the format and rounding are this library's reading).
// * Sequences sharing a block see it read-only; the first write into it copies the
//   whole block to a fresh one (same page, §3.2). copy_blocks performs those copies
//   for K and V of every layer given.
#include "pkv_launch.h"

namespace pkv {

// One thread per 8 consecutive elements of one (token, kv head) row.
template <int IT, int KVT>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  const int chunks = a.head_dim / 8;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= (int64_t)a.num_tokens * a.num_kv_heads * chunks) return;
  const int c = (int)(tid % chunks);
  const int h = (int)((tid / chunks) % a.num_kv_heads);
  const int64_t t = tid / ((int64_t)chunks * a.num_kv_heads);
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int P = kBlock << a.block_shift;
  const int64_t blk = slot / P, off = slot % P;
  const int64_t dst = ((blk * a.num_kv_heads + h) * P + off) * a.head_dim + 8 * c;
  const u32x4 kin = *(const u32x4*)((const uint16_t*)a.key + t * a.key_stride + (int64_t)h * a.head_dim + 8 * c);
  const u32x4 vin = *(const u32x4*)((const uint16_t*)a.value + t * a.value_stride + (int64_t)h * a.head_dim + 8 * c);
  store_cache_chunk<IT, KVT>(kin, a.k_cache, dst, a.k_scale);
  store_cache_chunk<IT, KVT>(vin, a.v_cache, dst, a.v_scale);
}

hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, int in_type, int kv_type, hipStream_t stream) {
  const int64_t threads = (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
#define PKV_CASE(IT, KVT)                                                                      \
  if (in_type == IT && kv_type == KVT) {                                                        \
    hipLaunchKernelGGL((reshape_and_cache_kernel<IT, KVT>), grid, dim3(256), 0, stream, a);     \
    return hipGetLastError();                                                                   \
  }
  PKV_CASE(kBF16, kBF16) PKV_CASE(kF16, kF16) PKV_CASE(kBF16, kFP8) PKV_CASE(kF16, kFP8)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

constexpr int kMaxCopyLayers = 64;

// Whole-block moves between two pools (the same pool for copy-on-write; a GPU pool and a
// pinned host pool for swapping). Every pointer is one layer's K or V pool, addressable by
// the GPU: device memory, or host memory pinned and mapped by the HIP runtime.
struct MoveArgs {
  const void* src_k[kMaxCopyLayers];
  const void* src_v[kMaxCopyLayers];
  void* dst_k[kMaxCopyLayers];
  void* dst_v[kMaxCopyLayers];
  const int64_t* pairs;       // [num_pairs, 2] (src block, dst block)
  int64_t block_bytes;        // bytes of one block of one layer's K (or V) pool
  int64_t num_src_blocks, num_dst_blocks;
  int num_pairs;
  int chunk_wgs;              // workgroups per (pair, layer, tensor)
};

// blockIdx.x = pair * chunk_wgs + chunk group, blockIdx.y = layer, blockIdx.z = 0 (K) / 1 (V).
// Each thread moves one 16-byte chunk; a pair with an id out of range is skipped.
__global__ __launch_bounds__(256) void move_blocks_kernel(const MoveArgs a) {
  const int pair = blockIdx.x / a.chunk_wgs;
  const int64_t chunk = (int64_t)(blockIdx.x % a.chunk_wgs) * 256 + threadIdx.x;
  if (chunk * 16 >= a.block_bytes) return;
  const int64_t src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
  if (src < 0 || src >= a.num_src_blocks || dst < 0 || dst >= a.num_dst_blocks) return;
  const uint8_t* from = (const uint8_t*)(blockIdx.z == 0 ? a.src_k[blockIdx.y] : a.src_v[blockIdx.y]);
  uint8_t* to = (uint8_t*)(blockIdx.z == 0 ? a.dst_k[blockIdx.y] : a.dst_v[blockIdx.y]);
  const u32x4 x = *(const u32x4*)(from + src * a.block_bytes + chunk * 16);
  *(u32x4*)(to + dst * a.block_bytes + chunk * 16) = x;
}

hipError_t launch_move_blocks(const void* const* src_k, const void* const* src_v, void* const* dst_k,
                              void* const* dst_v, int num_layers, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_src_blocks, int64_t num_dst_blocks,
                              hipStream_t stream) {
  if (num_pairs == 0 || num_layers == 0) return hipSuccess;
  MoveArgs a;
  a.pairs = pairs;
  a.block_bytes = block_bytes;
  a.num_src_blocks = num_src_blocks;
  a.num_dst_blocks = num_dst_blocks;
  a.num_pairs = num_pairs;
  a.chunk_wgs = (int)((block_bytes / 16 + 255) / 256);
  for (int l0 = 0; l0 < num_layers; l0 += kMaxCopyLayers) {
    const int nl = num_layers - l0 < kMaxCopyLayers ? num_layers - l0 : kMaxCopyLayers;
    for (int l = 0; l < nl; ++l) {
      a.src_k[l] = src_k[l0 + l];
      a.src_v[l] = src_v[l0 + l];
      a.dst_k[l] = dst_k[l0 + l];
      a.dst_v[l] = dst_v[l0 + l];
    }
    hipLaunchKernelGGL(move_blocks_kernel, dim3(num_pairs * a.chunk_wgs, nl, 2), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pkv
