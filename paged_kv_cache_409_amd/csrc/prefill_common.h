// Pieces shared by the two prefill-chunk kernels (register-staged and direct-to-LDS).
// Both files that include this are compiled with -fno-honor-nans (see max_nn below).
#pragma once

#include "pkv_launch.h"

namespace pkv {

template <int QT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// acc + lo + hi of two packed 16-bit values (one v_dot2 against (1, 1)).
template <int QT>
__device__ __forceinline__ float dot2_ones(uint32_t p, float acc) {
  if constexpr (QT == kBF16) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
}

// Position of a named tile in one kv head's view of the pool, in units of one 16-token
// tile (-1 stays -1): block b's tiles of one kv head lie num_kv_heads << shift tiles apart.
// The prefill kernels stage positions rather than names, so that a load's address is the
// staged value times the tile size (a few scalar instructions per load instead of about
// fifteen); the host keeps (num_blocks << shift) * num_kv_heads within an int.
__device__ __forceinline__ int tile_position(int v, int shift, int num_kv_heads) {
  return v < 0 ? -1 : (v >> shift) * (num_kv_heads << shift) + (v & ((1 << shift) - 1));
}

constexpr float kLazyRescale = 8.0f;
constexpr int kIdsRing = 1024;   // block-table entries a workgroup keeps in LDS

// Work items visit sequences longest first: the sequence of rank r in decreasing order of
// work n (2 ctx - n) (new tokens times twice the mean context they attend to; ties by
// index), so the longest items start first and the short ones fill the tail. Every
// workgroup computes the same order; with more than kSortSeqs sequences the order is the
// batch's own. `scratch` is LDS of at least kSortSeqs + 1 ints, free on entry and on return.
constexpr int kSortSeqs = 256;
__device__ __forceinline__ int seq_of_rank(const PrefillArgs& a, int r, int* scratch) {
  const int S = a.num_seqs;
  if (S > kSortSeqs) return r;
  float* work = reinterpret_cast<float*>(scratch);
  for (int t = threadIdx.x; t < S; t += blockDim.x) {
    const int q0 = a.query_start_loc[t], q1 = a.query_start_loc[t + 1];
    const int ctx = min(max(a.context_lens[t], 0), (a.max_blocks * kBlock) << a.block_shift);
    const bool ok = q0 >= 0 && q1 >= q0 && q1 <= a.num_tokens;
    const int n = ok ? min(min(q1 - q0, a.max_query_len), ctx) : 0;
    work[t] = (float)n * (2.0f * (float)ctx - (float)n);   // in float: 2 ctx may exceed int
  }
  __syncthreads();
  for (int t = threadIdx.x; t < S; t += blockDim.x) {
    const float wt = work[t];
    int rank = 0;
    for (int u = 0; u < S; ++u) {
      const float wu = work[u];
      rank += (wu > wt || (wu == wt && u < t)) ? 1 : 0;
    }
    if (rank == r) scratch[kSortSeqs] = t;   // ranks are a permutation: exactly one writer
  }
  __syncthreads();
  const int s = scratch[kSortSeqs];
  __syncthreads();
  return s;
}

// Maxima of scores. The prefill files are compiled with -fno-honor-nans: no score that reaches a
// maximum or an exponent is NaN (stale rows are replaced by -inf through a select on an
// integer condition first), so IEEE max needs no NaN-quieting of operands that come
// straight from the matrix cores, and chains of maxima become v_max3.
__device__ __forceinline__ float max_nn(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float max3_nn(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float max_nn_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_nn_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace pkv
