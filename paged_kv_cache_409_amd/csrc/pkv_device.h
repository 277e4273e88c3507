// Device-side types and helpers shared by the paged KV-cache kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element-type tags. kF16/kBF16 are 16-bit floats; kFP8 is OCP E4M3FN.
enum ElemType { kF16 = 1, kBF16 = 2, kFP8 = 3 };

constexpr int kWave = 64;
constexpr int kBlock = 16;            // tokens per KV block
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- 16-bit float <-> fp32 on raw bits -------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <int T>
__device__ __forceinline__ float lo16(uint32_t w) { return T == kBF16 ? bf16_lo(w) : f16_lo(w); }
template <int T>
__device__ __forceinline__ float hi16(uint32_t w) { return T == kBF16 ? bf16_hi(w) : f16_hi(w); }

// Two fp32 -> packed 16-bit (round to nearest even, hardware convert).
template <int T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (T == kBF16) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Four E4M3FN codes (one dword) -> four 16-bit values of type T, exactly: every
// E4M3 value is representable in both bf16 and f16, and the scale is 1.
template <int T>
__device__ __forceinline__ u32x2 fp8x4_to_16(uint32_t w) {
  u32x2 r;
  if constexpr (T == kBF16) {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  } else {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  return r;
}

// OCP E4M3FN encoder, written from the format's definition: bias 7, 3 mantissa bits,
// no infinities, S.1111.111 = NaN, largest finite 448, smallest subnormal 2^-9.
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (ax != ax) return 0x7Fu | sign;                 // NaN
  if (ax >= 448.0f) return 0x7Eu | sign;             // saturate (infinities too)
  if (ax < 0.015625f) {                              // below 2^-6: multiples of 2^-9
    return (uint32_t)__builtin_rintf(ax * 512.0f) | sign;   // exact scaling, then RNE
  }
  const uint32_t ab = __float_as_uint(ax);
  const uint32_t r = ab + 0x7FFFFu + ((ab >> 20) & 1u);     // RNE at the 3rd mantissa bit
  const uint32_t e = (r >> 23) - 127u + 7u;                   // biased E4M3 exponent, 1..15
  return sign | (e << 3) | ((r >> 20) & 7u);
}


// 8 consecutive elements of a new token's K or V row (packed 16-bit values of type IT) in
// the storage format of a cache of type KVT: a 16-bit cache takes the bits as they are
// (all 16 bytes); an fp8 cache takes E4M3FN(fl32(x / scale)) of each element (IEEE fp32
// division, round to nearest even, saturating, NaN kept; the 8 codes in the first two
// dwords). Both the cache-write kernel and the fused decode step convert new tokens
// through this function.
template <int IT, int KVT>
__device__ __forceinline__ u32x4 convert_cache_chunk(const u32x4 in, float scale) {
  if constexpr (KVT == kFP8) {
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pair = in[2 * w + e / 2];
        const float x = (e & 1) ? hi16<IT>(pair) : lo16<IT>(pair);
        packed |= e4m3_from_f32(x / scale) << (8 * e);
      }
      out[w] = packed;
    }
    return out;
  } else {
    return in;
  }
}

// Stores a converted chunk (8 elements) at element index `elem` of the cache.
template <int KVT>
__device__ __forceinline__ void store_converted_chunk(const u32x4 c, void* cache, int64_t elem) {
  if constexpr (KVT == kFP8)
    *(u32x2*)((uint8_t*)cache + elem) = u32x2{c[0], c[1]};
  else
    *(u32x4*)((uint16_t*)cache + elem) = c;
}

template <int IT, int KVT>
__device__ __forceinline__ void store_cache_chunk(const u32x4 in, void* cache, int64_t elem, float scale) {
  store_converted_chunk<KVT>(convert_cache_chunk<IT, KVT>(in, scale), cache, elem);
}

// ---- cross-lane butterflies (VALU permlane swaps, gfx950) ------------------------------
// Combine lane l with lane l^16 / l^32. permlane16_swap(v, v) hands each lane the pair
// {v[l & ~16], v[l | 16]}; permlane32_swap(v, v) the pair {v[l & 31], v[(l & 31) + 32]}.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane l exchanges with lane l ^ m for m < 16 through DPP-capable shuffles.
__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, kWave); }

__device__ __forceinline__ int readfirstlane(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace pkv
