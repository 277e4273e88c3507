// Paged decode attention for one query head per kv head (multi-head attention) on the
// vector ALUs of gfx950.
//
// What is computed is the pages' decode attention: Softmax(Q K^T / sqrt(d)) V with K
// and V gathered through the block table ("vLLM 推理优化技术深度调研报告", 维度一.1 and
// 维度一.3 公式 3-4). With a single query row per kv head there is no dense
// contraction to give the matrix cores, so the work stays on the VALU:
// * one wavefront per (sequence, kv head, context partition), block-table slice in LDS;
// * per 16-token block each lane owns one token row (lane >> 2) and a quarter of its
//   head_dim (lane & 3): 16-byte loads, dot2 instructions for q.k, then a DPP
//   quad butterfly completes each token's dot product;
// * online softmax: block max over the 16 tokens with DPP row rotations plus
//   permlane16/32 swaps; exp2 with log2 e folded into the scale;
// * each lane accumulates p * V for its token and columns; the 16 token partial
//   sums are combined once at the end of the partition.
#include "pkv_launch.h"

namespace pkv {

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;   // row_ror:4
constexpr int kRowRor8 = 0x128;   // row_ror:8

// Reduce over the 16 token rows (lane bits 2..5) of the wave.
__device__ __forceinline__ float sum_tokens(float x) {
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  return sum_xor32(sum_xor16(x));
}
__device__ __forceinline__ float max_tokens(float x) {
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor8>(x));
  return max_xor32(max_xor16(x));
}

template <int QT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

template <int QT, int KVT, int D>
struct ValuTraits {
  static constexpr int kElem = (KVT == kFP8) ? 1 : 2;
  static constexpr int kTileBytes = kBlock * D * kElem;
  static constexpr int kLoads = kTileBytes / (16 * kWave);   // 16-byte loads per lane per tile
  static constexpr int kPerLoad = 16 / kElem;                // elements per load
  static constexpr int kCols = D / 4;                        // head_dim columns per lane
};

// Column of the e-th element of load u for quarter q4: loads cover 16 bytes of the
// row each, quarters interleaved so that one instruction reads 64 contiguous bytes per row.
template <int KVT>
__device__ __forceinline__ int valu_col(int u, int q4) {
  return (KVT == kFP8 ? 16 : 8) * (4 * u + q4);
}

template <int QT, int KVT, int D>
struct VTile {
  u32x4 k[ValuTraits<QT, KVT, D>::kLoads];
  u32x4 v[ValuTraits<QT, KVT, D>::kLoads];
};

template <int QT, int KVT, int D>
__global__ __launch_bounds__(64) void paged_decode_valu(DecodeArgs a) {
  using Tr = ValuTraits<QT, KVT, D>;
  extern __shared__ int bt_lds[];

  const int j = item_of_workgroup(blockIdx.x);
  if (j >= a.num_items) return;
  const Item it = decode_item(j, a);
  const int lane = threadIdx.x, tr = lane >> 2, q4 = lane & 3;
  const int ctx = min(a.context_lens[it.s], a.max_blocks * kBlock);
  const int start = it.p * a.part_blocks * kBlock;
  const int head = it.g;   // one query head per kv head

  if (ctx <= start) {
    if (a.num_parts == 1 && tr == 0) {
      uint8_t* o = (uint8_t*)((uint16_t*)a.out + ((int64_t)it.s * a.num_q_heads + head) * D);
#pragma unroll
      for (int u = 0; u < Tr::kLoads; ++u) {
        const int c0 = valu_col<KVT>(u, q4);
        for (int e = 0; e < Tr::kPerLoad; e += 8) *(u32x4*)(o + (c0 + e) * 2) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }
  const int end = min(ctx, start + a.part_blocks * kBlock);
  const int nblk = (end - start + kBlock - 1) / kBlock;
  {
    const int32_t* bt = a.block_tables + (int64_t)it.s * a.max_blocks + (start / kBlock);
    for (int i = lane; i < nblk; i += kWave) bt_lds[i] = bt[i];
  }

  // q for this lane's columns, packed 16-bit pairs (same order as the K elements).
  uint32_t qv[Tr::kCols / 2];
  {
    const uint8_t* qrow = (const uint8_t*)((const uint16_t*)a.q + (int64_t)it.s * a.q_seq_stride +
                                           (int64_t)head * D);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      const int c0 = valu_col<KVT>(u, q4);
#pragma unroll
      for (int e = 0; e < Tr::kPerLoad; e += 8) {
        const u32x4 w = *(const u32x4*)(qrow + (c0 + e) * 2);
        const int base = (u * Tr::kPerLoad + e) / 2;
        qv[base + 0] = w[0]; qv[base + 1] = w[1]; qv[base + 2] = w[2]; qv[base + 3] = w[3];
      }
    }
  }
  __syncthreads();

  uint32_t off[Tr::kLoads];
#pragma unroll
  for (int u = 0; u < Tr::kLoads; ++u) off[u] = tr * D * Tr::kElem + valu_col<KVT>(u, q4) * Tr::kElem;

  const int64_t head_stride = (int64_t)Tr::kTileBytes;
  const uint8_t* kbase = (const uint8_t*)a.k_cache + (int64_t)it.g * head_stride;
  const uint8_t* vbase = (const uint8_t*)a.v_cache + (int64_t)it.g * head_stride;
  const int64_t block_stride = (int64_t)a.num_kv_heads * head_stride;

  auto load = [&](VTile<QT, KVT, D>& t, int i) {
    const int id = readfirstlane(i < nblk ? bt_lds[i < nblk ? i : 0] : -1);
    const bool live = id >= 0 && id < a.num_blocks;
    const int phys = live ? id : 0;
    const uint32_t bytes = live ? (uint32_t)Tr::kTileBytes : 0u;
    const auto rk = make_rsrc(kbase + phys * block_stride, bytes);
    const auto rv = make_rsrc(vbase + phys * block_stride, bytes);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.k[u] = buf_load16(rk, off[u]);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.v[u] = buf_load16(rv, off[u]);
  };

  float o[Tr::kCols];
#pragma unroll
  for (int c = 0; c < Tr::kCols; ++c) o[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = a.qk_scale_log2;

  // Packed 16-bit view of one loaded dword pair-list: for fp8 each dword widens to two.
  auto widen = [&](const u32x4& w, uint32_t* dst) {
    if constexpr (KVT == kFP8) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const u32x2 h = fp8x4_to_16<QT>(w[x]);
        dst[2 * x] = h[0];
        dst[2 * x + 1] = h[1];
      }
    } else {
      dst[0] = w[0]; dst[1] = w[1]; dst[2] = w[2]; dst[3] = w[3];
    }
  };
  constexpr int kWords = Tr::kPerLoad / 2;   // packed pairs per load after widening

  auto process = [&](const VTile<QT, KVT, D>& t, int i) {
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      uint32_t kw[kWords];
      widen(t.k[u], kw);
#pragma unroll
      for (int x = 0; x < kWords; ++x) dot = dot2<QT>(kw[x], qv[u * kWords + x], dot);
    }
    dot += dpp<kQuadXor1>(dot);
    dot += dpp<kQuadXor2>(dot);
    const bool valid = start + i * kBlock + tr < end;   // inside this partition and the context
    const float sc = valid ? dot * qk_scale : -INFINITY;
    const float m_new = fmaxf(m_run, max_tokens(sc));
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    const float p = exp2_fast(sc - m_new);
    l_run = l_run * alpha + p;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < Tr::kCols; ++c) o[c] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      uint32_t vw[kWords];
      widen(valid ? t.v[u] : u32x4{0u, 0u, 0u, 0u}, vw);
#pragma unroll
      for (int x = 0; x < kWords; ++x) {
        const int c = u * Tr::kPerLoad + 2 * x;
        o[c] = fmaf(p, lo16<QT>(vw[x]), o[c]);
        o[c + 1] = fmaf(p, hi16<QT>(vw[x]), o[c + 1]);
      }
    }
  };

  VTile<QT, KVT, D> t0, t1;
  load(t0, 0);
  load(t1, 1);
  // Two tiles in flight; see the matrix-core kernel for why a block past the end is
  // processed when nblk is odd (zero loads, all tokens masked, no effect).
  for (int i = 0; i < nblk; i += 2) {
    process(t0, i);
    load(t0, i + 2);
    process(t1, i + 1);
    load(t1, i + 3);
  }

  // Combine the 16 token rows.
  const float l_tot = sum_tokens(l_run);
#pragma unroll
  for (int c = 0; c < Tr::kCols; ++c) o[c] = sum_tokens(o[c]);
  if (tr != 0) return;
  const int64_t row = (int64_t)it.s * a.num_q_heads + head;
  if (a.num_parts == 1) {
    const float inv = a.v_scale / l_tot;
    uint8_t* orow = (uint8_t*)((uint16_t*)a.out + row * D);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      const int c0 = valu_col<KVT>(u, q4);
#pragma unroll
      for (int e = 0; e < Tr::kPerLoad; e += 8) {
        const int c = u * Tr::kPerLoad + e;
        u32x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = pack2<QT>(o[c + 2 * x] * inv, o[c + 2 * x + 1] * inv);
        *(u32x4*)(orow + (c0 + e) * 2) = w;
      }
    }
  } else {
    const int64_t prow = row * a.num_parts + it.p;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      const int c0 = valu_col<KVT>(u, q4);
#pragma unroll
      for (int e = 0; e < Tr::kPerLoad; e += 4) {
        const int c = u * Tr::kPerLoad + e;
        *(f32x4*)(po + c0 + e) = f32x4{o[c], o[c + 1], o[c + 2], o[c + 3]};
      }
    }
    if (q4 == 0) *(f32x2*)(a.part_ml + prow * 2) = f32x2{m_run, l_tot};
  }
}

template <int QT, int KVT, int D>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int grid = (a.num_items + 31) / 32 * 32;
  const size_t lds = (size_t)a.part_blocks * sizeof(int);
  hipLaunchKernelGGL((paged_decode_valu<QT, KVT, D>), dim3(grid), dim3(kWave), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeArgs& a, int q_type, int kv_type, int head_dim,
                              hipStream_t stream) {
#define PKV_CASE(QT, KVT, D) \
  if (q_type == QT && kv_type == KVT && head_dim == D) return launch_t<QT, KVT, D>(a, stream);
  PKV_CASE(kBF16, kBF16, 128) PKV_CASE(kBF16, kBF16, 64)
  PKV_CASE(kF16, kF16, 128) PKV_CASE(kF16, kF16, 64)
  PKV_CASE(kBF16, kFP8, 128) PKV_CASE(kBF16, kFP8, 64)
  PKV_CASE(kF16, kFP8, 128) PKV_CASE(kF16, kFP8, 64)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
