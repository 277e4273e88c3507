// Paged decode attention for one query head per kv head (multi-head attention) on the
// vector ALUs of gfx950.
//
// What is computed is the pages' decode attention: Softmax(Q K^T / sqrt(d)) V with K
// and V gathered through the block table ("vLLM 推理优化技术深度调研报告", 维度一.1 and
// 维度一.3 公式 3-4). With a single query row per kv head there is no dense
// contraction to give the matrix cores, so the work stays on the VALU:
// * one wavefront per (sequence, kv head, context partition), block-table slice in LDS;
// * each 16-byte load instruction reads whole rows of the block's tile (one contiguous
//   KiB), so lane l always holds the same column slice of head_dim, taken from a
//   different token row in each load; q and the output accumulators are that one slice;
// * q.k with dot2 instructions, then a DPP butterfly over the lanes of a row finishes each
//   token's dot product;
// * online softmax: block max and sum across the row groups with DPP row rotations and
//   permlane16/32 swaps; exp2 with log2 e folded into the scale;
// * each lane accumulates p * V for its rows and columns; the row groups are combined
//   once at the end of the partition.
#include "pkv_launch.h"

namespace pkv {

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane l <-> 7 - l within each 8 lanes
constexpr int kRowMirror = 0x140;      // lane l <-> 15 - l within each 16 lanes
constexpr int kRowRor4 = 0x124;        // row_ror:4
constexpr int kRowRor8 = 0x128;        // row_ror:8

// K+V tiles each wavefront keeps in flight (one measured best on gfx950: the two waves
// of a SIMD already overlap each other's loads).
constexpr int kValuTilesInFlight = 1;

template <int QT, int KVT, int D>
struct ValuTraits {
  static constexpr int kElem = (KVT == kFP8) ? 1 : 2;
  static constexpr int kTileBytes = kBlock * D * kElem;     // one kv head's slice of a block
  static constexpr int kLoads = kTileBytes / (16 * kWave);  // 16-byte loads per lane per tile
  static constexpr int kLanesPerRow = D * kElem / 16;       // lanes sharing one token row
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow; // token rows one load covers
  static constexpr int kCols = 16 / kElem;                  // head_dim columns per lane
  static constexpr int kWords = kCols / 2;                  // packed 16-bit pairs per lane
};

// Sum over the kLanesPerRow consecutive lanes holding one row (the result lands in all).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (LPR >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kRowMirror>(x);
  return x;
}

// Max / sum across the row groups: over all lanes that share l % LPR.
template <int LPR>
__device__ __forceinline__ float groups_max(float x) {
  if constexpr (LPR <= 4) x = fmaxf(x, dpp<kRowRor4>(x));
  if constexpr (LPR <= 8) x = fmaxf(x, dpp<kRowRor8>(x));
  return max_xor32(max_xor16(x));
}
template <int LPR>
__device__ __forceinline__ float groups_sum(float x) {
  if constexpr (LPR <= 4) x += dpp<kRowRor4>(x);
  if constexpr (LPR <= 8) x += dpp<kRowRor8>(x);
  return sum_xor32(sum_xor16(x));
}

template <int QT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// One 16-byte load as packed 16-bit pairs of the q dtype (fp8 codes widen exactly).
template <int QT, int KVT>
__device__ __forceinline__ void widen(const u32x4& w, uint32_t* dst) {
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
}

template <int QT, int KVT, int D>
struct VTile {
  u32x4 k[ValuTraits<QT, KVT, D>::kLoads];
  u32x4 v[ValuTraits<QT, KVT, D>::kLoads];
};

// One work item: query head it.g of sequence it.s over context partition it.p, which
// holds tokens [start, ctx) up to the partition's end.
template <int QT, int KVT, int D, int NBUF, int POLICY, bool PRIO>
__device__ __forceinline__ void valu_item(const DecodeArgs& a, const Item it, const int ctx, const int start,
                                          const BtSlice& sl, int* bt_lds, uint8_t* tok_rows, const bool writes,
                                          const TokenChunk& token) {
  using Tr = ValuTraits<QT, KVT, D>;
  constexpr int LPR = Tr::kLanesPerRow, RPL = Tr::kRowsPerLoad;
  const int lane = threadIdx.x, grp = lane / LPR, col0 = (lane % LPR) * Tr::kCols;
  const int head = it.g;   // one query head per kv head
  const int end = min(ctx, start + a.part_blocks * kBlock);
  const int nblk = (end - start + kBlock - 1) / kBlock;
  // q columns [col0, col0 + kCols) as packed 16-bit pairs.
  uint32_t qv[Tr::kWords];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)it.s * a.q_seq_stride + (int64_t)head * D + col0;
#pragma unroll
    for (int x = 0; x < Tr::kWords; x += 4) {
      const u32x4 w = *(const u32x4*)(qrow + 2 * x);
      qv[x] = w[0]; qv[x + 1] = w[1]; qv[x + 2] = w[2]; qv[x + 3] = w[3];
    }
  }
  {
    const CowRead cow = cow_read(a, it.s, ctx);
    stash_cow(tok_rows, cow);
    store_bt_slice(a, it.s, start / kBlock, nblk, sl, bt_lds, cow);
  }
  if (writes) stage_new_token<KVT, D>(token, tok_rows);
  __syncthreads();
  // Fused step: the tile of the new token (the sequence's last position, ctx - 1) gets the
  // token's row from its LDS copy before use; the cache slot still holds stale bytes.
  const int patch_tile = writes && token.written ? (ctx - 1) / kBlock - start / kBlock : -1;
  const int patch_row = (ctx - 1) % kBlock;

  const int shift = a.block_shift;
  const int64_t head_stride = (int64_t)Tr::kTileBytes << shift;   // one kv head's slice of a block
  const uint8_t* kbase = (const uint8_t*)a.k_cache + (int64_t)it.g * head_stride;
  const uint8_t* vbase = (const uint8_t*)a.v_cache + (int64_t)it.g * head_stride;
  const int64_t block_stride = (int64_t)a.num_kv_heads * head_stride;
  const uint32_t off0 = lane * 16;

  auto load = [&](VTile<QT, KVT, D>& t, int i) {
    const int id = readfirstlane(i < nblk ? bt_lds[i < nblk ? i : 0] : -1);
    const bool live = id >= 0;                                     // ids are tile names
    const int64_t off = live ? tile_offset(id, shift, block_stride, Tr::kTileBytes) : 0;
    const uint32_t bytes = live ? (uint32_t)Tr::kTileBytes : 0u;   // 0: loads return zeros
    const auto rk = make_rsrc(kbase + off, bytes);
    const auto rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.k[u] = buf_load16<POLICY>(rk, off0 + u * 1024);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.v[u] = buf_load16<POLICY>(rv, off0 + u * 1024);
  };

  float o[Tr::kCols];
#pragma unroll
  for (int c = 0; c < Tr::kCols; ++c) o[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = a.qk_scale_log2;

  auto process = [&](VTile<QT, KVT, D>& t, int i) {
    if (i == patch_tile) {
#pragma unroll
      for (int u = 0; u < Tr::kLoads; ++u) {
        patch_piece<KVT, D>(t.k[u], off0 + u * 1024, patch_row, tok_rows);
        patch_piece<KVT, D>(t.v[u], off0 + u * 1024, patch_row, tok_rows + row_bytes<KVT, D>());
      }
    }
    float sc[Tr::kLoads];
    bool valid[Tr::kLoads];
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      uint32_t kw[Tr::kWords];
      widen<QT, KVT>(t.k[u], kw);
      float dot = 0.f;
#pragma unroll
      for (int x = 0; x < Tr::kWords; ++x) dot = dot2<QT>(kw[x], qv[x], dot);
      dot = row_sum<LPR>(dot);
      valid[u] = start + i * kBlock + u * RPL + grp < end;   // inside this partition and the context
      sc[u] = valid[u] ? dot * qk_scale : -INFINITY;
    }
    float mb = sc[0];
#pragma unroll
    for (int u = 1; u < Tr::kLoads; ++u) mb = fmaxf(mb, sc[u]);
    const float m_new = fmaxf(m_run, groups_max<LPR>(mb));
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    float p[Tr::kLoads], psum = 0.f;
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      p[u] = exp2_fast(sc[u] - m_new);
      psum += p[u];
    }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < Tr::kCols; ++c) o[c] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      uint32_t vw[Tr::kWords];
      widen<QT, KVT>(valid[u] ? t.v[u] : u32x4{0u, 0u, 0u, 0u}, vw);   // stale rows never multiply
#pragma unroll
      for (int x = 0; x < Tr::kWords; ++x) {
        o[2 * x] = fmaf(p[u], lo16<QT>(vw[x]), o[2 * x]);
        o[2 * x + 1] = fmaf(p[u], hi16<QT>(vw[x]), o[2 * x + 1]);
      }
    }
  };

  // NBUF tiles in flight in a ring of register tiles; see the matrix-core kernel for why
  // blocks past the end may be processed (zero loads, all tokens masked, no effect).
  VTile<QT, KVT, D> t[NBUF];
#pragma unroll
  for (int b = 0; b < NBUF; ++b) load(t[b], b);
  for (int i = 0; i < nblk; i += NBUF) {
    if constexpr (PRIO) progress_priority(i, nblk);
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      process(t[b], i + b);
      load(t[b], i + b + NBUF);
    }
  }

  if (writes) {
    store_new_token<KVT>(a, token);
    cow_copy<KVT, D>(a, it.g, stashed_cow(tok_rows));
  }

  // Combine the row groups.
  const float l_tot = groups_sum<LPR>(l_run);
#pragma unroll
  for (int c = 0; c < Tr::kCols; ++c) o[c] = groups_sum<LPR>(o[c]);
  if (grp != 0) return;
  const int64_t row = (int64_t)it.s * a.num_q_heads + head;
  if (a.num_parts == 1) {
    const float inv = a.v_scale / l_tot;
    uint16_t* orow = (uint16_t*)a.out + row * D + col0;
#pragma unroll
    for (int x = 0; x < Tr::kWords; x += 4) {
      u32x4 w;
#pragma unroll
      for (int y = 0; y < 4; ++y) w[y] = pack2<QT>(o[2 * (x + y)] * inv, o[2 * (x + y) + 1] * inv);
      *(u32x4*)(orow + 2 * x) = w;
    }
  } else {
    const int64_t prow = row * a.num_parts + it.p;
    float* po = a.part_o + prow * D + col0;
#pragma unroll
    for (int c = 0; c < Tr::kCols; c += 4) *(f32x4*)(po + c) = f32x4{o[c], o[c + 1], o[c + 2], o[c + 3]};
    if (lane == 0) *(f32x2*)(a.part_ml + prow * 2) = f32x2{m_run, l_tot};
  }
}

template <int QT, int KVT, int D, int NBUF>
__global__ __launch_bounds__(64) void paged_decode_valu(DecodeArgs a) {
  using Tr = ValuTraits<QT, KVT, D>;
  extern __shared__ int bt_lds[];
  __shared__ __attribute__((aligned(16))) uint8_t tok_rows[kTokenRowsLds];
  const int j = item_of_workgroup(blockIdx.x, a);
  if (j >= a.num_items) return;
  const Item it = decode_item(j, a);
  if (it.s >= a.num_seqs) return;   // padding of the last run of 4 sequences
  const int start = it.p * a.part_blocks * kBlock;
  // The context length and the block ids at the partition's first logical block of this
  // sequence and its two neighbours, loaded at once (clamped into the batch).
  const int i0 = (start / kBlock) >> a.block_shift;   // block of the partition's first tile
  const int s_prev = max(it.s - 1, 0), s_next = min(it.s + 1, a.num_seqs - 1);
  const int ctx = min(a.context_lens[it.s], (a.max_blocks * kBlock) << a.block_shift);
  const int first_prev = a.block_tables[(int64_t)s_prev * a.max_blocks + i0];
  const int first = a.block_tables[(int64_t)it.s * a.max_blocks + i0];
  const int first_next = a.block_tables[(int64_t)s_next * a.max_blocks + i0];
  // The block-table slice, and with one partition (where every item writes its
  // sequence's new token in a fused step) the new token, are loaded before the context
  // length arrives.
  BtSlice sl;
  prefetch_bt_slice(a, it.s, start / kBlock, sl);
  const bool token_early = a.new_key != nullptr && a.num_parts == 1;
  TokenChunk token = {};
  if (token_early) token = load_new_token<QT, KVT, D>(a, it.s, it.g);
  const bool writes = owns_new_token(a, ctx, it.p);
  if (writes && !token_early) token = load_new_token<QT, KVT, D>(a, it.s, it.g);
  if (ctx <= start) {
    if (writes) store_new_token<KVT>(a, token);
    // Nothing in this partition. A whole sequence with no context writes zeros.
    const int lane = threadIdx.x;
    if (a.num_parts == 1 && lane < Tr::kLanesPerRow) {
      uint16_t* o = (uint16_t*)a.out + ((int64_t)it.s * a.num_q_heads + it.g) * D + lane * Tr::kCols;
#pragma unroll
      for (int x = 0; x < Tr::kCols; x += 8) *(u32x4*)(o + x) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const bool shared = (it.s > 0 && first_prev == first) || (it.s + 1 < a.num_seqs && first_next == first);
  if (shared)
    valu_item<QT, KVT, D, NBUF, kPolicyCached, false>(a, it, ctx, start, sl, bt_lds, tok_rows, writes, token);
  else
    valu_item<QT, KVT, D, NBUF, kPolicyStream, true>(a, it, ctx, start, sl, bt_lds, tok_rows, writes, token);
}

template <int QT, int KVT, int D>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int grid = decode_grid(a);
  const size_t lds = (size_t)a.part_blocks * sizeof(int);
  hipLaunchKernelGGL((paged_decode_valu<QT, KVT, D, kValuTilesInFlight>), dim3(grid), dim3(kWave), lds, stream, a);
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
