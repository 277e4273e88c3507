// Paged decode attention for grouped-query heads on gfx950 matrix cores.
//
// The method (what is computed) follows the pages: decode attention is the standard
// Softmax(Q K^T / sqrt(d)) V; only the read of K and V changes, which are gathered
// through the sequence's block table from 16-token physical blocks
// ("vLLM 推理优化技术深度调研报告", 维度一.1 误解二 and 维度一.3 公式 3-4;
// "vLLM推理引擎PagedAttention原理与性能优化实战", §2.2).
//
// How it is computed here (this design is not from the pages):
// * one wavefront per (sequence, kv head, context partition);
// * the partition's block-table slice is staged in LDS;
// * per 16-token block the G query heads of the kv head form a small dense
//   contraction: S^T[16 tok x 16 heads] = K[16 x D] . Q^T[D x 16] on
//   v_mfma_f32_16x16x32 (heads padded to 16 columns), then
//   O^T[D x 16 heads] += V^T[D x 16 tok] . P[16 tok x 16 heads] on
//   v_mfma_f32_16x16x16. The accumulator layout of S^T is exactly the operand
//   layout P needs, so softmax weights never leave their lanes;
// * K goes straight from HBM into MFMA operand registers (16-byte buffer loads);
//   V is staged through LDS (XOR-swizzled 16-byte chunks) and read back transposed
//   with ds_read_b64_tr_b16;
// * online softmax in fp32 with exp2 (log2 e folded into the scale); the running
//   max is combined across the four lane rows with permlane16/32 swaps;
// * tokens past the partition's end are excluded by select (K side) and by zeroing their
//   V rows (0 * stale NaN would otherwise poison the product);
// * an fp8 (OCP E4M3FN) cache is widened exactly to the q dtype in registers; its
//   per-tensor scales are folded into the logit scale and the output scale.
#include "pkv_launch.h"

namespace pkv {

template <int QT, int KVT, int D>
struct MfmaTraits {
  static constexpr int kElem = (KVT == kFP8) ? 1 : 2;   // bytes per cache element
  static constexpr int kTileBytes = kBlock * D * kElem; // one kv head's slice of a block
  static constexpr int kQk = D / 32;                    // 16x16x32 steps per block (QK)
  static constexpr int kPv = D / 16;                    // 16x16x16 steps per block (PV)
  static constexpr int kLoads = kTileBytes / (16 * kWave);  // 16-byte loads per lane per tile
  static constexpr int kRowChunks = D / 8;              // 16-byte chunks per 16-bit row in LDS
  static constexpr int kTileLds = kBlock * D * 2;       // one tile in LDS, 16-bit elements
  static constexpr int kLdsBytes = 2 * kTileLds;        // K tile, then V tile
};

template <int QT>
__device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int QT>
__device__ __forceinline__ f32x4 mfma_pv(i16x4 a, u32x2 b, f32x4 c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Element index d (within the head) that lane row j4 feeds as k-slots 8*j4..8*j4+7 of QK
// step c. The contraction order is free; it is fixed per cache dtype so that every way of
// reading K gives the same sums, bit for bit:
// * 16-bit caches: d = 32c + 8*j4 + i;
// * fp8 caches pair steps (2h, 2h+1) on one 16-byte load of 16 codes:
//   d = 64h + 16*j4 + 8*(c&1) + i.
// K reaches the matrix cores in one of two ways:
// * through LDS: the tile is loaded from HBM with whole rows per instruction (each 16-byte
//   load instruction covers one contiguous KiB), widened to 16-bit if it is fp8, stored
//   XOR-swizzled, and each lane reads its A-operand fragment (row n, elements d..d+7) as one
//   16-byte LDS read;
// * straight into registers: lane (n, j4) loads its own fragment of row n, so one load
//   instruction covers 16 rows x 64 bytes.
template <int KVT>
__device__ __forceinline__ int qk_d0(int c, int j4) {
  if constexpr (KVT == kFP8)
    return 64 * (c >> 1) + 16 * j4 + 8 * (c & 1);
  else
    return 32 * c + 8 * j4;
}

template <int QT, int KVT, int D>
struct Tile {
  u32x4 k[MfmaTraits<QT, KVT, D>::kLoads];
  u32x4 v[MfmaTraits<QT, KVT, D>::kLoads];
};

// One work item: the G query heads of kv head it.g of sequence it.s over context
// partition it.p, which holds tokens [start, ctx) up to the partition's end.
template <int QT, int KVT, int D, int NBUF, int POLICY, bool PRIO, bool KLDS>
__device__ __forceinline__ void mfma_item(const DecodeArgs& a, const Item it, const int ctx, const int start,
                                          int* bt_lds, uint8_t (*kv_lds)[MfmaTraits<QT, KVT, D>::kLdsBytes]) {
  using Tr = MfmaTraits<QT, KVT, D>;
  const int lane = threadIdx.x, n = lane & 15, j4 = lane >> 4;
  const int G = a.group;
  const int head = it.g * G + n;
  const int end = min(ctx, start + a.part_blocks * kBlock);
  const int nblk = (end - start + kBlock - 1) / kBlock;

  // Stage this partition's block-table slice in LDS.
  {
    const int32_t* bt = a.block_tables + (int64_t)it.s * a.max_blocks + (start / kBlock);
    for (int i = lane; i < nblk; i += kWave) bt_lds[i] = bt[i];
  }

  // Q^T as the B operand of the QK steps (rows of padded heads are zero).
  u32x4 qb[Tr::kQk];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)it.s * a.q_seq_stride + (int64_t)head * D;
#pragma unroll
    for (int c = 0; c < Tr::kQk; ++c)
      qb[c] = (n < G) ? *(const u32x4*)(qrow + qk_d0<KVT>(c, j4)) : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // Per-lane byte offsets inside one kv head's tile. V (and K through LDS): lane l reads
  // bytes [16 (64 u + l), +16) with load u, one contiguous KiB per instruction. K straight
  // into registers: lane (n, j4) reads its own fragment of row n.
  uint32_t koff[Tr::kLoads], voff[Tr::kLoads];
#pragma unroll
  for (int u = 0; u < Tr::kLoads; ++u) {
    voff[u] = (u * kWave + lane) * 16;
    if constexpr (KLDS)
      koff[u] = voff[u];
    else if constexpr (KVT == kFP8)
      koff[u] = n * D + 64 * u + 16 * j4;                       // row n, 16 fp8 values
    else
      koff[u] = (n * D + qk_d0<KVT>(u, j4)) * 2;          // row n, 8 values
  }

  const int64_t head_stride = (int64_t)Tr::kTileBytes;
  const uint8_t* kbase = (const uint8_t*)a.k_cache + (int64_t)it.g * head_stride;
  const uint8_t* vbase = (const uint8_t*)a.v_cache + (int64_t)it.g * head_stride;
  const int64_t block_stride = (int64_t)a.num_kv_heads * head_stride;

  auto load = [&](Tile<QT, KVT, D>& t, int i) {
    const int id = readfirstlane(i < nblk ? bt_lds[i < nblk ? i : 0] : -1);
    const bool live = id >= 0 && id < a.num_blocks;
    const int phys = live ? id : 0;
    const uint32_t bytes = live ? (uint32_t)Tr::kTileBytes : 0u;   // 0: loads return zeros
    const auto rk = make_rsrc(kbase + phys * block_stride, bytes);
    const auto rv = make_rsrc(vbase + phys * block_stride, bytes);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.k[u] = buf_load16<POLICY>(rk, koff[u]);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.v[u] = buf_load16<POLICY>(rv, voff[u]);
  };

  f32x4 o[Tr::kPv];
#pragma unroll
  for (int c = 0; c < Tr::kPv; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = a.qk_scale_log2;

  // A tile -> LDS as 16-bit rows; chunk k of row r is stored at k ^ (r mod chunks). Rows
  // at or past `valid_rows` are stored as zeros when `mask` is set.
  auto stage = [&](const u32x4* w_in, uint8_t* dst, bool mask, int valid_rows) {
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      const int f = u * kWave + lane;
      if constexpr (KVT == kFP8) {
        const int r = f / (D / 16), ch = f % (D / 16);
        u32x4 w = w_in[u];
        if (mask && r >= valid_rows) w = u32x4{0u, 0u, 0u, 0u};
        const u32x2 a0 = fp8x4_to_16<QT>(w[0]), a1 = fp8x4_to_16<QT>(w[1]);
        const u32x2 a2 = fp8x4_to_16<QT>(w[2]), a3 = fp8x4_to_16<QT>(w[3]);
        const int sw = r & (Tr::kRowChunks - 1);
        *(u32x4*)(dst + (r * Tr::kRowChunks + ((2 * ch) ^ sw)) * 16) = u32x4{a0[0], a0[1], a1[0], a1[1]};
        *(u32x4*)(dst + (r * Tr::kRowChunks + ((2 * ch + 1) ^ sw)) * 16) = u32x4{a2[0], a2[1], a3[0], a3[1]};
      } else {
        const int r = f / Tr::kRowChunks, ch = f % Tr::kRowChunks;
        u32x4 w = w_in[u];
        if (mask && r >= valid_rows) w = u32x4{0u, 0u, 0u, 0u};
        *(u32x4*)(dst + (r * Tr::kRowChunks + (ch ^ (r & (Tr::kRowChunks - 1)))) * 16) = w;
      }
    }
  };

  auto process = [&](const Tile<QT, KVT, D>& t, int i, uint8_t* lds) {
    uint8_t* kl = lds;
    uint8_t* vl = lds + Tr::kTileLds;
    // K rows past the partition are not masked here: their scores are replaced by -inf.
    // V rows past it are zeroed, since 0 * stale NaN would poison the product.
    const int valid_rows = end - start - i * kBlock;
    if constexpr (KLDS) stage(t.k, kl, false, 0);
    stage(t.v, vl, valid_rows < kBlock, valid_rows);
    __syncthreads();

    // S^T = K . Q^T for this block.
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < Tr::kQk; ++c) {
      u32x4 ka;
      if constexpr (KLDS) {
        const int ch = qk_d0<KVT>(c, j4) >> 3;   // 16-byte chunk of 8 16-bit elements
        ka = *(const u32x4*)(kl + (n * Tr::kRowChunks + (ch ^ (n & (Tr::kRowChunks - 1)))) * 16);
      } else if constexpr (KVT == kFP8) {
        const u32x4 w = t.k[c >> 1];
        const u32x2 lo = fp8x4_to_16<QT>(w[(c & 1) * 2]);
        const u32x2 hi = fp8x4_to_16<QT>(w[(c & 1) * 2 + 1]);
        ka = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        ka = t.k[c];
      }
      sacc = mfma_qk<QT>(ka, qb[c], sacc);
    }
    // Scores of tokens 4*j4 .. 4*j4+3 of the block for head n; masked ones are -inf.
    const int tok0 = start + i * kBlock + 4 * j4;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (tok0 + r < end) ? sacc[r] * qk_scale : -INFINITY;
    float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mb = max_xor16(mb);
    mb = max_xor32(mb);
    const float m_new = fmaxf(m_run, mb);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    const uint32_t p01 = pack2<QT>(exp2_fast(sc[0] - m_new), exp2_fast(sc[1] - m_new));
    const uint32_t p23 = pack2<QT>(exp2_fast(sc[2] - m_new), exp2_fast(sc[3] - m_new));
    // The denominator sums the rounded weights that the PV product uses.
    l_run = l_run * alpha + ((lo16<QT>(p01) + hi16<QT>(p01)) + (lo16<QT>(p23) + hi16<QT>(p23)));
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < Tr::kPv; ++c) o[c] *= alpha;
    }

    // O^T += V^T . P
    const u32x2 pb = {p01, p23};
    const int rr = 4 * j4 + (n >> 2);
    const int sw = rr & (Tr::kRowChunks - 1);
#pragma unroll
    for (int c = 0; c < Tr::kPv; ++c) {
      const int ch = 2 * c + ((n & 3) >> 1);
      const uint32_t addr = (rr * Tr::kRowChunks + (ch ^ sw)) * 16 + (n & 1) * 8;
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vl + addr));
      o[c] = mfma_pv<QT>(va, pb, o[c]);
    }
  };

  // NBUF tiles in flight, kept in a ring of register tiles. The loop body has no branch
  // around a load, so the waitcnt counts stay exact; when nblk is not a multiple of NBUF
  // the last round processes blocks past the end, which is harmless: their loads return
  // zeros and every one of their tokens is masked (alpha = 1, p = 0).
  Tile<QT, KVT, D> t[NBUF];
#pragma unroll
  for (int b = 0; b < NBUF; ++b) load(t[b], b);
  for (int i = 0; i < nblk; i += NBUF) {
    if constexpr (PRIO) progress_priority(i, nblk);
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      process(t[b], i + b, kv_lds[b & 1]);
      load(t[b], i + b + NBUF);
    }
  }

  const float l_tot = sum_xor32(sum_xor16(l_run));
  if (n >= G) return;
  const int64_t row = (int64_t)it.s * a.num_q_heads + head;
  if (a.num_parts == 1) {
    const float inv = a.v_scale / l_tot;
    uint16_t* orow = (uint16_t*)a.out + row * D;
#pragma unroll
    for (int c = 0; c < Tr::kPv; ++c) {
      const f32x4 v = o[c] * inv;
      *(u32x2*)(orow + 16 * c + 4 * j4) = u32x2{pack2<QT>(v[0], v[1]), pack2<QT>(v[2], v[3])};
    }
  } else {
    const int64_t prow = row * a.num_parts + it.p;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int c = 0; c < Tr::kPv; ++c) *(f32x4*)(po + 16 * c + 4 * j4) = o[c];
    if (j4 == 0) *(f32x2*)(a.part_ml + prow * 2) = f32x2{m_run, l_tot};
  }
}

template <int QT, int KVT, int D>
__global__ __launch_bounds__(64) void paged_decode_mfma(DecodeArgs a) {
  using Tr = MfmaTraits<QT, KVT, D>;
  extern __shared__ int bt_lds[];
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2][Tr::kLdsBytes];

  const int j = item_of_workgroup(blockIdx.x);
  if (j >= a.num_items) return;
  const Item it = decode_item(j, a);
  const int ctx = min(a.context_lens[it.s], a.max_blocks * kBlock);
  const int start = it.p * a.part_blocks * kBlock;
  if (ctx <= start) {
    // Nothing in this partition. A whole sequence with no context writes zeros.
    const int n = threadIdx.x & 15, j4 = threadIdx.x >> 4;
    if (a.num_parts == 1 && n < a.group) {
      uint16_t* o = (uint16_t*)a.out + ((int64_t)it.s * a.num_q_heads + it.g * a.group + n) * D;
#pragma unroll
      for (int c = 0; c < Tr::kPv; ++c) *(u32x2*)(o + 16 * c + 4 * j4) = u32x2{0u, 0u};
    }
    return;
  }
  // Blocks shared with a neighbouring sequence: cached loads (the other readers hit L2),
  // two tiles in flight, default priority, K straight into registers (these items are
  // bound by per-block latency more than by HBM). Private blocks stream, with K through
  // LDS; a whole context in one partition does best with one tile in flight per wave, a
  // split context (more items than wave slots) with two.
  if (neighbour_shares_block(a, it.s, start / kBlock))
    mfma_item<QT, KVT, D, 2, kPolicyCached, false, false>(a, it, ctx, start, bt_lds, kv_lds);
  else if (a.num_parts > 1)
    mfma_item<QT, KVT, D, 2, kPolicyStream, true, true>(a, it, ctx, start, bt_lds, kv_lds);
  else
    mfma_item<QT, KVT, D, 1, kPolicyStream, true, true>(a, it, ctx, start, bt_lds, kv_lds);
}

template <int QT, int KVT, int D>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int grid = (a.num_items + 31) / 32 * 32;
  const size_t lds = (size_t)a.part_blocks * sizeof(int);
  hipLaunchKernelGGL((paged_decode_mfma<QT, KVT, D>), dim3(grid), dim3(kWave), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int q_type, int kv_type, int head_dim,
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
