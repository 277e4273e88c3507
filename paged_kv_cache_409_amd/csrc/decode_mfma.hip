// Paged decode attention for grouped-query heads on gfx950 matrix cores.
//
// The method (what is computed) follows the pages: decode attention is the standard
// Softmax(Q K^T / sqrt(d)) V; only the read of K and V changes, which are gathered
// through the sequence's block table from 16-token physical blocks
// ("vLLM 推理优化技术深度调研报告", 维度一.1 误解二 and 维度一.3 公式 3-4;
// "vLLM推理引擎PagedAttention原理与性能优化实战", §2.2). Sequences forked from one prompt
// (beams) share its blocks ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.1-3.2).
//
// How it is computed here (this design is not from the pages):
// * a workgroup holds B = 16 / G wavefronts for B consecutive sequences of one kv head
//   and one context partition;
// * per 16-token block the query heads form a small dense contraction:
//   S^T[16 tok x 16 cols] = K[16 x D] . Q^T[D x 16] on v_mfma_f32_16x16x32, then
//   O^T[D x 16 cols] += V^T[D x 16 tok] . P[16 tok x 16 cols] on v_mfma_f32_16x16x16.
//   The accumulator layout of S^T is exactly the operand layout P needs, so softmax
//   weights never leave their lanes;
// * independent mode: each wavefront runs its own sequence; its G query heads are
//   columns 0..G-1 (the rest are masked);
// * group mode, when the workgroup's sequences share blocks: the 16 columns are the
//   B sequences x G heads. Wave 0 lists, per logical block, the distinct physical
//   blocks of the B sequences with the set of sequences that read each; the waves split
//   that list, so a shared block is read from HBM and multiplied once for all of its
//   readers; at the end the waves' softmax states are merged in LDS;
// * V (and K for blocks read once) is loaded with whole rows per instruction, staged in
//   LDS as XOR-swizzled 16-byte chunks and read back as MFMA operands (V transposed with
//   ds_read_b64_tr_b16);
// * online softmax in fp32 with exp2 (log2 e folded into the scale); the running max
//   of a column is combined across its four lane rows with permlane16/32 swaps;
// * tokens outside a column's context are excluded by select, and V rows past every
//   reader's context are zeroed (0 * stale NaN would otherwise poison the product);
// * an fp8 (OCP E4M3FN) cache is widened exactly to the q dtype; its per-tensor scales
//   are folded into the logit scale and the output scale.
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
  static constexpr int kLdsBytes = 2 * kTileLds;        // K tile, then V tile (per wavefront)
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
  int pos;          // logical block index within the sequences
  int rows;         // V rows [0, rows) hold live tokens of some reader; the rest are zeroed
  uint32_t readers; // bit b: sequence b of the group reads this block (bit 0 in independent mode)
};

// Running softmax state of one wavefront: per lane (column n, rows 4*j4..4*j4+3 of each
// 16-row chunk of D).
template <int D>
struct State {
  f32x4 o[D / 16];
  float m, l;
};

// The tiles of one wavefront. With LIST, tile k is entry k * stride of (ids, meta); meta
// packs the logical block index (bits 0-15), the reader set (bits 16-23) and the live V
// rows (bits 24-28). Without LIST, ids is the block-table slice and tile k is logical
// block pos0 + k, read by sequence 0, with live rows up to `tile_end`.
// col_bit / col_end: the reader bit of this lane's column (0: padded column), and the end
// (exclusive, absolute token index) of that reader's context in this partition.
// Fused step: the tile that holds a new token is patched with the token's row before use
// (its cache slot still holds stale bytes). Without LIST: the token is at logical block
// `ppos` (-1: none), row `prow`, its rows in LDS at `tok_rows`. With LIST: sequence b of
// the group has its token at block patch_pos[b] (-1: none), row patch_row[b], rows at
// tok_rows + b * kTokenRowsLds; only a block with a single reader can hold one.
template <int QT, int KVT, int D, int NBUF, int POLICY, bool PRIO, bool KLDS, bool LIST>
__device__ __forceinline__ void mfma_tiles(const DecodeArgs& a, const int g, const int ntiles, const int* ids,
                                           const int* meta, const int stride, const int pos0, const int tile_end,
                                           const u32x4* qb, const uint32_t col_bit, const int col_end,
                                           uint8_t* lds, State<D>& st, const int ppos, const int prow,
                                           const int* patch_pos, const int* patch_row, const uint8_t* tok_rows) {
  using Tr = MfmaTraits<QT, KVT, D>;
  const int lane = threadIdx.x & (kWave - 1), n = lane & 15, j4 = lane >> 4;

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
      koff[u] = (n * D + qk_d0<KVT>(u, j4)) * 2;                // row n, 8 values
  }

  const int shift = a.block_shift;
  const int64_t head_stride = (int64_t)Tr::kTileBytes << shift;   // one kv head's slice of a block
  const uint8_t* kbase = (const uint8_t*)a.k_cache + (int64_t)g * head_stride;
  const uint8_t* vbase = (const uint8_t*)a.v_cache + (int64_t)g * head_stride;
  const int64_t block_stride = (int64_t)a.num_kv_heads * head_stride;

  auto load = [&](Tile<QT, KVT, D>& t, int k) {
    int id = -1, pos = 0, rows = 0, readers = 0;
    if (k < ntiles) {
      if constexpr (LIST) {
        id = ids[k * stride];
        const int m = meta[k * stride];
        pos = m & 0xffff;
        readers = (m >> 16) & 0xff;
        rows = (m >> 24) & 0x1f;
      } else {
        id = ids[k];
        pos = pos0 + k;
        readers = 1;
        rows = min(tile_end - pos * kBlock, kBlock);
      }
    }
    id = readfirstlane(id);
    t.pos = readfirstlane(pos);
    t.rows = readfirstlane(rows);
    t.readers = (uint32_t)readfirstlane(readers);
    const bool live = id >= 0;                                     // ids are tile names
    const int64_t off = live ? tile_offset(id, shift, block_stride, Tr::kTileBytes) : 0;
    const uint32_t bytes = live ? (uint32_t)Tr::kTileBytes : 0u;   // 0: loads return zeros
    const auto rk = make_rsrc(kbase + off, bytes);
    const auto rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.k[u] = buf_load16<POLICY>(rk, koff[u]);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) t.v[u] = buf_load16<POLICY>(rv, voff[u]);
  };

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

  const float qk_scale = a.qk_scale_log2;
  uint8_t* kl = lds;
  uint8_t* vl = lds + Tr::kTileLds;

  // Processes tile t. With one tile in flight its registers are reloaded with tile `next`
  // as soon as they are free (after staging for K through LDS, after the QK products for K
  // in registers), so that the next tile's loads overlap this tile's products and softmax
  // (1.3% on the 70B batch). With two tiles in flight the reload follows the processing: a
  // third tile's worth of loads in flight measured slower there.
  constexpr bool kEarly = NBUF == 1;
  auto process = [&](Tile<QT, KVT, D>& t, const int next) {
    const int pos = t.pos;
    const uint32_t readers_of = t.readers;
    // Fused step: swap the new token's row into the tile.
    int trow = -1;
    const uint8_t* tsrc = tok_rows;
    if constexpr (LIST) {
      const uint32_t r = t.readers;
      if (r != 0u && (r & (r - 1u)) == 0u) {
        const int b = __builtin_ctz(r);
        if (patch_pos[b] == t.pos) {
          trow = patch_row[b];
          tsrc = tok_rows + b * kTokenRowsLds;
        }
      }
    } else {
      if (t.pos == ppos) trow = prow;
    }
    if (trow >= 0) {
#pragma unroll
      for (int u = 0; u < Tr::kLoads; ++u) {
        patch_piece<KVT, D>(t.k[u], koff[u], trow, tsrc);
        patch_piece<KVT, D>(t.v[u], voff[u], trow, tsrc + row_bytes<KVT, D>());
      }
    }
    // K rows of dead tokens are not masked here: their scores are replaced by -inf.
    // V rows past every reader's context are zeroed.
    if constexpr (KLDS) stage(t.k, kl, false, 0);
    stage(t.v, vl, t.rows < kBlock, t.rows);
    if constexpr (kEarly && KLDS) load(t, next);
    wave_lds_sync();

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
    if constexpr (kEarly && !KLDS) load(t, next);
    // Scores of tokens 4*j4 .. 4*j4+3 of the block for column n; dead ones are -inf.
    const int tok0 = pos * kBlock + 4 * j4;
    const bool reads = (readers_of & col_bit) != 0u;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (reads && tok0 + r < col_end) ? sacc[r] * qk_scale : -INFINITY;
    float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mb = max_xor16(mb);
    mb = max_xor32(mb);
    const float m_new = fmaxf(st.m, mb);
    // A column that has seen no live token yet keeps m = -inf; exponents are then taken
    // against 0 so that they come out as exp2(-inf) = 0, never as exp2(-inf + inf).
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = st.m == m_new ? 1.0f : exp2_fast(st.m - m_ref);
    st.m = m_new;
    const uint32_t p01 = pack2<QT>(exp2_fast(sc[0] - m_ref), exp2_fast(sc[1] - m_ref));
    const uint32_t p23 = pack2<QT>(exp2_fast(sc[2] - m_ref), exp2_fast(sc[3] - m_ref));
    // The denominator sums the rounded weights that the PV product uses.
    st.l = st.l * alpha + ((lo16<QT>(p01) + hi16<QT>(p01)) + (lo16<QT>(p23) + hi16<QT>(p23)));
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < Tr::kPv; ++c) st.o[c] *= alpha;
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
      st.o[c] = mfma_pv<QT>(va, pb, st.o[c]);
    }
  };

  // NBUF tiles in flight, kept in a ring of register tiles. The loop body has no branch
  // around a load, so the waitcnt counts stay exact; when ntiles is not a multiple of
  // NBUF the last round processes tiles past the end, which is harmless: their loads
  // return zeros and no column reads them (alpha = 1, p = 0).
  Tile<QT, KVT, D> t[NBUF];
#pragma unroll
  for (int b = 0; b < NBUF; ++b) load(t[b], b);
  for (int k = 0; k < ntiles; k += NBUF) {
    if constexpr (PRIO) progress_priority(k, ntiles);
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      process(t[b], k + b + NBUF);
      if constexpr (!kEarly) load(t[b], k + b + NBUF);
    }
  }
}

// Q^T as the B operand of the QK steps for column n = lane & 15: query head `head` of
// sequence s, or zeros for a padded column.
template <int QT, int KVT, int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, bool valid, int s, int head, u32x4* qb) {
  const int j4 = (threadIdx.x & (kWave - 1)) >> 4;
  const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)s * a.q_seq_stride + (int64_t)head * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    qb[c] = valid ? *(const u32x4*)(qrow + qk_d0<KVT>(c, j4)) : u32x4{0u, 0u, 0u, 0u};
}

// Column n's result: out[s, head] (one partition) or the fp32 partial of partition p.
// `l` is the column's full sum; o holds this lane's rows. The caller writes the 16-row
// chunks c of D with c mod nw == w (all of them with the defaults); chunk owner 0 also
// writes the partition's (max, sum).
template <int QT, int D>
__device__ __forceinline__ void write_column(const DecodeArgs& a, int s, int head, int p, const f32x4* o,
                                             float m, float l, int w = 0, int nw = 1) {
  const int j4 = (threadIdx.x & (kWave - 1)) >> 4;
  const int64_t row = (int64_t)s * a.num_q_heads + head;
  if (a.num_parts == 1) {
    const float inv = a.v_scale / l;
    uint16_t* orow = (uint16_t*)a.out + row * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      if (c % nw != w) continue;
      const f32x4 v = o[c] * inv;
      *(u32x2*)(orow + 16 * c + 4 * j4) = u32x2{pack2<QT>(v[0], v[1]), pack2<QT>(v[2], v[3])};
    }
  } else {
    const int64_t prow = row * a.num_parts + p;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      if (c % nw == w) *(f32x4*)(po + 16 * c + 4 * j4) = o[c];
    if (j4 == 0 && w == 0) *(f32x2*)(a.part_ml + prow * 2) = f32x2{m, l};
  }
}

// Independent mode: one wavefront, the G query heads of kv head g of sequence s over
// partition p, which holds tokens [start, ctx) up to the partition's end.
template <int QT, int KVT, int D, int NBUF, int POLICY, bool PRIO, bool KLDS>
__device__ __forceinline__ void mfma_single(const DecodeArgs& a, const int s, const int g, const int p,
                                            const int ctx, const int start, const BtSlice& sl, int* bt_lds,
                                            uint8_t* lds, uint8_t* tok_rows, const bool writes,
                                            const TokenChunk& token) {
  const int lane = threadIdx.x & (kWave - 1), n = lane & 15;
  const int G = a.group;
  const int end = min(ctx, start + a.part_blocks * kBlock);
  const int nblk = (end - start + kBlock - 1) / kBlock;
  {
    const CowRead cow = cow_read(a, s, ctx);
    stash_cow(tok_rows, cow);
    store_bt_slice(a, s, start / kBlock, nblk, sl, bt_lds, cow);
  }
  if (writes) stage_new_token<KVT, D>(token, tok_rows);
  u32x4 qb[D / 32];
  load_q<QT, KVT, D>(a, n < G, s, g * G + n, qb);
  wave_lds_sync();

  State<D> st;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  // The new token sits at the sequence's last position, ctx - 1.
  mfma_tiles<QT, KVT, D, NBUF, POLICY, PRIO, KLDS, false>(a, g, nblk, bt_lds, nullptr, 1, start / kBlock, end,
                                                          qb, n < G ? 1u : 0u, end, lds, st,
                                                          writes && token.written ? (ctx - 1) / kBlock : -1,
                                                          (ctx - 1) % kBlock,
                                                          nullptr, nullptr, tok_rows);
  if (writes) {
    store_new_token<KVT>(a, token);
    cow_copy<KVT, D>(a, g, stashed_cow(tok_rows));
  }
  const float l_tot = sum_xor32(sum_xor16(st.l));
  if (n < G) write_column<QT, D>(a, s, g * G + n, p, st.o, st.m, l_tot);
}

// Group mode: the B wavefronts of the workgroup compute sequences s0 .. s0+B-1 of kv head
// g over partition p together. Every one of them has tokens in the partition. Wave w's
// sequence s0 + w has context length ctx; its block-table slice was prefetched into sl,
// and its new token (fused step) is in `token` when token_loaded.
template <int QT, int KVT, int D>
__device__ __forceinline__ void mfma_group(const DecodeArgs& a, const int s0, const int g, const int p,
                                           const int start, const int ctx, const BtSlice& sl,
                                           TokenChunk token, const bool token_loaded, uint8_t* smem) {
  using Tr = MfmaTraits<QT, KVT, D>;
  const int B = a.seqs_per_group, G = a.group, PB = a.part_blocks;
  const int lstride = group_list_stride(PB);
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1), n = lane & 15, j4 = lane >> 4;
  uint8_t* tiles = smem;
  uint8_t* tok_rows = smem + B * Tr::kLdsBytes;             // B new-token row copies
  int* bts = (int*)(tok_rows + B * kTokenRowsLds);           // B slices of PB block ids
  int* small = bts + B * PB;                                 // kDecodeSmallLds bytes
  int* ends = small;                                         // [kMaxSeqsPerGroup]
  float* merge_ml = (float*)(small + 16);                    // [B][16][2]
  int* patch_pos = small + 160;                              // [B] new token's block, -1: none
  int* patch_row = small + 168;                              // [B] its row in the block
  int* list_id = small + kDecodeSmallLds / 4;                // B lists of up to lstride entries
  int* list_meta = list_id + B * lstride;

  // 1. Each wave stages its sequence's block-table slice and context end, and writes its
  //    sequence's new token (fused step). The query fragments are loaded here too, so
  //    that their latency passes during the listing.
  const int s = s0 + w;
  const bool writes = owns_new_token(a, ctx, p);
  if (writes && !token_loaded) token = load_new_token<QT, KVT, D>(a, s, g);
  const int end = min(ctx, start + PB * kBlock);
  const int nblk = (end - start + kBlock - 1) / kBlock;
  // The slices keep the block table's names, which decide which tiles the sequences share (a
  // copy-on-write block is private to its sequence); the list names the source instead.
  store_bt_slice(a, s, start / kBlock, nblk, sl, bts + w * PB, CowRead{-1, -1, -1, -1});
  stash_cow(tok_rows + w * kTokenRowsLds, cow_read(a, s, ctx));
  if (lane == 0) {
    ends[w] = end;
    patch_pos[w] = writes && token.written ? (ctx - 1) / kBlock : -1;
    patch_row[w] = (ctx - 1) % kBlock;
  }
  if (writes) stage_new_token<KVT, D>(token, tok_rows + w * kTokenRowsLds);
  const int ncols = B * G;
  const bool col_ok = n < ncols;
  const int cb = col_ok ? n / G : 0;                         // reader (sequence) of column n
  u32x4 qb[D / 32];
  load_q<QT, KVT, D>(a, col_ok, s0 + cb, g * G + (col_ok ? n % G : 0), qb);
  __syncthreads();

  // 2. Each wave lists its share of the logical blocks, every B-th one from index w: for
  //    each, the distinct physical blocks of the B sequences, in logical order, each with
  //    the set of sequences that read it. Interleaving the logical blocks spreads the
  //    blocks only one sequence reads (diverged tails) evenly over the waves. Each wave
  //    then reads the tiles of its own list, so no workgroup barrier is needed between.
  int* my_id = list_id + w * lstride;
  int* my_meta = list_meta + w * lstride;
  int ntiles = 0;
  {
    // The context ends in registers: the list is written to the same LDS allocation, so
    // reading them there would make every entry written wait for a fresh LDS read.
    int endr[kMaxSeqsPerGroup];
#pragma unroll
    for (int b = 0; b < kMaxSeqsPerGroup; ++b) endr[b] = b < B ? ends[b] : 0;
    int npos = 0;
    for (int b = 0; b < B; ++b) npos = max(npos, (endr[b] - start + kBlock - 1) / kBlock);
    for (int i0 = w; i0 < npos; i0 += B * kWave) {
      const int i = i0 + lane * B;
      const int pos = start / kBlock + i;
      int ids_b[kMaxSeqsPerGroup];
      uint32_t live = 0;
#pragma unroll
      for (int b = 0; b < kMaxSeqsPerGroup; ++b) {
        const bool has = b < B && i < npos && pos * kBlock < endr[b];
        ids_b[b] = has ? bts[b * PB + i] : -1;
        live |= has ? (1u << b) : 0u;
      }
      int cnt = 0;
      uint32_t done = 0;
      int e_id[kMaxSeqsPerGroup];
      uint32_t e_readers[kMaxSeqsPerGroup];
#pragma unroll
      for (int b = 0; b < kMaxSeqsPerGroup; ++b) {
        e_id[b] = -1;
        e_readers[b] = 0;
        if (((live >> b) & 1u) && !((done >> b) & 1u)) {
          uint32_t rd = 0;
#pragma unroll
          for (int c = 0; c < kMaxSeqsPerGroup; ++c)
            if (c >= b && ((live >> c) & 1u) && ids_b[c] == ids_b[b]) rd |= 1u << c;
          done |= rd;
          e_id[b] = ids_b[b];
          e_readers[b] = rd;
          ++cnt;
        }
      }
      // Exclusive prefix sum of cnt over the lanes.
      int before = 0, total = 0;
      for (int k = 0; k < B; ++k) {
        const uint64_t bal = __ballot(cnt > k);
        before += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        total += __popcll(bal);
      }
      int e = ntiles + before;
#pragma unroll
      for (int b = 0; b < kMaxSeqsPerGroup; ++b) {
        if (e_readers[b] == 0u) continue;
        int rows = 0;
#pragma unroll
        for (int c = 0; c < kMaxSeqsPerGroup; ++c)
          if ((e_readers[b] >> c) & 1u) rows = max(rows, min(endr[c] - pos * kBlock, kBlock));
        my_id[e] = e_id[b];
        my_meta[e] = pos | (int)(e_readers[b] << 16) | (rows << 24);
        ++e;
      }
      ntiles += total;
    }
  }
  // Copy-on-write: an entry whose only reader has its last block copied names the source.
  // (The pass runs in every step: testing for copy-on-write here would keep its pointer live.)
  wave_lds_sync();
  for (int e = lane; e < ntiles; e += kWave) {
    const int meta = my_meta[e];
    const uint32_t rd = (uint32_t)(meta >> 16) & 0xFFu;
    if (rd != 0u && (rd & (rd - 1u)) == 0u) {
      const CowRead c = stashed_cow(tok_rows + __builtin_ctz(rd) * kTokenRowsLds);
      if (c.src >= 0) my_id[e] = cow_tile(c, meta & 0xFFFF, a.block_shift, my_id[e]);
    }
  }
  wave_lds_sync();

  // 3. The wave's tiles, for all of the group's columns (two tiles in flight, default issue
  //    priority: with every wave listing its own share, the stepped priority of private
  //    streams measured 0.7% slower here).
  State<D> st;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  mfma_tiles<QT, KVT, D, 2, kPolicyStream, false, true, true>(a, g, ntiles, my_id, my_meta, 1, 0, 0, qb,
                                                             col_ok ? (1u << cb) : 0u, col_ok ? ends[cb] : 0,
                                                             tiles + w * Tr::kLdsBytes, st, -1, 0,
                                                             patch_pos, patch_row, tok_rows);
  // Copy-on-write: the source's bytes are requested now and stored after the merge below.
  CowRead cow{-1, -1, -1, -1};
  CowChunks<D> cow_chunks;
  if (writes) {
    cow = stashed_cow(tok_rows + w * kTokenRowsLds);
    cow_copy_begin<KVT, D>(a, g, cow, cow_chunks);
    store_new_token<KVT>(a, token);
  }
  const float l_w = sum_xor32(sum_xor16(st.l));

  // 4. Merge the waves' states column by column (the tile staging area is free again). The
  //    waves share the work: wave w merges and writes the 16-row chunks c of D with
  //    c mod B == w, for every column.
  __syncthreads();
  f32x4* merge_o = (f32x4*)tiles;                            // [B][kPv][64 lanes]
#pragma unroll
  for (int c = 0; c < Tr::kPv; ++c) merge_o[(w * Tr::kPv + c) * kWave + lane] = st.o[c];
  if (j4 == 0) {
    merge_ml[(w * 16 + n) * 2] = st.m;
    merge_ml[(w * 16 + n) * 2 + 1] = l_w;
  }
  __syncthreads();
  if (writes) cow_copy_end<KVT, D>(a, g, cow, cow_chunks);
  if (!col_ok) return;
  float M = -INFINITY;
  for (int v = 0; v < B; ++v) M = fmaxf(M, merge_ml[(v * 16 + n) * 2]);
  float L = 0.f;
  f32x4 o[Tr::kPv];
#pragma unroll
  for (int c = 0; c < Tr::kPv; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int v = 0; v < B; ++v) {
    const float f = exp2_fast(merge_ml[(v * 16 + n) * 2] - M);   // a wave that saw no token: f = 0
    L = fmaf(f, merge_ml[(v * 16 + n) * 2 + 1], L);
#pragma unroll
    for (int c = 0; c < Tr::kPv; ++c)
      if (c % B == w) o[c] += f * merge_o[(v * Tr::kPv + c) * kWave + lane];
  }
  write_column<QT, D>(a, s0 + cb, g * G + n % G, p, o, M, L, w, B);
}

template <int QT, int KVT, int D>
__global__ __launch_bounds__(kWave * kMaxSeqsPerGroup, 2) void paged_decode_mfma(DecodeArgs a) {
  using Tr = MfmaTraits<QT, KVT, D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int j = item_of_workgroup(blockIdx.x, a);
  if (j >= a.num_items) return;
  const Item it = decode_item(j, a);
  const int B = a.seqs_per_group;
  const int w = threadIdx.x / kWave;
  const int start = it.p * a.part_blocks * kBlock;

  // The values the first decisions need are independent loads, issued together (one
  // memory latency rather than a chain): this wave's context length and the block ids at
  // logical block i0 of its sequence and of the sequences on either side, for the group
  // check the same of every sequence of the group (indices clamped into the batch), then
  // the wave's block-table slice and, with one partition (where every item writes its
  // sequence's new token in a fused step), the new token.
  const int i0 = (start / kBlock) >> a.block_shift;   // block of the partition's first tile
  const int max_tokens = (a.max_blocks * kBlock) << a.block_shift;
  const int64_t mb = a.max_blocks;
  const int s = it.s + w;
  const int s_own = min(s, a.num_seqs - 1);
  const int ctx = min(a.context_lens[s_own], max_tokens);
  const int mine = a.block_tables[s_own * mb + i0];
  const int prev = a.block_tables[max(s_own - 1, 0) * mb + i0];
  const int next = a.block_tables[min(s_own + 1, a.num_seqs - 1) * mb + i0];
  int grp_ctx[kMaxSeqsPerGroup], grp_first[kMaxSeqsPerGroup];
#pragma unroll
  for (int b = 0; b < kMaxSeqsPerGroup; ++b) {
    const int sb = min(it.s + b, a.num_seqs - 1);
    grp_ctx[b] = a.context_lens[sb];
    grp_first[b] = a.block_tables[sb * mb + i0];
  }
  BtSlice sl;
  prefetch_bt_slice(a, s_own, start / kBlock, sl);
  const bool token_early = a.new_key != nullptr && a.num_parts == 1;
  TokenChunk token = {};
  if (token_early) token = load_new_token<QT, KVT, D>(a, s_own, it.g);

  // Group mode when every sequence of the group has tokens in this partition and another
  // sequence reads the first sequence's first block of it. Every wave evaluates the same
  // condition, so the whole workgroup takes the same branch.
  if (a.group_mode_ok && it.s + B <= a.num_seqs) {
    bool all_live = true, shares = false;
#pragma unroll
    for (int b = 0; b < kMaxSeqsPerGroup; ++b) {
      if (b < B) {
        all_live = all_live && min(grp_ctx[b], max_tokens) > start;
        if (b > 0) shares = shares || grp_first[b] == grp_first[0];
      }
    }
    if (all_live && shares) {
      mfma_group<QT, KVT, D>(a, it.s, it.g, it.p, start, ctx, sl, token, token_early, smem);
      return;
    }
  }

  // Independent mode: wave w runs sequence it.s + w with its own LDS areas.
  if (s >= a.num_seqs) return;
  const bool writes = owns_new_token(a, ctx, it.p);
  if (writes && !token_early) token = load_new_token<QT, KVT, D>(a, s, it.g);
  if (ctx <= start) {
    if (writes) store_new_token<KVT>(a, token);
    // Nothing in this partition. A whole sequence with no context writes zeros.
    const int n = threadIdx.x & 15, j4 = (threadIdx.x & (kWave - 1)) >> 4;
    if (a.num_parts == 1 && n < a.group) {
      uint16_t* o = (uint16_t*)a.out + ((int64_t)s * a.num_q_heads + it.g * a.group + n) * D;
#pragma unroll
      for (int c = 0; c < Tr::kPv; ++c) *(u32x2*)(o + 16 * c + 4 * j4) = u32x2{0u, 0u};
    }
    return;
  }
  uint8_t* lds = smem + w * Tr::kLdsBytes;
  uint8_t* tok_rows = smem + B * Tr::kLdsBytes + w * kTokenRowsLds;
  int* bt_lds = (int*)(smem + B * (Tr::kLdsBytes + kTokenRowsLds)) + w * a.part_blocks;
  // Does the previous or next sequence of the batch read this sequence's first block?
  const bool shared = (s > 0 && prev == mine) || (s + 1 < a.num_seqs && next == mine);
  if (shared)
    mfma_single<QT, KVT, D, 2, kPolicyCached, false, false>(a, s, it.g, it.p, ctx, start, sl, bt_lds, lds, tok_rows, writes, token);
  else if (a.num_parts > 1)
    mfma_single<QT, KVT, D, 2, kPolicyStream, true, true>(a, s, it.g, it.p, ctx, start, sl, bt_lds, lds, tok_rows, writes, token);
  else
    mfma_single<QT, KVT, D, 1, kPolicyStream, true, true>(a, s, it.g, it.p, ctx, start, sl, bt_lds, lds, tok_rows, writes, token);
}

template <int QT, int KVT, int D>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int grid = decode_grid(a);
  const size_t lds = mfma_decode_lds_bytes(D, a.seqs_per_group, a.part_blocks, a.group_mode_ok != 0);
  hipLaunchKernelGGL((paged_decode_mfma<QT, KVT, D>), dim3(grid), dim3(kWave * a.seqs_per_group), lds, stream, a);
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
