// Paged attention of prefill chunks on gfx950 matrix cores, over an fp8 cache (a 16-bit
// cache is served by the direct-to-LDS kernel in prefill_lds.hip, whose tiles go to LDS
// unchanged; here every tile passes through registers to be widened).
//
// The method (what is computed): long prompts are cut into chunks that run between
// decode steps ("vLLM推理引擎PagedAttention原理与性能优化实战", §六). A chunk of n new
// tokens is the last n positions of its sequence's context; their K/V are already in the
// paged cache, and new token i attends causally to positions 0 .. ctx - n + i through the
// sequence's block table, with ordinary softmax attention ("vLLM 推理优化技术深度调研报告",
// 维度一.3 公式 3-4). Prefill is the compute-bound phase (same page, 公式 5), so here the
// matrix cores carry the work.
//
// How it is computed here (this design is not from the pages):
// * rows of one (sequence, kv head) are its new tokens x the G query heads of the group,
//   token-major; a workgroup of 4 wavefronts takes 128 consecutive rows, 32 per wavefront
//   as two 16-column MFMA blocks, so the K/V tiles it stages in LDS serve every query
//   head of the group;
// * keys are taken 64 at a time (four cache blocks): the workgroup loads the next tile
//   into registers (16-byte loads, each instruction covering one contiguous KiB of a
//   block) while computing on the current one, then stores it to the other half of a
//   double-buffered LDS area as XOR-swizzled 16-byte chunks; one barrier per tile;
// * S^T[16 keys x 16 rows] = K . Q^T on v_mfma_f32_16x16x32 with Q^T held in registers;
//   O^T[16 d x 16 rows] += V^T . P^T on v_mfma_f32_16x16x32 over 32 keys, with V^T read by
//   ds_read_b64_tr_b16. The contraction runs over keys (4j4..4j4+3 of one 16-key tile,
//   then the same of the next), the order in which the score accumulators already hold P,
//   so softmax weights never leave their lanes;
// * online softmax in fp32 with exp2 (log2 e folded into the scale); the causal limit of
//   each row is applied by select only on tiles that reach past the wavefront's first
//   row's limit; a wavefront skips tiles wholly past its last row;
// * V rows past the workgroup's last key are zeroed when staged (0 * stale NaN would
//   poison the product); the fp8 (OCP E4M3FN) cache is widened exactly to the q dtype as
//   it is staged, its per-tensor scales folded into the logit and output scales;
// * work items are ordered kv head, sequence (the most work first), row tile (last rows
//   first: they see the most keys), and each XCD takes a contiguous range of them, so the
//   row tiles of one (sequence, kv head) run on one XCD and re-read its K/V from that
//   XCD's L2, and the longest items start first.
#include "prefill_common.h"

namespace pkv {

template <int KVT, int D>
struct PrefillTraits {
  static_assert(KVT == kFP8, "16-bit caches use the direct-to-LDS kernel");
  static constexpr int kThreads = kWave * kPrefillWaves;
  static constexpr int kElem = 1;                                  // bytes per cache element
  static constexpr int kBlockBytes = kBlock * D * kElem;           // one kv head's slice of a 16-token tile
  static constexpr int kChunksPerBlock = kBlockBytes / 16;
  static constexpr int kLoads = kPrefillKeys * D * kElem / 16 / kThreads;  // per thread, K (or V)
  // LDS rows are padded rather than swizzled, so that every operand read is a per-lane
  // base plus an immediate offset. K rows (read 16 bytes per lane, 8 rows per bank
  // cycle) step 4 banks; V rows (read transposed, 4 rows x 32 bytes per bank cycle) step
  // 8 banks.
  static constexpr int kKRow = D * 2 + 16;
  static constexpr int kVRow = D * 2 + 32;
  static constexpr int kKTile = kPrefillKeys * kKRow;
  static constexpr int kVTile = kPrefillKeys * kVRow;
  static_assert(kChunksPerBlock % kWave == 0, "a wavefront's loads stay inside one block");
  static_assert(kLoads >= 1, "every thread loads");
};

template <int QT, int KVT, int D>
__global__ __launch_bounds__(kWave * kPrefillWaves, 2) void paged_prefill_mfma(const PrefillArgs a) {
  using Tr = PrefillTraits<KVT, D>;
  constexpr int NCB = kPrefillCols / 16;   // 16-column MFMA blocks per wavefront
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][Tr::kKTile + Tr::kVTile];   // [buffer]: K tile, V tile
  __shared__ __attribute__((aligned(16))) int ids_lds[kIdsRing];

  // ---- work item ----------------------------------------------------------------------
  const int nb = gridDim.x;                       // a multiple of 8
  const int item = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (item >= a.num_items) return;
  const int pair = item / a.row_tiles;
  const int tile = a.row_tiles - 1 - item % a.row_tiles;
  const int g = pair / a.num_seqs, s = seq_of_rank(a, pair % a.num_seqs, ids_lds);
  const int G = a.group;

  const int shift = a.block_shift;   // a cache block holds kBlock << shift tokens, walked in kBlock-token tiles
  const int ctx = min(max(a.context_lens[s], 0), (a.max_blocks * kBlock) << shift);
  const int q0 = a.query_start_loc[s], q1 = a.query_start_loc[s + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.num_tokens) return;
  const int n = min(min(q1 - q0, a.max_query_len), ctx);
  const int R = n * G;
  const int row0 = tile * kPrefillRows;
  if (row0 >= R) return;
  const int prefix = ctx - n;
  const int kv_end = prefix + (min(R, row0 + kPrefillRows) - 1) / G + 1;   // keys the workgroup needs
  const int ntiles = (kv_end + kBlock - 1) / kBlock;   // 16-token tiles the workgroup reads
  const int n_iter = (kv_end + kPrefillKeys - 1) / kPrefillKeys;

  const int t = threadIdx.x, w = readfirstlane(t / kWave), lane = t & (kWave - 1);
  __builtin_assume(w >= 0 && w < kPrefillWaves);
  const int n16 = lane & 15, j4 = lane >> 4;

  // ---- this wavefront's rows: Q^T operands and causal limits ------------------------------
  const int wrow0 = row0 + w * kPrefillCols;
  u32x4 qb[NCB][D / 32];
  int limit[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int r = wrow0 + cb * 16 + n16;
    const bool valid = r < R;
    const int tok = valid ? r / G : 0, h = valid ? r % G : 0;
    limit[cb] = valid ? prefix + tok + 1 : 0;
    const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)(q0 + tok) * a.q_token_stride + (int64_t)(g * G + h) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      qb[cb][c] = valid ? *(const u32x4*)(qrow + 32 * c + 8 * j4) : u32x4{0u, 0u, 0u, 0u};
  }
  const bool wave_live = wrow0 < R;
  const int wave_lo = wave_live ? prefix + wrow0 / G + 1 : 0;                      // first row's limit
  const int wave_hi = wave_live ? prefix + (min(R, wrow0 + kPrefillCols) - 1) / G + 1 : 0;   // last row's

  // ---- K/V tiles: global -> registers -> LDS ----------------------------------------------
  const int64_t head_stride = (int64_t)Tr::kBlockBytes << shift;   // one kv head's slice of a block
  const uint8_t* kbase = (const uint8_t*)a.k_cache + (int64_t)g * head_stride;
  const uint8_t* vbase = (const uint8_t*)a.v_cache + (int64_t)g * head_stride;
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;

  // The positions of the 16-token tiles (tile_position of their names; -1 past the last
  // tile or for a block id out of the pool) are staged in an LDS ring of kIdsRing entries,
  // refilled by the whole workgroup when the walk reaches its end. A key tile's four names
  // are read from the ring one iteration before its loads are issued.
  auto fill_ids = [&](int first) {   // tiles [first, first + kIdsRing); first is a multiple of kIdsRing
    for (int k = t; k < kIdsRing; k += Tr::kThreads)
      ids_lds[k] = first + k < ntiles
                       ? tile_position(tile_name(bt, first + k, shift, a.num_blocks), shift, a.num_kv_heads)
                       : -1;
  };
  auto read_ids = [&](int i) -> u32x4 {   // ids of tile i's four blocks (same address in every lane)
    return *(const u32x4*)(ids_lds + ((i * (kPrefillKeys / kBlock)) & (kIdsRing - 1)));
  };

  // Two register sets: even tiles in A, odd tiles in B. Tile i + 2 is loaded while tile i
  // is multiplied and tile i + 1 is staged, so a load has two tiles' time to arrive.
  // Loads are issued for every tile, past the last one too (as zero-length loads), so that
  // the count of loads in flight is the same on every path.
  u32x4 rk_a[Tr::kLoads], rv_a[Tr::kLoads], rk_b[Tr::kLoads], rv_b[Tr::kLoads];
  // Load u of thread t covers 16-byte chunk f = u * threads + t of the tile; its block
  // (0..3) is the same for the whole wavefront.
  auto load_tile = [&](const u32x4 ids, u32x4* rk, u32x4* rv) {
    const int id0 = readfirstlane((int)ids[0]), id1 = readfirstlane((int)ids[1]);
    const int id2 = readfirstlane((int)ids[2]), id3 = readfirstlane((int)ids[3]);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      const int j = (u * Tr::kThreads + w * kWave) / Tr::kChunksPerBlock;
      const int id = j == 0 ? id0 : j == 1 ? id1 : j == 2 ? id2 : id3;
      const bool live = id >= 0;                                    // ids are tile positions
      const int64_t off = live ? (int64_t)id * Tr::kBlockBytes : 0;
      const uint32_t bytes = live ? (uint32_t)Tr::kBlockBytes : 0u;   // 0: loads return zeros
      const uint32_t c16 = (uint32_t)((u * Tr::kThreads + t) % Tr::kChunksPerBlock) * 16;
      rk[u] = buf_load16<kPolicyCached>(make_rsrc(kbase + off, bytes), c16);
      rv[u] = buf_load16<kPolicyCached>(make_rsrc(vbase + off, bytes), c16);
    }
  };
  // LDS row r of a tile holds key r of the tile as 16-bit values. V rows at or past
  // kv_end are stored as zeros.
  auto stage_tile = [&](int i, int buf, const u32x4* rk, const u32x4* rv) {
    uint8_t* kl = lds[buf];
    uint8_t* vl = lds[buf] + Tr::kKTile;
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      const int f = u * Tr::kThreads + t;
      const int j = f / Tr::kChunksPerBlock, c = f % Tr::kChunksPerBlock;
      {
        const int r = j * kBlock + c / (D / 16), ch = c % (D / 16);   // 16 codes = 2 LDS chunks
        const u32x4 wk = rk[u];
        const u32x4 wv = i * kPrefillKeys + r < kv_end ? rv[u] : u32x4{0u, 0u, 0u, 0u};
        const u32x2 k0 = fp8x4_to_16<QT>(wk[0]), k1 = fp8x4_to_16<QT>(wk[1]);
        const u32x2 k2 = fp8x4_to_16<QT>(wk[2]), k3 = fp8x4_to_16<QT>(wk[3]);
        const u32x2 v0 = fp8x4_to_16<QT>(wv[0]), v1 = fp8x4_to_16<QT>(wv[1]);
        const u32x2 v2 = fp8x4_to_16<QT>(wv[2]), v3 = fp8x4_to_16<QT>(wv[3]);
        uint8_t* kd = kl + r * Tr::kKRow + ch * 32;
        uint8_t* vd = vl + r * Tr::kVRow + ch * 32;
        *(u32x4*)(kd) = u32x4{k0[0], k0[1], k1[0], k1[1]};
        *(u32x4*)(kd + 16) = u32x4{k2[0], k2[1], k3[0], k3[1]};
        *(u32x4*)(vd) = u32x4{v0[0], v0[1], v1[0], v1[1]};
        *(u32x4*)(vd + 16) = u32x4{v2[0], v2[1], v3[0], v3[1]};
      }
    }
  };

  // ---- running softmax state: per lane, column n16 of each block, rows 4j4.. of each d-tile
  // m: a row's reference point (log2 units), m_ref: the one exponents are taken against
  // (0 while m = -inf), m_bound = m + kLazyRescale.
  f32x4 o[NCB][D / 16];
  float m[NCB], m_ref[NCB], m_bound[NCB], l[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) o[cb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[cb] = -INFINITY;
    m_ref[cb] = 0.f;
    m_bound[cb] = -INFINITY;
    l[cb] = 0.f;
  }
  const float qk_scale = a.qk_scale_log2;

  // Per-lane LDS bases: K fragment (row n16, elements 8j4..), V^T fragment (rows 4j4 +
  // n16/4, elements 4 (n16 & 3)..).
  const int k_lane = n16 * Tr::kKRow + j4 * 16;
  const int v_lane = (4 * j4 + (n16 >> 2)) * Tr::kVRow + (n16 & 3) * 8;

  // Per tile: all of QK^T, then the causal select, then each column's new reference
  // maximum (one branch for the rare rescale), then the exponentials of the first 32 keys,
  // the PV products of the first 32 keys (independent of the exponentials of the last 32,
  // so the two can overlap in one straight-line block), and the last 32 keys.
  auto compute = [&](int i, int buf) {
    const uint8_t* kl = lds[buf] + k_lane;
    const uint8_t* vl = lds[buf] + Tr::kKTile + v_lane;
    const int k0 = i * kPrefillKeys;
    // S^T = K . Q^T for the four 16-key tiles. A wavefront in a matrix-core phase runs at
    // a raised issue priority, so the two wavefronts of a SIMD drift into complementary
    // phases (one multiplying while the other computes exponentials).
    __builtin_amdgcn_s_setprio(1);
    f32x4 sc[4][NCB];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) sc[kt][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 ka = *(const u32x4*)(kl + kt * 16 * Tr::kKRow + c * 64);   // elements 32c + 8j4 .. + 7
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) sc[kt][cb] = mfma16x16x32<QT>(ka, qb[cb][c], sc[kt][cb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // Causal limits (and keys past the workgroup's last one) on tiles that reach them.
    if (k0 + kPrefillKeys > wave_lo) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (k0 + kt * 16 + 4 * j4 + e >= limit[cb]) sc[kt][cb][e] = -INFINITY;
    }
    // Lazy rescaling: the reference point m of a column moves only when a score exceeds it
    // by more than kLazyRescale (log2 units), so weights stay below 2^8 and the
    // accumulators are rescaled rarely. Any reference gives the same quotient. Each lane
    // tests its own sixteen scores of the column; only a wavefront where some test fires
    // takes the column maxima across lanes and rescales (columns whose reference stays
    // put get a factor of 1).
    float lmax[NCB];
    bool over = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // (scores are never NaN here: stale rows were replaced by -inf above)
      const float m0 = max3_nn(sc[0][cb][0], sc[0][cb][1], sc[0][cb][2]);
      const float m1 = max3_nn(sc[0][cb][3], sc[1][cb][0], sc[1][cb][1]);
      const float m2 = max3_nn(sc[1][cb][2], sc[1][cb][3], sc[2][cb][0]);
      const float m3 = max3_nn(sc[2][cb][1], sc[2][cb][2], sc[2][cb][3]);
      const float m4 = max3_nn(sc[3][cb][0], sc[3][cb][1], sc[3][cb][2]);
      lmax[cb] = max_nn(max3_nn(m0, m1, m2), max3_nn(m3, m4, sc[3][cb][3]));
      over = over || lmax[cb] * qk_scale > m_bound[cb];   // the scale is positive
    }
    if (__any(over)) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float mx = max_nn_xor32(max_nn_xor16(lmax[cb])) * qk_scale;
        const float m_new = mx > m_bound[cb] ? mx : m[cb];
        const float alpha = m[cb] == m_new ? 1.0f : exp2_fast(m[cb] - m_new);   // exp2(-inf) = 0
        m[cb] = m_new;
        // A column that has seen no live key keeps m = -inf; exponents are then taken
        // against 0 so that they come out as exp2(-inf) = 0, never as exp2(-inf + inf).
        m_ref[cb] = m_new == -INFINITY ? 0.f : m_new;
        m_bound[cb] = m_new + kLazyRescale;
        l[cb] *= alpha;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) o[cb][c] *= alpha;
      }
    }
    // P^T of 32 keys (16-key tiles 2hf, 2hf + 1) as the B operands of one PV step; the
    // denominator sums the rounded weights that the PV product uses.
    auto weights = [&](int hf, u32x4* pb) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f32x4 a = sc[2 * hf][cb], b = sc[2 * hf + 1][cb];
        const float r = m_ref[cb];
        const uint32_t p0 = pack2<QT>(exp2_fast(fmaf(a[0], qk_scale, -r)), exp2_fast(fmaf(a[1], qk_scale, -r)));
        const uint32_t p1 = pack2<QT>(exp2_fast(fmaf(a[2], qk_scale, -r)), exp2_fast(fmaf(a[3], qk_scale, -r)));
        const uint32_t p2 = pack2<QT>(exp2_fast(fmaf(b[0], qk_scale, -r)), exp2_fast(fmaf(b[1], qk_scale, -r)));
        const uint32_t p3 = pack2<QT>(exp2_fast(fmaf(b[2], qk_scale, -r)), exp2_fast(fmaf(b[3], qk_scale, -r)));
        l[cb] = dot2_ones<QT>(p3, dot2_ones<QT>(p2, dot2_ones<QT>(p1, dot2_ones<QT>(p0, l[cb]))));
        pb[cb] = u32x4{p0, p1, p2, p3};
      }
    };
    // O^T += V^T . P^T over the 32 keys of step hf.
    auto pv = [&](int hf, const u32x4* pb) {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const uint8_t* va_p = vl + hf * 32 * Tr::kVRow + c * 32;
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)va_p);
        const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(va_p + 16 * Tr::kVRow));
        const u32x2 wa = __builtin_bit_cast(u32x2, va), wb = __builtin_bit_cast(u32x2, vb);
        const u32x4 av = {wa[0], wa[1], wb[0], wb[1]};
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[cb][c] = mfma16x16x32<QT>(av, pb[cb], o[cb][c]);
      }
    };
    u32x4 pb0[NCB], pb1[NCB];
    weights(0, pb0);
    __builtin_amdgcn_s_setprio(1);
    pv(0, pb0);
    __builtin_amdgcn_s_setprio(0);
    weights(1, pb1);
    __builtin_amdgcn_s_setprio(1);
    pv(1, pb1);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- main loop: one tile in LDS, the next two in flight ------------------------------
  // ids: the block ids of tile i + 2 on entry; ld: registers that receive tile i + 2;
  // st: registers that hold tile i + 1.
  auto iteration = [&](int i, u32x4& ids, u32x4* ld_k, u32x4* ld_v, const u32x4* st_k, const u32x4* st_v) {
    load_tile(ids, ld_k, ld_v);
    if (i * kPrefillKeys < wave_hi) compute(i, i & 1);
    if (((i + 3) * (kPrefillKeys / kBlock)) % kIdsRing == 0) {   // the ring moves on (all waves)
      fill_ids((i + 3) * (kPrefillKeys / kBlock));
      __syncthreads();
    }
    ids = read_ids(i + 3);
    if (i + 1 < n_iter) stage_tile(i + 1, (i + 1) & 1, st_k, st_v);
    __syncthreads();
  };
  fill_ids(0);
  __syncthreads();
  u32x4 ids = read_ids(0);
  load_tile(ids, rk_a, rv_a);
  ids = read_ids(1);
  load_tile(ids, rk_b, rv_b);
  ids = read_ids(2);
  stage_tile(0, 0, rk_a, rv_a);
  __syncthreads();
  for (int i = 0; i < n_iter; i += 2) {
    iteration(i, ids, rk_a, rv_a, rk_b, rv_b);
    if (i + 1 < n_iter) iteration(i + 1, ids, rk_b, rv_b, rk_a, rv_a);
  }

  // ---- results ----------------------------------------------------------------------------
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float l_tot = sum_xor32(sum_xor16(l[cb]));
    const int r = wrow0 + cb * 16 + n16;
    if (r < R) {
      const int tok = r / G, h = r % G;
      const float inv = a.v_scale / l_tot;
      uint16_t* orow = (uint16_t*)a.out + ((int64_t)(q0 + tok) * a.num_q_heads + g * G + h) * D;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const f32x4 v = o[cb][c] * inv;
        *(u32x2*)(orow + 16 * c + 4 * j4) = u32x2{pack2<QT>(v[0], v[1]), pack2<QT>(v[2], v[3])};
      }
    }
  }
}

template <int QT, int KVT, int D>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int grid = (a.num_items + 7) / 8 * 8;
  hipLaunchKernelGGL((paged_prefill_mfma<QT, KVT, D>), dim3(grid), dim3(kWave * kPrefillWaves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int q_type, int kv_type, int head_dim, hipStream_t stream) {
#define PKV_CASE(QT, KVT, D) \
  if (q_type == QT && kv_type == KVT && head_dim == D) return launch_t<QT, KVT, D>(a, stream);
  PKV_CASE(kBF16, kFP8, 128) PKV_CASE(kBF16, kFP8, 64)
  PKV_CASE(kF16, kFP8, 128) PKV_CASE(kF16, kFP8, 64)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
