// Paged attention of prefill chunks over a 16-bit cache, with K/V loaded straight into LDS.
//
// What is computed is the same as the register-staged prefill kernel (prefill_mfma.hip;
// "vLLM推理引擎PagedAttention原理与性能优化实战", §六 and "vLLM 推理优化技术深度调研报告",
// 维度一.3 公式 3-5): each sequence's chunk of new tokens attends causally to its paged
// context. This kernel is the one used when the cache holds the q dtype (no widening on
// the way in). How it differs from the register-staged one:
// * K and V tiles of 32 keys (two 16-token tiles) go from HBM/L2 to LDS with buffer loads
//   that write LDS directly (buffer_load_dwordx4 ... lds): no registers hold tiles in
//   flight, so a wavefront fits 168 VGPRs and a CU holds three workgroups (three
//   wavefronts per SIMD) instead of two;
// * three LDS stages: tile i + 2 is loaded while tile i is multiplied; the wait before a
//   tile is used is an explicit counter wait that leaves the next tile's loads in flight,
//   followed by one barrier;
// * a wavefront's load instruction fills one contiguous KiB of LDS (lane l at +16 l), so
//   rows are not padded; bank conflicts are avoided by XOR-swizzling 16-byte chunks within
//   a row, applied on the global side (each lane loads the chunk that belongs at its LDS
//   position): K chunk k of row r sits at k ^ (r mod chunks per row); V uses a swizzle
//   under which the four rows a transposed read touches fall in distinct banks;
// * the stages are three distinct LDS arrays and the loop is unrolled by three, so every
//   access names its stage at compile time: the compiler, which tracks loads into LDS per
//   LDS variable, then makes a read of one stage wait only for that stage's loads;
// * key rows past the workgroup's last key are loaded as zeros by the buffer range check
//   (their lanes get an offset past the buffer), tiles outside the pool likewise.
// QK^T and PV on v_mfma_f32_16x16x32 with V^T read by ds_read_b64_tr_b16, online softmax
// with lazy rescaling and the causal select are as in the register-staged kernel.
#include <type_traits>

#include "prefill_common.h"

namespace pkv {

template <int S>
using Stage = std::integral_constant<int, S>;

using lds_ptr = __attribute__((address_space(3))) void*;

// 16 bytes per lane from a buffer straight into LDS: lane l writes lds + 16 l (the LDS
// base is wave-uniform). Out-of-range offsets write zeros. The builtin exists only for
// the device; in the host pass, which only emits the kernel's launch stub, the body is
// empty (the builtin there would silently drop the stub).
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, lds_ptr dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
#endif
}

constexpr int kLdsKeys = 32;    // keys per LDS stage (two 16-token tiles)
constexpr int kLdsStages = 3;

template <int D, int W>
struct LdsTraits {
  static constexpr int kThreads = kWave * W;
  static constexpr int kRow = D * 2;                         // bytes of one 16-bit row
  static constexpr int kRowChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kTile16 = kBlock * kRow;              // one kv head's slice of a 16-token tile
  static constexpr int kStageTile = kLdsKeys * kRow;         // K (or V) part of a stage
  static constexpr int kLoads = kStageTile / 16 / kThreads;  // direct-to-LDS loads per thread, K (or V)
  static constexpr int kRowsPerLoad = kWave * 16 / kRow;     // rows one wavefront instruction fills
  static_assert(kLoads >= 1 && kStageTile % (16 * kThreads) == 0, "whole instructions per stage");
  static_assert(kBlock % kRowsPerLoad == 0, "an instruction stays inside one 16-token tile");
};

// Swizzles (chunk index XOR a function of the row): K rows are read 16 bytes per lane, 8
// rows of one chunk column per bank cycle; V rows are read transposed, 4 rows x 2 adjacent
// chunks per 16 lanes.
template <int RC>
__device__ __forceinline__ int k_swz(int r) { return r & (RC - 1); }
template <int RC>
__device__ __forceinline__ int v_swz(int r) {
  return RC >= 16 ? ((2 * (r & 3)) ^ (8 * ((r >> 2) & 1))) : 2 * (r & 3);
}

template <int QT, int D, int W>
__global__ __launch_bounds__(kWave * W, 3) void paged_prefill_lds(const PrefillArgs a) {
  using Tr = LdsTraits<D, W>;
  constexpr int kRows = W * kPrefillCols;   // query rows of a workgroup
  constexpr int RC = Tr::kRowChunks;
  constexpr int NCB = kPrefillCols / 16;
  constexpr int kStageBytes = 2 * Tr::kStageTile;
  // stage: K tile, V tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds_st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_st1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_st2[kStageBytes];
  auto stage = [&](auto stg) -> uint8_t* {
    if constexpr (decltype(stg)::value == 0) return lds_st0;
    else if constexpr (decltype(stg)::value == 1) return lds_st1;
    else return lds_st2;
  };
  __shared__ __attribute__((aligned(16))) int ids_lds[kIdsRing];

  // ---- work item (as in the register-staged kernel) -------------------------------------
  const int nb = gridDim.x;
  const int item = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (item >= a.num_items) return;
  const int pair = item / a.row_tiles;
  const int tile = a.row_tiles - 1 - item % a.row_tiles;
  const int g = pair / a.num_seqs, s = seq_of_rank(a, pair % a.num_seqs, ids_lds);
  const int G = a.group;
  const int shift = a.block_shift;
  const int ctx = min(max(a.context_lens[s], 0), (a.max_blocks * kBlock) << shift);
  const int q0 = a.query_start_loc[s], q1 = a.query_start_loc[s + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.num_tokens) return;
  const int n = min(min(q1 - q0, a.max_query_len), ctx);
  const int R = n * G;
  const int row0 = tile * kRows;
  if (row0 >= R) return;
  const int prefix = ctx - n;
  const int kv_end = prefix + (min(R, row0 + kRows) - 1) / G + 1;
  const int ntiles = (kv_end + kBlock - 1) / kBlock;
  const int n_iter = (kv_end + kLdsKeys - 1) / kLdsKeys;

  const int t = threadIdx.x, w = readfirstlane(t / kWave), lane = t & (kWave - 1);
  __builtin_assume(w >= 0 && w < W);
  const int n16 = lane & 15, j4 = lane >> 4;

  // ---- this wavefront's rows ---------------------------------------------------------------
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
  const int wave_lo = wave_live ? prefix + wrow0 / G + 1 : 0;
  const int wave_hi = wave_live ? prefix + (min(R, wrow0 + kPrefillCols) - 1) / G + 1 : 0;

  // ---- tile names and direct-to-LDS loads ----------------------------------------------------
  const int64_t head_stride = (int64_t)Tr::kTile16 << shift;
  const uint8_t* kbase = (const uint8_t*)a.k_cache + (int64_t)g * head_stride;
  const uint8_t* vbase = (const uint8_t*)a.v_cache + (int64_t)g * head_stride;
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  auto position = [&](int tt) {   // of 16-token tile tt of the context, or -1
    return tt < ntiles ? tile_position(tile_name(bt, tt, shift, a.num_blocks), shift, a.num_kv_heads) : -1;
  };
  auto fill_ids = [&](int first) {   // positions of 16-token tiles [first, first + kIdsRing)
    for (int k = t; k < kIdsRing; k += Tr::kThreads) ids_lds[k] = position(first + k);
  };
  auto read_ids = [&](int i) -> u32x2 {   // the two 16-token tiles of stage tile i
    return *(const u32x2*)(ids_lds + ((i * (kLdsKeys / kBlock)) & (kIdsRing - 1)));
  };
  // Lane l of load u of wavefront w fills LDS bytes [1024 (u W + w) + 16 l, +16) of a K (or
  // V) stage tile: row rr, chunk position pc; it loads the chunk that the swizzle puts there.
  uint32_t koff[Tr::kLoads], voff[Tr::kLoads];
  int rrow[Tr::kLoads];
#pragma unroll
  for (int u = 0; u < Tr::kLoads; ++u) {
    const int o = (u * W + w) * 1024 + lane * 16;
    const int rr = o / Tr::kRow, pc = (o % Tr::kRow) / 16;
    rrow[u] = rr;
    koff[u] = (uint32_t)((rr % kBlock) * Tr::kRow + (pc ^ k_swz<RC>(rr)) * 16);
    voff[u] = (uint32_t)((rr % kBlock) * Tr::kRow + (pc ^ v_swz<RC>(rr)) * 16);
  }
  auto issue_loads = [&](auto stg, int i, u32x2 ids) {   // stage tile i into stage stg
    uint8_t* st = stage(stg);
#pragma unroll
    for (int u = 0; u < Tr::kLoads; ++u) {
      const int sub = ((u * W + w) * 1024) / Tr::kRow / kBlock;   // 16-token tile of this instruction
      const int id = readfirstlane((int)(sub == 0 ? ids[0] : ids[1]));   // tile position
      const bool live = id >= 0;
      const int64_t off = live ? (int64_t)id * Tr::kTile16 : 0;
      const uint32_t bytes = live ? (uint32_t)Tr::kTile16 : 0u;
      // rows past the workgroup's last key load as zeros (offset past the buffer)
      const bool row_live = i * kLdsKeys + rrow[u] < kv_end;
      uint8_t* dk = st + (u * W + w) * 1024;
      buf_load_lds16(make_rsrc(kbase + off, bytes), (lds_ptr)dk, row_live ? koff[u] : 0x80000000u);
      buf_load_lds16(make_rsrc(vbase + off, bytes), (lds_ptr)(dk + Tr::kStageTile), row_live ? voff[u] : 0x80000000u);
    }
  };

  // ---- running softmax state ---------------------------------------------------------------
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
  // Per-lane LDS operand offsets: K fragment (row n16 of a 16-key tile, chunk 4c + j4),
  // V^T fragment (rows 4 j4 + n16 / 4, chunk 2c + (n16 & 3) / 2, half n16 & 1).
  uint32_t kadr[D / 32], vadr[D / 16];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) kadr[c] = n16 * Tr::kRow + (((4 * c + j4) ^ k_swz<RC>(n16)) * 16);
  {
    const int vr = 4 * j4 + (n16 >> 2);
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      vadr[c] = vr * Tr::kRow + (((2 * c + ((n16 & 3) >> 1)) ^ v_swz<RC>(vr)) * 16) + (n16 & 1) * 8;
  }

  auto compute = [&](auto stg, int i) {   // stage tile i, held in stage stg
    const uint8_t* kl = stage(stg);
    const uint8_t* vl = kl + Tr::kStageTile;
    const int k0 = i * kLdsKeys;
    __builtin_amdgcn_s_setprio(1);
    f32x4 sc[2][NCB];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) sc[kt][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 ka = *(const u32x4*)(kl + kt * kBlock * Tr::kRow + kadr[c]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) sc[kt][cb] = mfma16x16x32<QT>(ka, qb[cb][c], sc[kt][cb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (k0 + kLdsKeys > wave_lo) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (k0 + kt * 16 + 4 * j4 + e >= limit[cb]) sc[kt][cb][e] = -INFINITY;
    }
    // Lazy rescaling: a row's reference point moves only when one of its scores exceeds it
    // by more than kLazyRescale (log2 units). Each lane tests its own eight scores of the
    // row; only a wavefront where some test fires takes the row maxima across lanes and
    // rescales (rows whose reference stays put get a factor of 1).
    float lmax[NCB];
    bool over = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const f32x4 x = sc[0][cb], y = sc[1][cb];
      const float mx = max3_nn(max3_nn(x[0], x[1], x[2]), max3_nn(x[3], y[0], y[1]), max_nn(y[2], y[3]));
      lmax[cb] = mx;
      over = over || mx * qk_scale > m_bound[cb];   // the scale is positive
    }
    if (__any(over)) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float mx = max_nn_xor32(max_nn_xor16(lmax[cb])) * qk_scale;
        const float m_new = mx > m_bound[cb] ? mx : m[cb];
        const float alpha = m[cb] == m_new ? 1.0f : exp2_fast(m[cb] - m_new);   // exp2(-inf) = 0
        m[cb] = m_new;
        m_ref[cb] = m_new == -INFINITY ? 0.f : m_new;
        m_bound[cb] = m_new + kLazyRescale;
        l[cb] *= alpha;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) o[cb][c] *= alpha;
      }
    }
    u32x4 pb[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const f32x4 x = sc[0][cb], y = sc[1][cb];
      const float r = m_ref[cb];
      const uint32_t p0 = pack2<QT>(exp2_fast(fmaf(x[0], qk_scale, -r)), exp2_fast(fmaf(x[1], qk_scale, -r)));
      const uint32_t p1 = pack2<QT>(exp2_fast(fmaf(x[2], qk_scale, -r)), exp2_fast(fmaf(x[3], qk_scale, -r)));
      const uint32_t p2 = pack2<QT>(exp2_fast(fmaf(y[0], qk_scale, -r)), exp2_fast(fmaf(y[1], qk_scale, -r)));
      const uint32_t p3 = pack2<QT>(exp2_fast(fmaf(y[2], qk_scale, -r)), exp2_fast(fmaf(y[3], qk_scale, -r)));
      l[cb] = dot2_ones<QT>(p3, dot2_ones<QT>(p2, dot2_ones<QT>(p1, dot2_ones<QT>(p0, l[cb]))));
      pb[cb] = u32x4{p0, p1, p2, p3};
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vl + vadr[c]));
      const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vl + kBlock * Tr::kRow + vadr[c]));
      const u32x2 wa = __builtin_bit_cast(u32x2, va), wb = __builtin_bit_cast(u32x2, vb);
      const u32x4 av = {wa[0], wa[1], wb[0], wb[1]};
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[cb][c] = mfma16x16x32<QT>(av, pb[cb], o[cb][c]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- main loop ------------------------------------------------------------------------------
  // Every stage tile's loads are issued, past the last one too (as zero-length loads), so
  // each thread always has the next tile's kLoads * 2 loads in flight when it waits.
  constexpr int kPerTile = 2 * Tr::kLoads;
  static_assert(kPerTile <= 63, "the counter wait below names the loads left in flight");
  fill_ids(0);
  __syncthreads();
  issue_loads(Stage<0>{}, 0, read_ids(0));
  issue_loads(Stage<1>{}, 1, read_ids(1));
  // Stage tile 2's positions come from the table itself: a read of the ring here would be
  // merged with the one at the end of the loop into a single read through a pointer the
  // compiler can no longer tie to the ring, and it would then wait for every load in flight.
  u32x2 ids = {(uint32_t)position(4), (uint32_t)position(5)};
  // Stage tile i sits in stage i mod 3; tile i + 2 goes into the stage read at i - 1.
  auto iteration = [&](auto stg, int i) {
    constexpr int S = decltype(stg)::value;
    // Tile i has landed once only tile i + 1's loads are left (vmcnt counts in order);
    // every wavefront's own LDS reads of earlier tiles have returned (lgkmcnt 0).
    __builtin_amdgcn_s_waitcnt((kPerTile & 15) | ((kPerTile >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    issue_loads(Stage<(S + 2) % kLdsStages>{}, i + 2, ids);
    if (i * kLdsKeys < wave_hi) compute(stg, i);
    const int first = (i + 3) * (kLdsKeys / kBlock);
    if (first % kIdsRing == 0) {   // the ring moves on (all waves)
      __syncthreads();
      fill_ids(first);
      __syncthreads();
    }
    ids = read_ids(i + 3);
  };
  // Whole rounds of three: an iteration past the last tile computes nothing and issues
  // zero-length loads, and every round has the same pattern of loads, which lets the
  // compiler see that each stage's last loads are two tiles old when it is read.
  static_assert(kLdsStages == 3, "the loop below is unrolled by the stage count");
  for (int i = 0; i < n_iter; i += 3) {
    iteration(Stage<0>{}, i);
    iteration(Stage<1>{}, i + 1);
    iteration(Stage<2>{}, i + 2);
  }

  // ---- results --------------------------------------------------------------------------------
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
  // Loads of the two tiles past the end are still in flight; the workgroup's LDS must
  // outlive them.
  __builtin_amdgcn_s_waitcnt((0 & 15) | (0 << 14) | (0x7 << 4) | (0xF << 8));
}

// Four wavefronts (128 query rows, the host's row tiles) per workgroup, three workgroups
// per CU. (Eight wavefronts share each tile among twice the rows but leave room for only
// two wavefronts per SIMD, which measured slower.)
template <int QT, int D>
static hipError_t launch_lds(const PrefillArgs& a, hipStream_t stream) {
  constexpr int W = kPrefillWaves;
  static_assert(W * kPrefillCols == kPrefillRows, "row tiles as the host counts them");
  const int grid = (a.num_items + 7) / 8 * 8;
  hipLaunchKernelGGL((paged_prefill_lds<QT, D, W>), dim3(grid), dim3(kWave * W), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_lds(const PrefillArgs& a, int q_type, int head_dim, hipStream_t stream) {
  if (q_type == kBF16 && head_dim == 128) return launch_lds<kBF16, 128>(a, stream);
  if (q_type == kBF16 && head_dim == 64) return launch_lds<kBF16, 64>(a, stream);
  if (q_type == kF16 && head_dim == 128) return launch_lds<kF16, 128>(a, stream);
  if (q_type == kF16 && head_dim == 64) return launch_lds<kF16, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
