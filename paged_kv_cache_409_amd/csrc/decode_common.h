// Parameters and helpers shared by the paged decode-attention kernels.
#pragma once

#include "pkv_device.h"

namespace pkv {

// One launch of the decode main kernel. Work item = (sequence, kv head, context
// partition); one wavefront per item.
struct DecodeArgs {
  void* out;                      // [S, Hq, D] q dtype (written when num_parts == 1)
  const void* q;                  // [S, Hq, D] q dtype, sequence stride q_seq_stride elements
  const void* k_cache;            // [NB, Hkv, 16, D]
  const void* v_cache;            // [NB, Hkv, 16, D]
  const int32_t* block_tables;    // [S, max_blocks]
  const int32_t* context_lens;    // [S]
  float* part_ml;                 // [S, Hq, num_parts, 2]: running max (log2 units), sum
  float* part_o;                  // [S, Hq, num_parts, D]: unnormalised weighted sums
  int64_t q_seq_stride;
  int64_t num_blocks;
  int num_seqs, num_q_heads, num_kv_heads, group;
  int max_blocks;                 // block-table row length
  int block_shift;                // a cache block holds kBlock << block_shift tokens
  int num_parts;                  // partitions per sequence (grid dimension)
  int part_blocks;                // KV blocks per partition
  int num_items;                  // workgroups with work: num_seq_groups * num_kv_heads * num_parts
  int seqs_per_group;             // sequences (one wavefront each) per workgroup; 1 for the VALU kernel
  int num_seq_groups;             // ceil(num_seqs / seqs_per_group)
  int group_mode_ok;              // the workgroup's LDS holds a tile list for sharing groups
  float qk_scale_log2;            // scale * log2(e) (* k_scale for an fp8 cache)
  float v_scale;                  // 1, or v_scale for an fp8 cache
  // Fused step only (new_key == nullptr otherwise): the new token of every sequence,
  // written into its slot by the work item that holds the sequence's last position.
  const void* new_key;            // [S, Hkv, D] q dtype, token stride key_stride elements
  const void* new_value;          // [S, Hkv, D] q dtype, token stride value_stride elements
  const int64_t* slot_mapping;    // [S]: slot of each new token; negative = no write
  // Fused step with copy-on-write (nullptr: none): cow_src[s] >= 0 names the block that the
  // block holding sequence s's last position becomes a copy of before the new token is written.
  const int32_t* cow_src;         // [S]
  int64_t key_stride, value_stride;
  int64_t num_slots;              // num_blocks * block size
  float k_quant, v_quant;         // fp8 scales the new values are divided by
  // Work order (see decode_item): 0 = kv-head-major, 1 = kv head fastest; and the number
  // of consecutive work items each XCD takes in turn (item_of_workgroup).
  int item_order, xcd_run;
};

// Cache blocks hold kBlock << shift tokens (16, 32 or 64); the kernels walk a context in
// tiles of kBlock tokens, tile t lying in block t >> shift. A tile is named by
// block * 2^shift + (t mod 2^shift), or -1 when its block id is out of the pool.
__device__ __forceinline__ int tile_name(const int32_t* row, int t, int shift, int64_t num_blocks) {
  const int b = row[t >> shift];
  return (b >= 0 && b < num_blocks) ? b * (1 << shift) + (t & ((1 << shift) - 1)) : -1;
}

// Byte offset of a named tile in one kv head's view of a pool whose blocks are
// block_stride bytes apart.
__device__ __forceinline__ int64_t tile_offset(int v, int shift, int64_t block_stride, int tile_bytes) {
  return (int64_t)(v >> shift) * block_stride + (int64_t)(v & ((1 << shift) - 1)) * tile_bytes;
}

// Work items and their order. Which order reads the random block gather fastest on
// gfx950 depends on the kernel and was chosen by measurement:
// * order 1, (partition, sequence group, kv head) with the kv head fastest, each XCD in
//   turn taking the items of one sequence group (xcd_run = num_kv_heads): a block's kv-head
//   slices, adjacent in the pool, are read together through one XCD, and consecutive groups
//   spread over the XCDs. The matrix-core kernel with 4 sequences per workgroup runs 1-2%
//   faster this way;
// * order 2, for the vector-ALU kernel (one sequence per workgroup): (partition, run of 4
//   sequences, kv head, sequence in the run), each XCD taking 8 items in turn (two kv heads
//   of 4 neighbouring sequences). About 5% faster than order 0 and 0.4-1% faster than
//   order 1 on the 7B batch, and the beams of a request (neighbours) share one XCD's L2.
//   The item count is padded to whole runs of 4 sequences; padding items (sequence index
//   past the batch) do nothing;
// * order 0, (kv head, partition, sequence group) with the group fastest, each XCD taking
//   4 consecutive items in turn (xcd_run = 4): the matrix-core kernel with 2 sequences per
//   workgroup (8 query heads per kv head) runs 0.7% faster this way.
// Workgroups are dealt to the 8 XCDs round-robin; item_of_workgroup gives each XCD runs of
// xcd_run consecutive items. The grid is padded to a multiple of 8 * xcd_run (and of 32);
// ids past num_items do nothing.
__device__ __forceinline__ int item_of_workgroup(int w, const DecodeArgs& a) {
  const int R = a.xcd_run, xcd = w & 7, k = w >> 3;
  return ((k / R) * 8 + xcd) * R + (k % R);
}

struct Item {
  int s, g, p;
};

// it.s is the group's first sequence (groups of one sequence for the VALU kernel).
__device__ __forceinline__ Item decode_item(int j, const DecodeArgs& a) {
  Item it;
  if (a.item_order == 2) {
    const int sl = j % 4, r = j / 4;
    it.g = r % a.num_kv_heads;
    const int r2 = r / a.num_kv_heads, runs = (a.num_seq_groups + 3) / 4;
    it.s = ((r2 % runs) * 4 + sl) * a.seqs_per_group;
    it.p = r2 / runs;
  } else if (a.item_order == 1) {
    it.g = j % a.num_kv_heads;
    const int r = j / a.num_kv_heads;
    it.s = (r % a.num_seq_groups) * a.seqs_per_group;
    it.p = r / a.num_seq_groups;
  } else {
    it.s = (j % a.num_seq_groups) * a.seqs_per_group;
    const int r = j / a.num_seq_groups;
    it.p = r % a.num_parts;
    it.g = r / a.num_parts;
  }
  return it;
}

// Grid of a decode launch: item_of_workgroup reaches items in whole blocks of 8 * xcd_run
// workgroups, so the grid covers num_items in such blocks (then rounds up to 32, which
// only adds ids past num_items).
inline int decode_grid(const DecodeArgs& a) {
  const long long block = 8LL * a.xcd_run;
  const long long g = ((long long)a.num_items + block - 1) / block * block;
  return (int)((g + 31) / 32 * 32);
}

// Orders a wavefront's own LDS writes before its later LDS reads of other lanes' data
// (what a workgroup barrier does for a one-wave workgroup), without involving the
// other wavefronts of the workgroup.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A work item's block-table slice (the tile names of its partition) is staged in LDS.
// Its first kBtBatch * kWave entries are loaded at the very start of the item, before
// the context length is known: their bound comes from the table's row length, so the
// context length and the slice take one memory latency rather than two in a chain.
// Entries past the context are loaded but never used.
constexpr int kBtBatch = 8;
struct BtSlice {
  int v[kBtBatch];   // entry k * kWave + lane
};

__device__ __forceinline__ void prefetch_bt_slice(const DecodeArgs& a, int s, int t0, BtSlice& sl) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t* row = a.block_tables + (int64_t)s * a.max_blocks;
  // t0 lies inside the table (t0 < max_blocks << shift), so hi >= 1.
  const int hi = min(a.part_blocks, (a.max_blocks << a.block_shift) - t0);
#pragma unroll
  for (int k = 0; k < kBtBatch; ++k)
    sl.v[k] = tile_name(row, t0 + min(k * kWave + lane, hi - 1), a.block_shift, a.num_blocks);
}

// Copy-on-write in the fused step ("vLLM推理引擎PagedAttention原理与性能优化实战", §3.2: the
// first write into a block that several sequences share goes to a private copy of it). When
// cow_src[s] names a block, the block that holds sequence s's last position (block `lb` of
// its table, `dst`, private to s) is to become a copy of block `src` before the new token
// lands in it. Within the step that block still holds stale bytes: its tiles are read from
// `src` instead (the new token's row is patched in as always), and the work item that
// writes the new token also copies `src` into `dst`, every row but the token's (`skip`).
// A source or destination outside the pool, or a block copied onto itself, copies nothing.
struct CowRead {
  int lb;     // logical block of the sequence's last position
  int src;    // its source block, -1: no copy
  int dst;    // the block-table entry lb
  int skip;   // row of dst the new token is written to, -1: none
};

__device__ __forceinline__ CowRead cow_read(const DecodeArgs& a, int s, int ctx) {
  CowRead c{-1, -1, -1, -1};
  if (a.cow_src == nullptr || ctx <= 0) return c;
  const int b = a.cow_src[s];
  const int P = kBlock << a.block_shift;
  const int lb = (ctx - 1) / P;
  const int dst = a.block_tables[(int64_t)s * a.max_blocks + lb];
  if (b >= 0 && b < a.num_blocks && dst >= 0 && dst < a.num_blocks && dst != b) {
    const int64_t slot = a.slot_mapping[s];
    c.lb = lb;
    c.src = b;
    c.dst = dst;
    c.skip = (slot >= 0 && slot < a.num_slots && slot / P == dst) ? (int)(slot % P) : -1;
  }
  return c;
}

// The name of 16-token tile tt (whose name in the block table is `name`) as the step reads it.
__device__ __forceinline__ int cow_tile(const CowRead& c, int tt, int shift, int name) {
  return (c.src >= 0 && (tt >> shift) == c.lb) ? c.src * (1 << shift) + (tt & ((1 << shift) - 1)) : name;
}

// Stores entries [0, n) of the slice of sequence s from tile t0 into dst (n <= the
// prefetch bound): the prefetched ones, then any further ones, eight loads in flight per
// lane (indices past n re-read entry n - 1 and are not stored). Tiles of a copy-on-write
// block are stored under their source's name (`cow`).
__device__ __forceinline__ void store_bt_slice(const DecodeArgs& a, int s, int t0, int n, const BtSlice& sl,
                                               int* dst, const CowRead& cow) {
  const int lane = threadIdx.x & (kWave - 1), shift = a.block_shift;
#pragma unroll
  for (int k = 0; k < kBtBatch; ++k) {
    const int i = k * kWave + lane;
    if (i < n) dst[i] = cow_tile(cow, t0 + i, shift, sl.v[k]);
  }
  const int32_t* row = a.block_tables + (int64_t)s * a.max_blocks;
  for (int i0 = kBtBatch * kWave; i0 < n; i0 += kBtBatch * kWave) {
    int v[kBtBatch];
#pragma unroll
    for (int k = 0; k < kBtBatch; ++k)
      v[k] = tile_name(row, t0 + min(i0 + k * kWave + lane, n - 1), shift, a.num_blocks);
#pragma unroll
    for (int k = 0; k < kBtBatch; ++k) {
      const int i = i0 + k * kWave + lane;
      if (i < n) dst[i] = cow_tile(cow, t0 + i, shift, v[k]);
    }
  }
}

// Fused step: the work item of partition p of a sequence with (clamped) context length
// ctx writes that sequence's new token when p holds position ctx - 1 (partition 0 when
// ctx is 0).
__device__ __forceinline__ bool owns_new_token(const DecodeArgs& a, int ctx, int p) {
  if (a.new_key == nullptr) return false;
  const int last = ctx > 0 ? ctx - 1 : 0;
  return p == min(last / (a.part_blocks * kBlock), a.num_parts - 1);
}

// Fused step: one lane's share of sequence s's new token for kv head g, already in the
// cache's storage format: lanes 0 .. D/8-1 hold 8 elements of its K row, lanes D/8 ..
// D/4-1 8 elements of its V row. The work item keeps the row in registers and in an LDS
// copy (stage_new_token): the tile that holds the token's position is patched from that
// copy before use (the cache slot still holds stale bytes), and the row is stored into
// the cache at the end of the item, where the store does not compete with the item's
// loads. No other work item reads the slot.
struct TokenChunk {
  u32x4 data;    // converted chunk (fp8: 8 codes in the first two dwords)
  int64_t dst;   // element index in the cache
  bool store;    // this lane stores a chunk
  bool is_v;
  bool written;  // the token has a valid slot (the same in every lane): only then does the
                 // item see it in place of the slot's old bytes, as after a separate write
};

template <int QT, int KVT, int D>
__device__ __forceinline__ TokenChunk load_new_token(const DecodeArgs& a, int s, int g) {
  constexpr int kChunks = D / 8;
  TokenChunk t;
  t.data = u32x4{0u, 0u, 0u, 0u};
  t.dst = 0;
  t.store = false;
  t.is_v = false;
  const int64_t slot = a.slot_mapping[s];
  t.written = slot >= 0 && slot < a.num_slots;
  const int lane = threadIdx.x & (kWave - 1);
  if (lane >= 2 * kChunks) return t;
  // The slot and the row are loaded independently (neither address depends on the other).
  t.is_v = lane >= kChunks;
  const int c = t.is_v ? lane - kChunks : lane;
  const uint16_t* src = (const uint16_t*)(t.is_v ? a.new_value : a.new_key) +
                        (int64_t)s * (t.is_v ? a.value_stride : a.key_stride) + (int64_t)g * D + 8 * c;
  t.data = convert_cache_chunk<QT, KVT>(*(const u32x4*)src, t.is_v ? a.v_quant : a.k_quant);
  t.store = t.written;
  const int P = kBlock << a.block_shift;
  t.dst = t.store ? ((slot / P * a.num_kv_heads + g) * P + slot % P) * D + 8 * c : 0;
  return t;
}

// Bytes of one cache row (one token, one kv head) in storage format.
template <int KVT, int D>
constexpr int row_bytes() { return D * (KVT == kFP8 ? 1 : 2); }

// Writes the lane's chunk into `rows` (K row, then V row, storage format). Every lane of
// the wavefront calls this; lanes without a chunk write nothing.
template <int KVT, int D>
__device__ __forceinline__ void stage_new_token(const TokenChunk& t, uint8_t* rows) {
  constexpr int kChunks = D / 8, kChunkBytes = 8 * (KVT == kFP8 ? 1 : 2);
  const int lane = threadIdx.x & (kWave - 1);
  if (lane >= 2 * kChunks) return;
  uint8_t* dst = rows + (t.is_v ? row_bytes<KVT, D>() : 0) + (lane % kChunks) * kChunkBytes;
  if constexpr (KVT == kFP8)
    *(u32x2*)dst = u32x2{t.data[0], t.data[1]};
  else
    *(u32x4*)dst = t.data;
}

template <int KVT>
__device__ __forceinline__ void store_new_token(const DecodeArgs& a, const TokenChunk& t) {
  if (t.store) store_converted_chunk<KVT>(t.data, const_cast<void*>(t.is_v ? a.v_cache : a.k_cache), t.dst);
}

// A work item keeps its sequence's CowRead in LDS (at kCowSlot of the sequence's token-row
// area, after the new token's two rows of up to 256 bytes each) from its start to the copy
// at its end, rather than in registers across its tile loop.
constexpr int kCowSlot = 512;
__device__ __forceinline__ void stash_cow(uint8_t* tok_rows, const CowRead& c) {
  if ((threadIdx.x & (kWave - 1)) == 0) {
    int* slot = (int*)(tok_rows + kCowSlot);
    slot[0] = c.lb;
    slot[1] = c.src;
    slot[2] = c.dst;
    slot[3] = c.skip;
  }
}
__device__ __forceinline__ CowRead stashed_cow(const uint8_t* tok_rows) {
  const int* slot = (const int*)(tok_rows + kCowSlot);
  return CowRead{slot[0], slot[1], slot[2], slot[3]};
}

// The copy of a copy-on-write block for kv head g, by one wavefront: kv head g's slice of
// block cow.src is copied, K and V, into block cow.dst, except row cow.skip, in 16-byte
// chunks (chunk c: tensor c / chunks, byte 16 (c mod chunks) of the slice). Done by the
// work item that writes the sequence's new token, after its tiles. cow_copy_begin loads the
// lane's first CowChunks<D>::kBatch chunks and cow_copy_end stores them and copies any further chunks:
// the group mode puts its merge between the two, which hides the loads' latency; the other
// paths call cow_copy (both at once). Nothing else in the launch reads the destination
// block.
// Chunks per lane that cow_copy_begin loads: a 16-token fp8 block's slice at D = 128, half of
// it at D = 64 (where four would cost the matrix-core kernel a wavefront per SIMD).
template <int D>
struct CowChunks {
  static constexpr int kBatch = D >= 128 ? 4 : 2;
  u32x4 v[kBatch];
};

template <int KVT, int D>
struct CowGeometry {
  static constexpr int kRB = row_bytes<KVT, D>();
  int chunks;            // 16-byte chunks per tensor
  int64_t src_off, dst_off;
  __device__ __forceinline__ CowGeometry(const DecodeArgs& a, int g, const CowRead& cow) {
    const int P = kBlock << a.block_shift;
    const int64_t slice = (int64_t)P * kRB;   // one kv head's share of a block
    chunks = P * kRB / 16;
    src_off = ((int64_t)cow.src * a.num_kv_heads + g) * slice;
    dst_off = ((int64_t)cow.dst * a.num_kv_heads + g) * slice;
  }
  __device__ __forceinline__ uint8_t* base(const DecodeArgs& a, int c) const {
    return (uint8_t*)const_cast<void*>(c >= chunks ? a.v_cache : a.k_cache);
  }
  __device__ __forceinline__ int64_t off(int c) const { return (int64_t)(c >= chunks ? c - chunks : c) * 16; }
  __device__ __forceinline__ bool skipped(int c, int skip) const {
    return (int)(off(c) / kRB) == skip;
  }
};

template <int KVT, int D>
__device__ __forceinline__ void cow_copy_begin(const DecodeArgs& a, int g, const CowRead& cow, CowChunks<D>& ch) {
  if (cow.src < 0) return;
  const CowGeometry<KVT, D> geo(a, g, cow);
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 0; k < CowChunks<D>::kBatch; ++k) {
    const int c = lane + k * kWave;
    if (c < 2 * geo.chunks) ch.v[k] = *(const u32x4*)(geo.base(a, c) + geo.src_off + geo.off(c));
  }
}

template <int KVT, int D>
__device__ __forceinline__ void cow_copy_end(const DecodeArgs& a, int g, const CowRead& cow, const CowChunks<D>& ch) {
  if (cow.src < 0) return;
  const CowGeometry<KVT, D> geo(a, g, cow);
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 0; k < CowChunks<D>::kBatch; ++k) {
    const int c = lane + k * kWave;
    if (c < 2 * geo.chunks && !geo.skipped(c, cow.skip)) *(u32x4*)(geo.base(a, c) + geo.dst_off + geo.off(c)) = ch.v[k];
  }
  for (int c = lane + CowChunks<D>::kBatch * kWave; c < 2 * geo.chunks; c += kWave) {
    if (geo.skipped(c, cow.skip)) continue;
    const u32x4 x = *(const u32x4*)(geo.base(a, c) + geo.src_off + geo.off(c));
    *(u32x4*)(geo.base(a, c) + geo.dst_off + geo.off(c)) = x;
  }
}

template <int KVT, int D>
__device__ __forceinline__ void cow_copy(const DecodeArgs& a, int g, const CowRead& cow) {
  CowChunks<D> ch;
  cow_copy_begin<KVT, D>(a, g, cow, ch);
  cow_copy_end<KVT, D>(a, g, cow, ch);
}

// Replaces the bytes a lane loaded for one 16-byte piece of a tile with the new token's
// bytes when the piece lies in the token's row: `off` is the piece's byte offset in the
// tile (rows of row_bytes each), `row` the token's row in the block, `src` its row copy.
template <int KVT, int D>
__device__ __forceinline__ void patch_piece(u32x4& piece, uint32_t off, int row, const uint8_t* src) {
  constexpr int RB = row_bytes<KVT, D>();
  if ((int)(off / RB) == row) piece = *(const u32x4*)(src + off % RB);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache-policy operand of a buffer load: 0 is the default (allocate in L2), bit 1 is
// "nt" (non-temporal, streaming).
constexpr int kPolicyCached = 0;
constexpr int kPolicyStream = 2;

// 16-byte load of KV cache bytes. A block that only one sequence reads is read once per
// decode step, so its loads are marked non-temporal: they do not displace other lines in
// L2, and on gfx950 a random gather of whole blocks runs about 9% faster this way. Blocks
// that several sequences share keep the default policy so that the other readers hit L2.
template <int POLICY>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, POLICY));
}

// Two waves share each SIMD and the older one wins instruction arbitration, so without
// help it runs ahead and finishes long before its neighbour, leaving the memory system
// under-fed at the end of the launch. A wave that streams private blocks therefore
// lowers its issue priority as it works through them (3 in the first quarter ... 0 in
// the last), which lets a lagging wave catch up. (Waves reading shared blocks do better
// in step with each other, so they keep the default priority.)
__device__ __forceinline__ void progress_priority(int done, int total) {
  const int level = ((total - done) * 4 - 1) / total;   // 3 .. 0 while done < total
  if (level >= 3) __builtin_amdgcn_s_setprio(3);
  else if (level == 2) __builtin_amdgcn_s_setprio(2);
  else if (level == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

}  // namespace pkv
