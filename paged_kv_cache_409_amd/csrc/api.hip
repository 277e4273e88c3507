// C ABI of libpkv.so: host-side validation and dispatch. Contract in include/pkv.h.
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "pkv.h"
#include "pkv_block_manager.h"
#include "pkv_validate.h"
#include "gather_probe.h"
#include "pkv_launch.h"


namespace {

constexpr int kMaxGroup = 16;
constexpr int kMaxPartTokens = 32768;     // block-table slice of one partition: 2048 ids in LDS
// Work items (sequence, kv head, partition) to aim for when splitting contexts (measured
// over partition sizes on small batches):
// * matrix-core kernel: one per SIMD. Fewer, longer partitions stream longer and leave
//   less to merge; on the 32K-token batch, 2048-token partitions (1024 items) beat
//   1024-token ones by 3%, and at 1-2 sequences 128-256-token partitions lose 8-20%;
// * vector-ALU kernel (one query head per kv head): two per SIMD. Its wavefront keeps
//   fewer bytes in flight; batches of 4-32 Llama-2-7B-shaped sequences ran 23-34% faster
//   at 2048 items than at 1024.
// Partitions are multiples of kPartGrain tokens: short contexts in small batches want
// short partitions (8 sequences of 512-768 tokens at 8 kv heads: 64-token partitions
// 13.1 us, 256-token ones 19.6 us).
constexpr int kTargetItemsMfma = 1024;
constexpr int kTargetItemsValu = 2048;
constexpr int kPartGrain = 64;
constexpr size_t kAlign = 256;
constexpr size_t kMaxDynamicLds = 65536;  // dynamic LDS a decode workgroup may use

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is16bit(int t) { return t == PKV_F16 || t == PKV_BF16; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int part_tokens;
  int num_parts;
  size_t ml_bytes;
  size_t ws_bytes;
};

int resolve_partition(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len, int partition_size) {
  if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      max_context_len < 0)
    return PKV_ERR_SHAPE;
  if (partition_size < 0 || partition_size % 16 != 0 || partition_size > kMaxPartTokens) return PKV_ERR_SHAPE;
  if (partition_size > 0) return partition_size;
  const int whole = (int)round_up((size_t)(max_context_len > 0 ? max_context_len : 1), 16);
  const long long units = (long long)num_seqs * num_kv_heads;
  const int target = num_q_heads == num_kv_heads ? kTargetItemsValu : kTargetItemsMfma;
  int part = whole;
  if (units > 0 && units < target) {
    const long long want = (target + units - 1) / units;
    part = (int)round_up((size_t)((max_context_len + want - 1) / want), kPartGrain);
    if (part > whole) part = whole;
  }
  return part > kMaxPartTokens ? kMaxPartTokens : part;
}

int make_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_context_len,
              int partition_size, Plan* plan) {
  const int part = resolve_partition(num_seqs, num_q_heads, num_kv_heads, max_context_len, partition_size);
  if (part < 0) return part;
  plan->part_tokens = part;
  plan->num_parts = (max_context_len + part - 1) / part;
  if (plan->num_parts < 1) plan->num_parts = 1;
  plan->ml_bytes = 0;
  plan->ws_bytes = 0;
  if (plan->num_parts > 1) {
    const size_t rows = (size_t)num_seqs * num_q_heads * plan->num_parts;
    plan->ml_bytes = round_up(rows * 2 * sizeof(float), kAlign);
    plan->ws_bytes = plan->ml_bytes + round_up(rows * (size_t)head_dim * sizeof(float), kAlign);
  }
  return PKV_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// log2(block_size / 16) for the supported block sizes 16, 32 and 64; -1 otherwise.
int block_shift_of(int block_size) {
  return block_size == 16 ? 0 : block_size == 32 ? 1 : block_size == 64 ? 2 : -1;
}

// The address under which the GPU reaches p: p itself for device memory, the mapped address
// for host memory pinned through the HIP runtime. Pageable (unregistered) host memory is
// refused, since a kernel touching it would fault.
int gpu_address(const void* p, void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the runtime's error state
    return PKV_ERR_UNSUPPORTED;
  }
  switch (attr.type) {
    case hipMemoryTypeHost:
      if (!attr.devicePointer) return PKV_ERR_UNSUPPORTED;
      *out = attr.devicePointer;
      return PKV_OK;
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
      *out = const_cast<void*>(p);
      return PKV_OK;
    default:   // unregistered host memory, arrays, anything else
      return PKV_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case PKV_ERR_DTYPE: return "unknown or disallowed dtype combination";
    case PKV_ERR_UNSUPPORTED: return "request outside what the kernels implement";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_ALIGN: return "a device pointer or stride is not 16-byte aligned";
    case PKV_ERR_HIP: return "the HIP runtime reported an error";
    case PKV_ERR_NO_BLOCKS: return "not enough free blocks";
    case PKV_ERR_SEQ: return "unknown or duplicate sequence id, or the sequence is swapped the other way";
    case PKV_ERR_CAPACITY: return "an output array is too small";
    default: return "unknown status";
  }
}

int pkv_api_version(void) { return PKV_API_VERSION; }

int pkv_decode_partition_tokens(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len,
                                int partition_size) {
  return resolve_partition(num_seqs, num_q_heads, num_kv_heads, max_context_len, partition_size);
}

size_t pkv_paged_attention_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                          int max_context_len, int partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  Plan plan;
  if (make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size, &plan) != PKV_OK)
    return 0;
  return plan.ws_bytes;
}

}  // extern "C"

namespace {

// New tokens of a fused decode step (all null for plain decoding).
struct NewTokens {
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  int64_t key_stride, value_stride;
  const int32_t* cow_src;   // may be null
};

int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens,
                int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                int64_t num_blocks, int max_blocks_per_seq, int max_context_len,
                int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                int64_t q_seq_stride, int partition_size, const NewTokens* tok,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((long long)num_seqs * num_q_heads > (1LL << 30)) return PKV_ERR_SHAPE;
  if (!is16bit(q_dtype)) return PKV_ERR_DTYPE;
  if (kv_dtype != q_dtype && kv_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  const int shift = block_shift_of(block_size);
  if (shift < 0 || (head_dim != 64 && head_dim != 128)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
  // tiles are named block * 2^shift + sub-tile in an int
  if ((num_blocks << shift) > 0x7fffffffLL || ((int64_t)max_blocks_per_seq << shift) > 0x7fffffffLL / 16)
    return PKV_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (group > kMaxGroup) return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  if (kv_dtype == PKV_FP8_E4M3 &&
      !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return PKV_ERR_SHAPE;
  if (q_seq_stride == 0) q_seq_stride = (int64_t)num_q_heads * head_dim;
  if (q_seq_stride < (int64_t)num_q_heads * head_dim) return PKV_ERR_SHAPE;
  const int64_t kv_row = (int64_t)num_kv_heads * head_dim;
  int64_t key_stride = 0, value_stride = 0;
  if (tok) {
    key_stride = tok->key_stride ? tok->key_stride : kv_row;
    value_stride = tok->value_stride ? tok->value_stride : kv_row;
    if (key_stride < kv_row || value_stride < kv_row) return PKV_ERR_SHAPE;
  }
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_NULL;
  if (tok && (!tok->key || !tok->value || !tok->slot_mapping)) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || q_seq_stride % 8 != 0)
    return PKV_ERR_ALIGN;
  if (tok && (!aligned16(tok->key) || !aligned16(tok->value) || key_stride % 8 != 0 || value_stride % 8 != 0))
    return PKV_ERR_ALIGN;
  if (tok && reinterpret_cast<uintptr_t>(tok->cow_src) % alignof(int32_t) != 0) return PKV_ERR_ALIGN;

  Plan plan;
  const int st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size, &plan);
  if (st != PKV_OK) return st;
  if ((long long)num_seqs * num_kv_heads * plan.num_parts > (1LL << 30)) return PKV_ERR_SHAPE;
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  }

  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.part_ml = plan.ws_bytes ? reinterpret_cast<float*>(workspace) : nullptr;
  a.part_o = plan.ws_bytes ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + plan.ml_bytes)
                           : nullptr;
  a.q_seq_stride = q_seq_stride;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.max_blocks = max_blocks_per_seq;
  a.block_shift = shift;
  a.num_parts = plan.num_parts;
  a.part_blocks = plan.part_tokens / 16;
  // Sequences per workgroup: the matrix-core kernel puts up to 16 / G neighbouring
  // sequences (one wavefront each) in a workgroup, so that sequences sharing blocks can
  // read them once; group mode needs the tile list to fit in LDS.
  int per_group = 1;
  bool group_mode = false;
  if (group > 1) {
    per_group = 16 / group < pkv::kMaxSeqsPerGroup ? 16 / group : pkv::kMaxSeqsPerGroup;
    // (list entries keep the logical block index in 16 bits)
    group_mode = per_group > 1 && (long long)per_group * a.part_blocks <= pkv::kMaxGroupListEntries &&
                 ((long long)max_blocks_per_seq << shift) <= 65536;
    if (pkv::mfma_decode_lds_bytes(head_dim, per_group, a.part_blocks, group_mode) > kMaxDynamicLds)
      group_mode = false;
    if (pkv::mfma_decode_lds_bytes(head_dim, per_group, a.part_blocks, group_mode) > kMaxDynamicLds)
      per_group = 1;
  }
  a.seqs_per_group = per_group;
  a.num_seq_groups = (num_seqs + per_group - 1) / per_group;
  a.group_mode_ok = group_mode ? 1 : 0;
  a.num_items = (int)((long long)a.num_seq_groups * num_kv_heads * plan.num_parts);
  // Work order (measured; see decode_item): runs of 4 sequences with the kv heads next for
  // the vector-ALU kernel, kv head fastest for matrix-core workgroups of 4 sequences,
  // kv-head-major for smaller workgroups.
  a.item_order = group == 1 ? 2 : (per_group >= 4 ? 1 : 0);
  a.xcd_run = a.item_order == 2 ? 8 : (a.item_order == 1 ? num_kv_heads : 4);
  if (a.item_order == 2) {   // whole runs of 4 sequences; the padding items do nothing
    const long long padded = (long long)(a.num_seq_groups + 3) / 4 * 4 * num_kv_heads * plan.num_parts;
    if (padded > (1LL << 30)) return PKV_ERR_SHAPE;
    a.num_items = (int)padded;
  }
  const float log2e = 1.4426950408889634f;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  a.qk_scale_log2 = scale * log2e * (fp8 ? k_scale : 1.0f);
  a.v_scale = fp8 ? v_scale : 1.0f;
  a.new_key = tok ? tok->key : nullptr;
  a.new_value = tok ? tok->value : nullptr;
  a.slot_mapping = tok ? tok->slot_mapping : nullptr;
  a.cow_src = tok ? tok->cow_src : nullptr;
  a.key_stride = key_stride;
  a.value_stride = value_stride;
  a.num_slots = num_blocks * block_size;
  a.k_quant = fp8 ? k_scale : 1.0f;
  a.v_quant = fp8 ? v_scale : 1.0f;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int qt = q_dtype == PKV_BF16 ? pkv::kBF16 : pkv::kF16;
  const int kt = fp8 ? pkv::kFP8 : qt;
  hipError_t e = group == 1 ? pkv::launch_decode_valu(a, qt, kt, head_dim, s)
                            : pkv::launch_decode_mfma(a, qt, kt, head_dim, s);
  if (e != hipSuccess) return PKV_ERR_HIP;
  if (plan.num_parts > 1) {
    pkv::ReduceArgs r;
    r.out = out;
    r.part_ml = a.part_ml;
    r.part_o = a.part_o;
    r.context_lens = context_lens;
    r.num_seqs = num_seqs;
    r.num_q_heads = num_q_heads;
    r.num_parts = plan.num_parts;
    r.part_tokens = plan.part_tokens;
    r.max_tokens = max_blocks_per_seq * block_size;
    r.v_scale = a.v_scale;
    e = pkv::launch_decode_reduce(r, qt, head_dim, s);
  }
  return hip_status(e);
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                               int64_t num_blocks, int max_blocks_per_seq, int max_context_len,
                               int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                               int64_t q_seq_stride, int partition_size,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, scale,
                     k_scale, v_scale, q_seq_stride, partition_size, nullptr, workspace, workspace_bytes, stream);
}

int pkv_decode_step(void* out, const void* q, void* k_cache, void* v_cache,
                    const void* key, const void* value, const int64_t* slot_mapping, const int32_t* cow_src,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                    int64_t num_blocks, int max_blocks_per_seq, int max_context_len,
                    int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                    int64_t q_seq_stride, int64_t key_stride, int64_t value_stride, int partition_size,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const NewTokens tok{key, value, slot_mapping, key_stride, value_stride, cow_src};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, scale,
                     k_scale, v_scale, q_seq_stride, partition_size, &tok, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Split-context partials of pkv_decode_step_no_alloc: a fixed array in the library's
// device image, so that the entry point needs no allocation. Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol); it uses the device
// address looked up per GPU below.
static __device__ __align__(256) uint8_t scratch[PKV_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];   // device address of `scratch` on each GPU, once looked up

// Device address of `scratch` on the GPU that runs `stream`. The first call for a GPU looks
// it up with that GPU current (each GPU holds its own copy of the array at its own address).
int scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return PKV_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return PKV_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return PKV_ERR_HIP;
    if (e != hipSuccess || !p) return PKV_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_decode_step_no_alloc(void* out, const void* q, void* k_cache, void* v_cache,
                             const void* key, const void* value, const int64_t* slot_mapping, const int32_t* cow_src,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             int64_t num_blocks, int max_blocks_per_seq, int max_context_len,
                             int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                             int64_t q_seq_stride, int64_t key_stride, int64_t value_stride, int partition_size,
                             void* stream) {
  void* ws = nullptr;
  const int st = scratch_address(reinterpret_cast<hipStream_t>(stream), &ws);
  if (st != PKV_OK) return st;
  const NewTokens tok{key, value, slot_mapping, key_stride, value_stride, cow_src};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, scale,
                     k_scale, v_scale, q_seq_stride, partition_size, &tok, ws, PKV_NO_ALLOC_SCRATCH_BYTES, stream);
}

int pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_start_loc,
                                int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int64_t num_blocks, int max_blocks_per_seq, int max_query_len,
                                int q_dtype, int kv_dtype, float scale, float k_scale, float v_scale,
                                int64_t q_token_stride, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_query_len < 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (!is16bit(q_dtype)) return PKV_ERR_DTYPE;
  if (kv_dtype != q_dtype && kv_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  const int shift = block_shift_of(block_size);
  if (shift < 0 || (head_dim != 64 && head_dim != 128)) return PKV_ERR_UNSUPPORTED;
  if ((num_blocks << shift) > 0x7fffffffLL || ((int64_t)max_blocks_per_seq << shift) > 0x7fffffffLL / 16)
    return PKV_ERR_SHAPE;
  // tile positions in one kv head's view of the pool are ints
  if ((num_blocks << shift) * num_kv_heads > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (!(std::isfinite(scale) && scale > 0.f)) return PKV_ERR_SHAPE;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  if (fp8 && !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return PKV_ERR_SHAPE;
  if (q_token_stride == 0) q_token_stride = (int64_t)num_q_heads * head_dim;
  if (q_token_stride < (int64_t)num_q_heads * head_dim) return PKV_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  const long long rows = (long long)max_query_len * group;
  if (rows > (1LL << 30) || (long long)num_tokens * num_q_heads > (1LL << 40)) return PKV_ERR_SHAPE;
  const long long row_tiles = (rows + pkv::kPrefillRows - 1) / pkv::kPrefillRows;
  const long long items = (long long)num_kv_heads * num_seqs * row_tiles;
  if (items > (1LL << 31) - 8) return PKV_ERR_SHAPE;
  if (items == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || q_token_stride % 8 != 0)
    return PKV_ERR_ALIGN;

  pkv::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.block_shift = shift;
  a.q_token_stride = q_token_stride;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.max_blocks = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.row_tiles = (int)row_tiles;
  a.num_items = (int)items;
  a.qk_scale_log2 = scale * 1.4426950408889634f * (fp8 ? k_scale : 1.0f);
  a.v_scale = fp8 ? v_scale : 1.0f;
  const int qt = q_dtype == PKV_BF16 ? pkv::kBF16 : pkv::kF16;
  const int kt = fp8 ? pkv::kFP8 : qt;
  // A 16-bit cache goes to the kernel that loads K/V straight into LDS; an fp8 cache is
  // widened on the way through registers.
  if (!fp8) return hip_status(pkv::launch_prefill_lds(a, qt, head_dim, reinterpret_cast<hipStream_t>(stream)));
  return hip_status(pkv::launch_prefill_mfma(a, qt, kt, head_dim, reinterpret_cast<hipStream_t>(stream)));
}

int pkv_reshape_and_cache(const void* key, const void* value, const int64_t* slot_mapping,
                          void* k_cache, void* v_cache,
                          int num_tokens, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                          int in_dtype, int kv_dtype, float k_scale, float v_scale,
                          int64_t key_stride, int64_t value_stride, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!is16bit(in_dtype)) return PKV_ERR_DTYPE;
  if (kv_dtype != in_dtype && kv_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  const int shift = block_shift_of(block_size);
  if (shift < 0 || head_dim <= 0 || head_dim % 8 != 0 || head_dim > 1024) return PKV_ERR_UNSUPPORTED;
  if (kv_dtype == PKV_FP8_E4M3 &&
      !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return PKV_ERR_SHAPE;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (key_stride == 0) key_stride = row;
  if (value_stride == 0) value_stride = row;
  if (key_stride < row || value_stride < row) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) || key_stride % 8 != 0 ||
      value_stride % 8 != 0)
    return PKV_ERR_ALIGN;
  if ((int64_t)num_tokens * num_kv_heads * (head_dim / 8) > (1LL << 40)) return PKV_ERR_SHAPE;

  pkv::CacheWriteArgs a;
  a.key = key;
  a.value = value;
  a.slot_mapping = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.key_stride = key_stride;
  a.value_stride = value_stride;
  a.num_slots = num_blocks * block_size;
  a.block_shift = shift;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  const int it = in_dtype == PKV_BF16 ? pkv::kBF16 : pkv::kF16;
  const int kt = kv_dtype == PKV_FP8_E4M3 ? pkv::kFP8 : it;
  return hip_status(pkv::launch_reshape_and_cache(a, it, kt, reinterpret_cast<hipStream_t>(stream)));
}

int pkv_gather_probe(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, int num_seqs, int num_kv_heads, int head_dim, int block_size,
                     int64_t num_blocks, int max_blocks_per_seq, int max_context_len, int kv_dtype, uint32_t* sink,
                     void* stream) {
  if (num_seqs < 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PKV_ERR_SHAPE;
  if (!is16bit(kv_dtype) && kv_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  const int shift = block_shift_of(block_size);
  if (shift < 0 || (head_dim != 64 && head_dim != 128)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
  if ((num_blocks << shift) > 0x7fffffffLL || ((int64_t)max_blocks_per_seq << shift) > 0x7fffffffLL / 16)
    return PKV_ERR_SHAPE;
  const long long tiles = ((long long)max_context_len + 15) / 16;
  int chunk = pkv::kProbeChunkMax;
  while (chunk > pkv::kProbeChunkMin &&
         (long long)num_seqs * num_kv_heads * ((tiles + chunk - 1) / chunk) < pkv::kProbeMinWaves)
    chunk /= 2;
  const long long chunks = (tiles + chunk - 1) / chunk;
  if ((long long)num_seqs * num_kv_heads * chunks > (1LL << 31) - 8) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || chunks == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !sink) return PKV_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return PKV_ERR_ALIGN;
  pkv::ProbeArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.sink = sink;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.block_shift = shift;
  a.chunk = chunk;
  a.num_chunks = (int)chunks;
  const int tile_bytes = 16 * head_dim * (kv_dtype == PKV_FP8_E4M3 ? 1 : 2);
  return hip_status(pkv::launch_gather_probe(a, tile_bytes, reinterpret_cast<hipStream_t>(stream)));
}

int pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int num_layers,
                    const int64_t* src_dst_pairs, int num_pairs, int64_t block_bytes, int64_t num_blocks,
                    void* stream) {
  if (num_layers < 0 || num_pairs < 0 || num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16 != 0)
    return PKV_ERR_SHAPE;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!k_caches || !v_caches || !src_dst_pairs) return PKV_ERR_NULL;
  for (int l = 0; l < num_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return PKV_ERR_NULL;
    if (!aligned16(k_caches[l]) || !aligned16(v_caches[l])) return PKV_ERR_ALIGN;
  }
  const long long chunk_wgs = (block_bytes / 16 + 255) / 256;
  if ((long long)num_pairs * chunk_wgs > (1LL << 31) - 1) return PKV_ERR_SHAPE;
  return hip_status(pkv::launch_move_blocks(k_caches, v_caches, k_caches, v_caches, num_layers, src_dst_pairs,
                                            num_pairs, block_bytes, num_blocks, num_blocks,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int pkv_swap_blocks(const void* const* src_k_caches, const void* const* src_v_caches, void* const* dst_k_caches,
                    void* const* dst_v_caches, int num_layers, const int64_t* src_dst_pairs, int num_pairs,
                    int64_t block_bytes, int64_t num_src_blocks, int64_t num_dst_blocks, void* stream) {
  if (num_layers < 0 || num_pairs < 0 || num_src_blocks <= 0 || num_dst_blocks <= 0 || block_bytes <= 0 ||
      block_bytes % 16 != 0)
    return PKV_ERR_SHAPE;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!src_k_caches || !src_v_caches || !dst_k_caches || !dst_v_caches || !src_dst_pairs) return PKV_ERR_NULL;
  for (int l = 0; l < num_layers; ++l) {
    if (!src_k_caches[l] || !src_v_caches[l] || !dst_k_caches[l] || !dst_v_caches[l]) return PKV_ERR_NULL;
    if (!aligned16(src_k_caches[l]) || !aligned16(src_v_caches[l]) || !aligned16(dst_k_caches[l]) ||
        !aligned16(dst_v_caches[l]))
      return PKV_ERR_ALIGN;
  }
  const long long chunk_wgs = (block_bytes / 16 + 255) / 256;
  if ((long long)num_pairs * chunk_wgs > (1LL << 31) - 1) return PKV_ERR_SHAPE;
  // Host pools and a host pair list are reached through their mapped addresses.
  std::vector<void*> sk(num_layers), sv(num_layers), dk(num_layers), dv(num_layers);
  for (int l = 0; l < num_layers; ++l) {
    int st = gpu_address(src_k_caches[l], &sk[l]);
    if (st == PKV_OK) st = gpu_address(src_v_caches[l], &sv[l]);
    if (st == PKV_OK) st = gpu_address(dst_k_caches[l], &dk[l]);
    if (st == PKV_OK) st = gpu_address(dst_v_caches[l], &dv[l]);
    if (st != PKV_OK) return st;
  }
  void* pairs = nullptr;
  const int st = gpu_address(src_dst_pairs, &pairs);
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_move_blocks(const_cast<const void* const*>(sk.data()), const_cast<const void* const*>(sv.data()), dk.data(), dv.data(), num_layers,
                                            static_cast<const int64_t*>(pairs), num_pairs, block_bytes,
                                            num_src_blocks, num_dst_blocks, reinterpret_cast<hipStream_t>(stream)));
}

int pkv_validate_inputs(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                        int max_blocks_per_seq, int block_size, int64_t num_blocks,
                        const int64_t* slot_mapping, int num_tokens, int decode_step,
                        const int32_t* cow_src, const int64_t* src_dst_pairs, int num_pairs, void* stream,
                        pkv_validation* result) {
  if (!result) return PKV_ERR_NULL;
  if (num_seqs < 0 || num_tokens < 0 || num_pairs < 0 || max_blocks_per_seq < 0) return PKV_ERR_SHAPE;
  if ((block_tables != nullptr) != (context_lens != nullptr)) return PKV_ERR_NULL;
  if (num_pairs > 0 && !src_dst_pairs) return PKV_ERR_NULL;
  // Host copies of the buffers, then the host checks (which repeat the argument checks).
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::vector<int32_t> bt, cl, cs;
  std::vector<int64_t> sm, pr;
  hipError_t e = hipSuccess;
  if (block_tables) {
    bt.resize((size_t)num_seqs * max_blocks_per_seq);
    cl.resize((size_t)num_seqs);
    if (!bt.empty())
      e = hipMemcpyAsync(bt.data(), block_tables, bt.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && !cl.empty())
      e = hipMemcpyAsync(cl.data(), context_lens, cl.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess && slot_mapping && num_tokens > 0) {
    sm.resize((size_t)num_tokens);
    e = hipMemcpyAsync(sm.data(), slot_mapping, sm.size() * sizeof(int64_t), hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess && cow_src && num_seqs > 0) {
    cs.resize((size_t)num_seqs);
    e = hipMemcpyAsync(cs.data(), cow_src, cs.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess && num_pairs > 0) {
    pr.resize((size_t)num_pairs * 2);
    e = hipMemcpyAsync(pr.data(), src_dst_pairs, pr.size() * sizeof(int64_t), hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return PKV_ERR_HIP;
  // Empty vectors still need non-null pointers where the caller passed a buffer.
  static const int32_t kNoInt = 0;
  static const int64_t kNoLong = 0;
  return pkv_validate_inputs_host(block_tables ? (bt.empty() ? &kNoInt : bt.data()) : nullptr,
                                  context_lens ? (cl.empty() ? &kNoInt : cl.data()) : nullptr, num_seqs,
                                  max_blocks_per_seq, block_size, num_blocks,
                                  slot_mapping ? (sm.empty() ? &kNoLong : sm.data()) : nullptr, num_tokens,
                                  decode_step, cow_src ? (cs.empty() ? &kNoInt : cs.data()) : nullptr,
                                  num_pairs > 0 ? pr.data() : nullptr, num_pairs, result);
}

}  // extern "C"
