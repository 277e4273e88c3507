// Second pass of split-context decode attention: merge the per-partition softmax pieces.
//
// The pages give no split of one sequence's context (they only name IO-aware
// attention as prior art, "vLLM 推理优化技术深度调研报告", 维度二.4). The merge is the
// softmax identity: with partition maxima m_p (log2 units), sums l_p and unnormalised
// outputs o_p, M = max m_p, out = sum 2^(m_p - M) o_p / sum 2^(m_p - M) l_p.
#include "pkv_launch.h"

namespace pkv {


// One workgroup of 256 threads per output row (sequence, q head). Thread (pg, cg) owns
// columns 4cg..4cg+3 of every partition p = pg (mod kSlices); the kSlices partial sums
// are added in LDS in a fixed order, so the result does not depend on timing. The
// pieces of a thread's first kBatch partitions are loaded at once, before the maximum
// is known, so that up to kSlices * kBatch partitions cost one memory latency; more
// partitions are read in further rounds.
template <int QT, int D>
__global__ __launch_bounds__(256) void paged_decode_reduce(ReduceArgs a) {
  constexpr int kGroups = D / 4;              // column groups of 4 floats
  constexpr int kSlices = 256 / kGroups;      // partition slices
  constexpr int kBatch = 8;                   // partitions per thread held in registers
  __shared__ float wave_max[256 / kWave];
  __shared__ f32x4 part_acc[kSlices][kGroups];
  __shared__ float part_l[kSlices];

  const int row = blockIdx.x;
  const int tid = threadIdx.x, cg = tid % kGroups, pg = tid / kGroups;
  const int s = row / a.num_q_heads;
  const int ctx = min(a.context_lens[s], a.max_tokens);
  const int np = min(ctx > 0 ? (ctx + a.part_tokens - 1) / a.part_tokens : 0, a.num_parts);
  const float* ml = a.part_ml + (int64_t)row * a.num_parts * 2;
  const float* po = a.part_o + (int64_t)row * a.num_parts * D + 4 * cg;

  float mr[kBatch], lr[kBatch];
  f32x4 orr[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int p = pg + k * kSlices;
    const bool live = p < np;
    const f32x2 v = live ? *(const f32x2*)(ml + 2 * p) : f32x2{-INFINITY, 0.f};
    mr[k] = v[0];
    lr[k] = v[1];
    orr[k] = live ? *(const f32x4*)(po + (int64_t)p * D) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // M = max over the partitions' running maxima (log2 units).
  float m = mr[0];
#pragma unroll
  for (int k = 1; k < kBatch; ++k) m = fmaxf(m, mr[k]);
  for (int p = kSlices * kBatch + tid; p < np; p += 256) m = fmaxf(m, ml[2 * p]);
#pragma unroll
  for (int x = kWave / 2; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x, kWave));
  if ((tid & (kWave - 1)) == 0) wave_max[tid / kWave] = m;
  __syncthreads();
  float M = wave_max[0];
#pragma unroll
  for (int w = 1; w < 256 / kWave; ++w) M = fmaxf(M, wave_max[w]);
  if (M == -INFINITY) M = 0.f;   // no partition (empty context): every weight is exp2(-inf) = 0

  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const float w = exp2_fast(mr[k] - M);     // an empty slot: exp2(-inf) = 0
    L = fmaf(w, lr[k], L);
    acc += w * orr[k];
  }
  for (int p = pg + kSlices * kBatch; p < np; p += kSlices) {
    const float w = exp2_fast(ml[2 * p] - M);
    L = fmaf(w, ml[2 * p + 1], L);
    acc += w * *(const f32x4*)(po + (int64_t)p * D);
  }
  part_acc[pg][cg] = acc;
  if (cg == 0) part_l[pg] = L;
  __syncthreads();
  if (pg != 0) return;
  f32x4 sum = part_acc[0][cg];
  float Lsum = part_l[0];
#pragma unroll
  for (int q = 1; q < kSlices; ++q) {
    sum += part_acc[q][cg];
    Lsum += part_l[q];
  }
  const float inv = np > 0 ? a.v_scale / Lsum : 0.f;
  sum *= inv;
  uint16_t* o = (uint16_t*)a.out + (int64_t)row * D + 4 * cg;
  *(u32x2*)o = u32x2{pack2<QT>(sum[0], sum[1]), pack2<QT>(sum[2], sum[3])};
}

hipError_t launch_decode_reduce(const ReduceArgs& a, int q_type, int head_dim, hipStream_t stream) {
  const dim3 grid(a.num_seqs * a.num_q_heads);
#define PKV_CASE(QT, D)                                                                    \
  if (q_type == QT && head_dim == D) {                                                      \
    hipLaunchKernelGGL((paged_decode_reduce<QT, D>), grid, dim3(256), 0, stream, a);        \
    return hipGetLastError();                                                               \
  }
  PKV_CASE(kBF16, 128) PKV_CASE(kBF16, 64) PKV_CASE(kF16, 128) PKV_CASE(kF16, 64)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
