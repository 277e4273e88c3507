// Second pass of split-context decode attention: merge the per-partition softmax pieces.
//
// The pages give no split of one sequence's context (they only name IO-aware
// attention as prior art, "vLLM 推理优化技术深度调研报告", 维度二.4). The merge is the
// softmax identity: with partition maxima m_p (log2 units), sums l_p and unnormalised
// outputs o_p, M = max m_p, out = sum 2^(m_p - M) o_p / sum 2^(m_p - M) l_p.
#include "pkv_launch.h"

namespace pkv {


template <int QT, int D>
__global__ __launch_bounds__(256) void paged_decode_reduce(ReduceArgs a) {
  constexpr int kTpr = D / 4;              // threads per output row, 4 columns each
  constexpr int kRows = 256 / kTpr;
  const int row = blockIdx.x * kRows + threadIdx.x / kTpr;
  const int col = (threadIdx.x % kTpr) * 4;
  if (row >= a.num_seqs * a.num_q_heads) return;
  const int s = row / a.num_q_heads;
  const int ctx = min(a.context_lens[s], a.max_tokens);
  const int np = min(ctx > 0 ? (ctx + a.part_tokens - 1) / a.part_tokens : 0, a.num_parts);
  const float* ml = a.part_ml + (int64_t)row * a.num_parts * 2;
  const float* po = a.part_o + (int64_t)row * a.num_parts * D + col;

  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < np; ++p) {
    const float w = exp2_fast(ml[2 * p] - M);
    L = fmaf(w, ml[2 * p + 1], L);
    acc += w * *(const f32x4*)(po + (int64_t)p * D);
  }
  const float inv = np > 0 ? a.v_scale / L : 0.f;
  acc *= inv;
  uint16_t* o = (uint16_t*)a.out + (int64_t)row * D + col;
  *(u32x2*)o = u32x2{pack2<QT>(acc[0], acc[1]), pack2<QT>(acc[2], acc[3])};
}

hipError_t launch_decode_reduce(const ReduceArgs& a, int q_type, int head_dim, hipStream_t stream) {
  const int rows = a.num_seqs * a.num_q_heads;
  const int rows_per_wg = 256 / (head_dim / 4);
  const dim3 grid((rows + rows_per_wg - 1) / rows_per_wg);
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
