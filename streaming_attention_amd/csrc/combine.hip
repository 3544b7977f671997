// Log-sum-exp merge of split-KV partials for gfx950.
//
// Method: "ADR-0060: AHBM GQA Fused Attention kernel (Llama3-70B)", section 4:
// two partials merge as m = max(m_a, m_b), l = l_a e^{m_a - m} + l_b e^{m_b - m},
// O = O_a e^{m_a - m} + O_b e^{m_b - m}, normalised once at the end.  With the
// partials carried as (lse_s, O_s / l_s) this is M = max_s lse_s,
// w_s = e^{lse_s - M}, O = sum w_s O_s / sum w_s, LSE = M + ln sum w_s.  The
// merge is associative and commutative, so one pass over all splits of a row
// is a valid merge order.
//
// MI355X mapping: one wave per (sequence, query head) row, each lane owning
// D / 64 consecutive output elements; the splits are read in order with
// coalesced 256/512-byte wave loads.  The split-lse maximum is a wave
// reduction.  This kernel moves ~1.6% of the decode KV bytes.
#include "common.h"
#include "launch.h"

namespace sa {
namespace {

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_lse_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const int32_t* __restrict__ num_splits, int B,
                                                          int Hq, int max_splits, void* __restrict__ o,
                                                          float* __restrict__ lse) {
  constexpr int PER = D / 64;   // output elements per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= B * Hq) return;
  const int b = row / Hq;
  int n = num_splits ? num_splits[b] : max_splits;
  n = n < 1 ? 1 : (n > max_splits ? max_splits : n);

  const float* L = part_lse + (size_t)row * max_splits;
  float M = kNegInf;
  for (int i = l; i < n; i += 64) M = fmaxf(M, L[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (M != kNegInf) {
    const float* Op = part_o + (size_t)row * max_splits * D + PER * l;
    for (int s = 0; s < n; ++s) {
      const float wgt = exp2_hw((L[s] - M) * kLog2e);
      wsum += wgt;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += wgt * Op[(size_t)s * D + i];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (OUT_BF16) {
    bf16* out = reinterpret_cast<bf16*>(o) + (size_t)row * D + PER * l;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] = (bf16)(acc[i] * inv);
  } else {
    float* out = reinterpret_cast<float*>(o) + (size_t)row * D + PER * l;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] = acc[i] * inv;
  }
  if (lse != nullptr && l == 0) lse[row] = wsum > 0.f ? M + __logf(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_combine_lse(const CombineArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq;
  const dim3 g((unsigned)((rows + 3) / 4)), blk(256);
#define SA_LAUNCH(DD, BF)                                                                                   \
  hipLaunchKernelGGL((combine_lse_kernel<DD, BF>), g, blk, 0, stream, a.part_o, a.part_lse, a.num_splits, a.B, \
                     a.Hq, a.max_splits, a.o, a.lse)
  if (a.d == 128) {
    if (a.out_bf16) SA_LAUNCH(128, true); else SA_LAUNCH(128, false);
  } else {
    if (a.out_bf16) SA_LAUNCH(64, true); else SA_LAUNCH(64, false);
  }
#undef SA_LAUNCH
  return hipGetLastError();
}

}  // namespace sa
