// Log-sum-exp merge of split-KV partials for gfx950.
//
// Method: "ADR-0060: AHBM GQA Fused Attention kernel (Llama3-70B)", section 4:
// two partials merge as m = max(m_a, m_b), l = l_a e^{m_a - m} + l_b e^{m_b - m},
// O = O_a e^{m_a - m} + O_b e^{m_b - m}, normalised once at the end.  With the
// partials carried as (lse_s, O_s / l_s) this is M = max_s lse_s,
// w_s = e^{lse_s - M}, O = sum w_s O_s / sum w_s, LSE = M + ln sum w_s.  The
// merge is associative and commutative, so any grouping of the splits is a
// valid merge order.
//
// MI355X mapping.  Many splits (split-KV decode: tens of splits, few rows):
// one workgroup (4 waves) per output row, row blocks of 8 placed by XCD.  The kernel is latency-bound (a few
// MB in total), so every load of a row is issued in one round: the split lse
// values (one per thread, for the workgroup max M) and, per wave, up to 16
// partial rows (splits w, w + 4, ...; each lane owns D / 64 output elements).
// The four wave sums are added through LDS.  Few splits (at most kNarrow:
// split-KV prefill, many rows): one wave per row, 4 rows per workgroup, every
// lane reads the row's few lse values and its D / 64 elements of each partial.
#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 16;
constexpr int kNarrow = 8;   // largest split count handled one wave per row

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_lse_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const int32_t* __restrict__ num_splits, int Hq,
                                                          int max_splits, void* __restrict__ o,
                                                          float* __restrict__ lse) {
  constexpr int PER = D / 64;   // output elements per lane
  __shared__ float red[kWaves];
  __shared__ float acc_s[kWaves][D];
  __shared__ float wsum_s[kWaves];

  // Row block rb of 8 consecutive rows runs on XCD rb % 8 when the rows come
  // in multiples of 64 (workgroups are dealt to the 8 XCDs round robin): with
  // 8 query heads per KV head that is the XCD whose L2 holds the rows'
  // partials from the split-KV decode.
  int row = blockIdx.x;
  if ((gridDim.x & 63) == 0) {
    const int xcd = row & 7, j = row >> 3;
    row = 8 * (8 * (j >> 3) + xcd) + (j & 7);
  }
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int b = row / Hq;
  int n = num_splits ? num_splits[b] : max_splits;
  n = n < 1 ? 1 : (n > max_splits ? max_splits : n);
  const float* L = part_lse + (size_t)row * max_splits;
  const float* Op = part_o + (size_t)row * max_splits * D + PER * l;

  // Every load of the row is issued up front, in one memory round: the split
  // lse values for the maximum (n <= 256, one per thread) and this wave's
  // first kUnroll partial rows.
  float M = tid < n ? L[tid] : kNegInf;
  float lv[kUnroll];
  float ov[kUnroll][PER];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = w + kWaves * u;
    lv[u] = s < n ? L[s] : kNegInf;
#pragma unroll
    for (int i = 0; i < PER; ++i) ov[u][i] = s < n ? Op[(size_t)s * D + i] : 0.f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (l == 0) red[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  const float Mb = (M == kNegInf) ? 0.f : M;   // all splits empty: every weight is exp2(-inf) = 0
  for (int s0 = w;; s0 += kWaves * kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float wgt = exp2_hw((lv[u] - Mb) * kLog2e);
      wsum += wgt;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += wgt * ov[u][i];
    }
    if (s0 + kWaves * kUnroll >= n) break;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {   // next batch of splits (rarely needed: n > 32)
      const int s = s0 + kWaves * kUnroll + kWaves * u;
      lv[u] = s < n ? L[s] : kNegInf;
#pragma unroll
      for (int i = 0; i < PER; ++i) ov[u][i] = s < n ? Op[(size_t)s * D + i] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) acc_s[w][PER * l + i] = acc[i];
  if (l == 0) wsum_s[w] = wsum;
  __syncthreads();
  if (w != 0) return;

  const float ws = wsum_s[0] + wsum_s[1] + wsum_s[2] + wsum_s[3];
  const float inv = ws > 0.f ? 1.f / ws : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = PER * l + i;
    const float val = (acc_s[0][d] + acc_s[1][d] + acc_s[2][d] + acc_s[3][d]) * inv;
    if (OUT_BF16)
      reinterpret_cast<bf16*>(o)[(size_t)row * D + d] = (bf16)val;
    else
      reinterpret_cast<float*>(o)[(size_t)row * D + d] = val;
  }
  if (lse != nullptr && l == 0) lse[row] = ws > 0.f ? M + __logf(ws) : kNegInf;
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_lse_narrow_kernel(const float* __restrict__ part_o,
                                                                 const float* __restrict__ part_lse,
                                                                 const int32_t* __restrict__ num_splits, int rows,
                                                                 int Hq, int max_splits, void* __restrict__ o,
                                                                 float* __restrict__ lse) {
  constexpr int PER = D / 64;   // output elements per lane (consecutive)
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int l = threadIdx.x & 63;
  int n = num_splits ? num_splits[row / Hq] : max_splits;
  n = n < 1 ? 1 : (n > max_splits ? max_splits : n);
  const float* L = part_lse + (size_t)row * max_splits;
  const float* Op = part_o + (size_t)row * max_splits * D + PER * l;

  float lv[kNarrow], ov[kNarrow][PER];
#pragma unroll
  for (int s = 0; s < kNarrow; ++s) {
    lv[s] = s < n ? L[s] : kNegInf;
#pragma unroll
    for (int i = 0; i < PER; ++i) ov[s][i] = s < n ? Op[(size_t)s * D + i] : 0.f;
  }
  float M = lv[0];
#pragma unroll
  for (int s = 1; s < kNarrow; ++s) M = fmaxf(M, lv[s]);
  const float Mb = (M == kNegInf) ? 0.f : M;   // all splits empty: every weight is exp2(-inf) = 0
  float acc[PER], wsum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
#pragma unroll
  for (int s = 0; s < kNarrow; ++s) {
    const float wgt = exp2_hw((lv[s] - Mb) * kLog2e);
    wsum += wgt;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += wgt * ov[s][i];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = PER * l + i;
    if (OUT_BF16)
      reinterpret_cast<bf16*>(o)[(size_t)row * D + d] = (bf16)(acc[i] * inv);
    else
      reinterpret_cast<float*>(o)[(size_t)row * D + d] = acc[i] * inv;
  }
  if (lse != nullptr && l == 0) lse[row] = wsum > 0.f ? M + __logf(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_combine_lse(const CombineArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq;
  const dim3 blk(256);
  if (a.max_splits <= kNarrow) {
    const dim3 g((unsigned)((rows + kWaves - 1) / kWaves));
#define SA_LAUNCH_N(DD, BF)                                                                                 \
  hipLaunchKernelGGL((combine_lse_narrow_kernel<DD, BF>), g, blk, 0, stream, a.part_o, a.part_lse,         \
                     a.num_splits, (int)rows, a.Hq, a.max_splits, a.o, a.lse)
    if (a.d == 128) {
      if (a.out_bf16) SA_LAUNCH_N(128, true); else SA_LAUNCH_N(128, false);
    } else {
      if (a.out_bf16) SA_LAUNCH_N(64, true); else SA_LAUNCH_N(64, false);
    }
#undef SA_LAUNCH_N
    return hipGetLastError();
  }
  const dim3 g((unsigned)rows);
#define SA_LAUNCH(DD, BF)                                                                                   \
  hipLaunchKernelGGL((combine_lse_kernel<DD, BF>), g, blk, 0, stream, a.part_o, a.part_lse, a.num_splits,      \
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
