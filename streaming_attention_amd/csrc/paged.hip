// Multi-token decode over a paged KV cache, for small query blocks (the G
// query heads of a KV head times the T_q new tokens of a sequence stack into at
// most 32 rows), on gfx950.
//
// Method: "ADR-0060: AHBM GQA Fused Attention kernel (Llama3-70B)", section
// 0.5.3 (the query block carries its start and length: q_start = kv_len - T_q,
// bottom-right causal), sections 2.1-2.2 (a sequence's keys sit in blocks that
// plain arithmetic maps back to positions -- here pages found through a block
// table -- and the valid length comes from a counter), section 5.2 (the G query
// heads of one KV head stacked into the GEMM M dimension, so every K/V byte is
// read once for all of them; here the T_q tokens stack in as well), section 3
// (per-tile online softmax) and section 4 (split partials merged by
// log-sum-exp).
//
// MI355X mapping
//   * Memory bound: every valid K/V byte is read once, so the kernel is built
//     like the contiguous split-KV decode: one workgroup per (sequence, KV
//     head, split), 4 waves, two workgroups per CU.  Wave w takes the split's
//     32-key chunks w, w + 4, ...; a chunk lies inside one 64-key page, whose
//     pool index is one scalar load from the block table.  The chunk's K and V
//     rows are loaded into registers (non-temporal, whole 256-byte rows per 16
//     lanes), written to the wave's own LDS region, and the wave then issues
//     the loads of its next chunk before it computes this one, so they are in
//     flight meanwhile.  Rows past the split end repeat its last key (finite
//     data, masked out), so pool rows past a sequence's length are never read.
//   * The <= 32 stacked rows (row = g T_q + t) are the N dimension of
//     v_mfma_f32_32x32x16_bf16, as in the prefill kernel: S^T = K Q^T with K
//     fragments read from LDS and Q^T held in registers; O^T += V^T P^T with
//     V^T from the transposing LDS read and P^T straight from the score
//     accumulators rounded to bf16.  Each lane owns one row.
//   * Softmax in base 2 against a fixed exponent base per row (the row max of
//     the wave's first chunk), raised only when a chunk's partial row sum
//     passes 2^24; that chunk's scores are then recomputed from its K, still
//     in LDS.  Masks (split end, causal tail) are selects to -inf on the
//     chunks that need them.
//   * The four wave states are merged through LDS at the end of the split
//     with the log-sum-exp rule; the split writes its normalised partial, or
//     O and LSE directly when there is one split.
#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kPW = 4;                 // waves per workgroup
constexpr int kPC = 32;                // keys per chunk
constexpr int kPage = 64;              // positions per page
constexpr float kPSumCap = 16777216.f;  // 2^24: largest partial row sum of a chunk kept without raising the base

template <int D>
__global__ __launch_bounds__(64 * kPW, 2) void decode_paged_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kpool, const bf16* __restrict__ vpool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ seq_splits, int B, int Hq, int Hkv, int T_q, int num_pages, int max_pages,
    int n_splits, float c, float* __restrict__ part_o, float* __restrict__ part_lse, bf16* __restrict__ o,
    float* __restrict__ lse) {
  constexpr int NT = 64 * kPW;
  constexpr int RB = 2 * D;            // bytes per K / V row
  constexpr int U = D / 8;             // 16-byte units per row
  constexpr int CB = kPC * RB;         // bytes of one chunk of K (or of V)
  constexpr int NL = kPC * U / 64;     // 16-byte loads per lane per chunk, for K and again for V
  constexpr int DS = D / 16;           // score MFMAs per chunk
  constexpr int DB = D / 32;           // 32-row d blocks of O^T
  constexpr int STAGE = kPW * 2 * CB;
  constexpr int MERGE = (kPW * 32 * D + 2 * kPW * 32) * 4;
  static_assert(NL * 64 == kPC * U, "a chunk is a whole number of wave loads");
  // Swizzles of the prefill kernel (64 LDS banks): K unit u of row r at
  // u ^ sk(r), V 32-byte unit h of row r at h ^ sv(r).
  auto sk = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto sv = [](int r) { return D == 128 ? 2 * (r & 3) : 2 * ((r >> 1) & 1); };
  __shared__ __attribute__((aligned(1024))) char smem[STAGE > MERGE ? STAGE : MERGE];
  __shared__ int len_s[kRankMax];
  __shared__ int pick;

  // Workgroup -> (sequence slot, split, KV head); slot r is the sequence of
  // rank r by length, longest first.
  const int per_seq = Hkv * n_splits;
  const int s = (blockIdx.x % per_seq) / Hkv;
  const int kvh = blockIdx.x % Hkv;
  const int cap = kPage * max_pages;
  const int b = seq_of_rank<NT>(kv_len, B, cap, blockIdx.x / per_seq, len_s, &pick);
  int len = kv_len[b];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  int n_b = n_splits;
  if (seq_splits != nullptr) {
    n_b = seq_splits[b];
    n_b = n_b < 1 ? 1 : (n_b > n_splits ? n_splits : n_b);
    if (s >= n_b) return;   // uniform over the workgroup
  }
  // Split s: keys [64 s c, min(64 (s + 1) c, len)), c = ceil(ceil(len / 64) / n_b).
  const int tiles = (len + kPage - 1) / kPage;
  const int per = (tiles + n_b - 1) / n_b;
  const int lo = min(len, s * per * kPage);
  const int hi = min(len, (s + 1) * per * kPage);

  const int G = Hq / Hkv;
  const int R = G * T_q;               // stacked rows, <= 32
  const int q_start = len - T_q;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lr = l & 31;               // the stacked row this lane owns
  const int hf = l >> 5;               // which half of the keys / d chunk the lane holds
  const bool row_ok = lr < R;
  const int pos = q_start + (row_ok ? lr % T_q : 0);
  // Output row of stacked row j: (b, head kvh G + j / T_q, token j % T_q).
  auto flat_row = [&](int j) { return ((size_t)b * Hq + (size_t)kvh * G + j / T_q) * T_q + j % T_q; };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;

  const int nch = __builtin_amdgcn_readfirstlane((hi - lo + kPC - 1) / kPC);
  if (nch > 0) {
    // Q^T B operands: lane holds Q[row lr][16 st + 8 hf .. + 7]; zero past R.
    bf16x8 qf[DS];
    const bf16* qrow = q + (row_ok ? flat_row(lr) : 0) * D;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_ok) x = ld16(qrow + 16 * st + 8 * hf);
      qf[st] = as_bf16x8(x);
    }

    u32x4 rk[NL], rv[NL];
    auto load = [&](int ci) __attribute__((always_inline)) {
      const int key0 = lo + ci * kPC;
      int pg = block_table[(size_t)b * max_pages + key0 / kPage];
      pg = pg < 0 ? 0 : (pg >= num_pages ? num_pages - 1 : pg);
      const size_t base = (((size_t)pg * Hkv + kvh) * kPage + key0 % kPage) * D;
      const int last = min(kPC, hi - key0) - 1;   // rows past the split end repeat its last key
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int p = 64 * i + l, r = min(p / U, last), u = p % U;
        rk[i] = ld16_nt(kpool + base + (size_t)r * D + 8 * u);
        rv[i] = ld16_nt(vpool + base + (size_t)r * D + 8 * u);
      }
    };
    lds_t* const KL = (lds_t*)smem + w * 2 * CB;
    lds_t* const VL = KL + CB;
    // Registers -> this wave's LDS region (only this wave reads it).
    auto stage = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int p = 64 * i + l, r = p / U, u = p % U;
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(KL + r * RB + 16 * (u ^ sk(r))) = rk[i];
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(VL + r * RB + 32 * ((u >> 1) ^ sv(r)) +
                                                                    16 * (u & 1)) = rv[i];
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    };
    // Operand read offsets (as in the prefill kernel).
    uint32_t k_rd[DS];
#pragma unroll
    for (int st = 0; st < DS; ++st) k_rd[st] = (uint32_t)(lr * RB + 16 * ((2 * st + hf) ^ sk(lr)));
    const int g4 = l >> 4, jj = l & 15;
    const int vrow = 4 * (g4 >> 1) + (jj >> 2);
    uint32_t v_rd[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_rd[db] = (uint32_t)(vrow * RB + 32 * ((2 * db + (g4 & 1)) ^ sv(vrow)) + 8 * (jj & 3));

    f32x16 S;
    auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < DS; ++st)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read16(KL + k_rd[st]), qf[st], st == 0 ? f32x16{} : S, 0, 0,
                                                    0);
    };
    // Accumulator register r holds key 8 (r / 4) + 4 hf + r % 4 of the chunk.
    auto mask = [&](int key0) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        S[r] = (key < hi && key <= pos) ? S[r] : kNegInf;
      }
    };
    auto row_max = [&]() __attribute__((always_inline)) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = fmaxf(S[i], S[i + 8]);
#pragma unroll
      for (int wd = 4; wd >= 1; wd >>= 1)
#pragma unroll
        for (int i = 0; i < wd; ++i) t[i] = fmaxf(t[i], t[i + wd]);
      return max_xor32(t[0]) * c;
    };
    float m_use = 0.f;
    auto exponentiate = [&]() __attribute__((always_inline)) {
      float t[8];
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = exp2_hw(__builtin_fmaf(S[r], c, -m_use));
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = S[i] + S[i + 8];
#pragma unroll
      for (int wd = 4; wd >= 1; wd >>= 1)
#pragma unroll
        for (int i = 0; i < wd; ++i) t[i] = t[i] + t[i + wd];
      return t[0];
    };

    int ci = w;
    bool first = true;
    if (ci < nch) load(ci);
    while (ci < nch) {
      stage();
      if (ci + kPW < nch) load(ci + kPW);   // in flight while this chunk is computed
      const int key0 = lo + ci * kPC;
      const bool need_mask = key0 + kPC > hi || key0 + kPC - 1 > q_start;
      scores();
      if (need_mask) mask(key0);
      if (first) {   // the exponent base: this wave's first chunk's row max
        m_run = row_max();
        m_use = m_run == kNegInf ? 0.f : m_run;
        first = false;
      }
      float psum = exponentiate();
      if (__builtin_amdgcn_ballot_w64(!(psum <= kPSumCap))) {   // rare; also catches inf / NaN
        scores();
        if (need_mask) mask(key0);
        const float m_new = fmaxf(m_run, row_max());
        const float corr = m_new == kNegInf ? 1.f : exp2_hw(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[i][j] *= corr;
        m_run = m_new;
        m_use = m_run == kNegInf ? 0.f : m_run;
        psum = exponentiate();
      }
      l_run += psum;
      // P^T operands: slot e of key chunk cc is accumulator register 8 cc + e.
      bf16x8 pf[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        pf[cc] = to_bf16x8(S[8 * cc + 0], S[8 * cc + 1], S[8 * cc + 2], S[8 * cc + 3], S[8 * cc + 4], S[8 * cc + 5],
                           S[8 * cc + 6], S[8 * cc + 7]);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const lds_t* vp = VL + 16 * cc * RB + v_rd[db];
          const s16x4 v0 = lds_read_tr16(vp), v1 = lds_read_tr16(vp + 8 * RB);
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[cc], oacc[db], 0, 0, 0);
        }
      ci += kPW;
    }
  }
  const float l_tot = sum_xor32(l_run);   // the row's sum over both halves of its keys

  // Merge the wave states through LDS: M = max_w m_w, weights 2^(m_w - M).
  __syncthreads();   // the staging regions are reused
  float* Ow = reinterpret_cast<float*>(smem);   // [kPW][32][D] unnormalised O
  float* mw = Ow + kPW * 32 * D;                // [kPW][32]
  float* lw = mw + kPW * 32;                    // [kPW][32]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) Ow[(w * 32 + lr) * D + 32 * db + 8 * (r >> 2) + 4 * hf + (r & 3)] = oacc[db][r];
  if (hf == 0) {
    mw[w * 32 + lr] = m_run;
    lw[w * 32 + lr] = l_tot;
  }
  __syncthreads();
  for (int i = tid; i < R * D; i += NT) {
    const int j = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kPW; ++ww) M = fmaxf(M, mw[ww * 32 + j]);
    float osum = 0.f, wsum = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < kPW; ++ww) {
        const float f = exp2_hw(mw[ww * 32 + j] - M);
        wsum += f * lw[ww * 32 + j];
        osum += f * Ow[(ww * 32 + j) * D + d];
      }
    }
    const bool has = wsum > 0.f;
    const float ov = has ? osum / wsum : 0.f;
    const float lv = has ? (M + __log2f(wsum)) * kLn2 : kNegInf;
    const size_t fr = flat_row(j);
    if (part_o != nullptr) {
      part_o[(fr * n_splits + s) * D + d] = ov;
      if (d == 0) part_lse[fr * n_splits + s] = lv;
    } else {
      o[fr * D + d] = (bf16)ov;
      if (d == 0 && lse != nullptr) lse[fr] = lv;
    }
  }
}

}  // namespace

bool decode_paged_fits(int Hq, int Hkv, int T_q, int d) {
  return (d == 64 || d == 128) && (long long)(Hq / Hkv) * T_q <= 32;
}

hipError_t launch_decode_paged(const PrefillArgs& a, hipStream_t stream) {
  const long long grid = (long long)a.B * a.Hkv * a.n_splits;
  const float c = a.scale * kLog2e;
  const dim3 g((unsigned)grid), blk(64 * kPW);
#define SA_LAUNCH(DD)                                                                                          \
  hipLaunchKernelGGL((decode_paged_bf16_kernel<DD>), g, blk, 0, stream, (const bf16*)a.q, (const bf16*)a.k,    \
                     (const bf16*)a.v, a.block_table, a.kv_len, a.seq_splits, a.B, a.Hq, a.Hkv, a.Sq,          \
                     a.num_pages, a.max_pages, a.n_splits, c, a.part_o, a.part_lse, (bf16*)a.o, a.lse)
  if (a.d == 128) SA_LAUNCH(128); else SA_LAUNCH(64);
#undef SA_LAUNCH
  return hipGetLastError();
}

}  // namespace sa
