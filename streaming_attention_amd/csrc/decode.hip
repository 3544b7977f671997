// Split-KV decode for gfx950: one query token per sequence, the valid key
// range cut into contiguous splits, one normalised partial (lse, O) per split.
//
// Method: "ADR-0060: AHBM GQA Fused Attention kernel (Llama3-70B)", section
// 5.2 (decode attends to all past keys, only the ragged last tile is masked;
// the G query rows of a KV head are stacked into the GEMM M dimension so each
// K/V byte is read once for all of them), sections 4 and 5.3 (each split sweeps
// its own key range with the per-tile online softmax of section 3 and yields
// (m_i, l_i, O_i)), section 2.1 (splits are contiguous key blocks).
//
// MI355X mapping
//   * One workgroup per (sequence, KV head, split), 4 waves, the splits of a
//     (sequence, KV head) on one XCD when the groups divide evenly.  The split's keys
//     are taken 32 at a time; wave w handles chunks w, w + 4, ...  Each wave
//     keeps its own running (m, l, O) and double-buffers its next chunk's K and
//     V in registers (non-temporal loads: every byte is read exactly once), so
//     every wave has 16 KB of loads in flight while it computes.  At the end
//     the four wave states are merged through LDS with the same log-sum-exp
//     rule as the split merge.
//   * Scores are S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows loaded
//     coalesced, whole 256-byte rows per 16 lanes, staged through a per-wave
//     LDS region and read back as the A operand; Q of the G <= 16 heads as the
//     B operand, zero-padded to 16 columns).  Each lane owns one query column
//     and 8 of the chunk's 32 keys; the other keys of that query sit in lanes
//     l ^ 16, l ^ 32, l ^ 48.
//   * O^T += V^T P^T: P^T is 8 accumulator registers of S^T rounded to bf16;
//     V^T comes from a per-wave LDS region that V is written into transposed
//     (8-byte writes of 4 keys, key order permuted to match P^T).
#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kWaves = 4;           // waves per workgroup
constexpr bool kKViaLds = true;     // K loaded row-coalesced and staged through LDS
constexpr int kChunk = 32;          // keys per wave iteration
constexpr int kSplitGranule = 64;   // split boundaries are multiples of this

template <int D>
struct DecodeCfg {
  static constexpr int DS = D / 32;          // S^T MFMA steps over d
  static constexpr int DB = D / 16;          // 16-row d blocks of O^T
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int LQ = 64 / CPR;        // lanes sharing a chunk column
  static constexpr int NGRP = 8 / LQ;        // 4-key groups per lane (2 or 1)
  static constexpr int VTP = kChunk + 8;     // V^T row pitch (elements), 80 B
  static constexpr int VT_ELEMS = D * VTP;   // per wave
  static constexpr int KP = D + 8;           // K row pitch in LDS (elements), 16 B pad
  static constexpr int K_ELEMS = kKViaLds ? kChunk * KP : 0;   // per wave
  static constexpr int K_RPI = 64 / CPR;     // K rows per coalesced load instruction
};

// A split's partial is written with a plain store, or with a device-scope store
// when the same launch merges it (see arrive_and_merge).
template <bool DEVICE_SCOPE>
__device__ __forceinline__ void publish(float* p, float v) {
  if constexpr (DEVICE_SCOPE) st_dev(p, v); else *p = v;
}

// Fused merge (attn_decode).  Every split workgroup of a (sequence, KV head)
// publishes its partials and counts itself in; the one that arrives last merges
// the group's n partials with the log-sum-exp rule (M = max lse_s,
// w_s = e^{lse_s - M}, O = sum w_s O_s / sum w_s, LSE = M + ln sum w_s) and
// resets the counter for the next call.  Nothing waits: a workgroup that is not
// last simply exits ("ADR-0060: AHBM GQA Fused Attention kernel", section 4.3:
// nodes merge as their children arrive and the root normalises once).
//
// Publication without a device-wide fence (which on this multi-XCD part writes
// back and invalidates the whole L2 of the workgroup's XCD): the partials are
// written with device-scope (sc1) stores, every thread waits until its stores
// have completed, the workgroup synchronises, and one relaxed device-scope
// atomic counts it in.  The last arriver reads the partials with device-scope
// loads, so no stale L2 copy from an earlier call can be returned.
template <int D, int NT>
__device__ void arrive_and_merge(unsigned char* smem, int32_t* counters, const float* part_o,
                                 const float* part_lse, bf16* o, float* lse, int b, int kvh, int Hkv, int G,
                                 size_t head0, int n, int max_splits) {
  constexpr int DQ = D / 4;          // 16-byte column groups of a partial row
  constexpr int kBatch = 32;         // partial rows in flight per thread
  const int tid = threadIdx.x;
  __shared__ int is_last;
  __builtin_amdgcn_s_waitcnt(0);     // this thread's device-scope partial stores have completed
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(&counters[b * Hkv + kvh], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              n - 1;
  __syncthreads();
  if (!is_last) return;

  // Split weights of each head into LDS: w[j][s] = e^{lse_js - M_j}.
  float* wts = reinterpret_cast<float*>(smem);            // [G][n]
  float* Mh = wts + G * n;                                 // [G]
  float* Wsum = Mh + G;                                    // [G]
  for (int i = tid; i < G * n; i += NT)
    wts[i] = ld_dev(part_lse + (head0 + i / n) * max_splits + i % n);
  __syncthreads();
  if (tid < G) {
    float M = kNegInf;
    for (int s2 = 0; s2 < n; ++s2) M = fmaxf(M, wts[tid * n + s2]);
    Mh[tid] = M;
  }
  __syncthreads();
  for (int i = tid; i < G * n; i += NT) {
    const float M = Mh[i / n];
    wts[i] = M == kNegInf ? 0.f : exp2_hw((wts[i] - M) * kLog2e);
  }
  __syncthreads();
  if (tid < G) {
    float ws = 0.f;
    for (int s2 = 0; s2 < n; ++s2) ws += wts[tid * n + s2];
    Wsum[tid] = ws;
    if (lse != nullptr) lse[head0 + tid] = ws > 0.f ? Mh[tid] + __logf(ws) : kNegInf;
  }
  __syncthreads();

  // O[j][4 dq .. 4 dq + 3] = sum_s w[j][s] O_s[j][...] / sum_s w[j][s].
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(part_o + head0 * max_splits * D, (uint32_t)(G * max_splits * D * 4));
  for (int item = tid; item < G * DQ; item += NT) {
    const int j = item / DQ, dq = item % DQ;
    const uint32_t voff = (uint32_t)((j * max_splits * D + 4 * dq) * 4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += kBatch) {
      f32x4 x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        x[u] = (s0 + u < n) ? buf_ld16_dev(rp, voff, (uint32_t)((s0 + u) * D * 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float wgt = (s0 + u < n) ? wts[j * n + s0 + u] : 0.f;
        acc += wgt * x[u];
      }
    }
    const float ws = Wsum[j];
    const float inv = ws > 0.f ? 1.f / ws : 0.f;
    const uint32_t lo2 = pack_lo(__builtin_bit_cast(uint16_t, (bf16)(acc[0] * inv)),
                                 __builtin_bit_cast(uint16_t, (bf16)(acc[1] * inv)));
    const uint32_t hi2 = pack_lo(__builtin_bit_cast(uint16_t, (bf16)(acc[2] * inv)),
                                 __builtin_bit_cast(uint16_t, (bf16)(acc[3] * inv)));
    u32x2 pr = {lo2, hi2};
    *reinterpret_cast<u32x2*>(o + (head0 + j) * D + 4 * dq) = pr;
  }
  if (tid == 0)   // ready for the next call
    __hip_atomic_store(&counters[b * Hkv + kvh], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool FUSED, int NW>
__global__ __launch_bounds__(64 * NW, 2) void decode_splitkv_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ num_splits, int Hq,
    int Hkv, int S_cap, int max_splits, float c, float* __restrict__ part_o,
    float* __restrict__ part_lse, int32_t* __restrict__ counters, bf16* __restrict__ o,
    float* __restrict__ lse) {
  using C = DecodeCfg<D>;
  constexpr int kThreads = 64 * NW;
  constexpr int MERGE_FLOATS = NW * 16 * D + 2 * NW * 16;
  constexpr int SMEM_BYTES_VT = NW * (C::VT_ELEMS + C::K_ELEMS) * 2;
  constexpr int SMEM_BYTES = SMEM_BYTES_VT > MERGE_FLOATS * 4 ? SMEM_BYTES_VT : MERGE_FLOATS * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];

  // Workgroups are dealt to the 8 XCDs round robin.  When the (sequence, KV
  // head) groups come in multiples of 8, every split of group gi runs on XCD
  // gi % 8, so a group's key range streams through one XCD and its partials
  // sit in that XCD's L2 for the merge (which places its row blocks to match).
  int wg = blockIdx.x;
  if (((gridDim.x / max_splits) & 7) == 0) {
    const int xcd = wg & 7, j = wg >> 3;
    wg = (8 * (j / max_splits) + xcd) * max_splits + j % max_splits;
  }
  const int s = wg % max_splits;
  const int kvh = (wg / max_splits) % Hkv;
  const int b = wg / (max_splits * Hkv);
  const int G = Hq / Hkv;

  int len = kv_len ? kv_len[b] : S_cap;
  len = len < 0 ? 0 : (len > S_cap ? S_cap : len);
  int n = num_splits ? num_splits[b] : max_splits;
  n = n < 1 ? 1 : (n > max_splits ? max_splits : n);
  if (s >= n) return;
  const int per = (len + n - 1) / n;
  const long long chunk = (long long)((per + kSplitGranule - 1) / kSplitGranule) * kSplitGranule;
  const long long lo_ll = (long long)s * chunk;
  const int lo = lo_ll < len ? (int)lo_ll : len;
  const int hi = (int)((lo_ll + chunk) < len ? (lo_ll + chunk) : len);

  const int tid = threadIdx.x;
  const size_t head0 = (size_t)b * Hq + (size_t)kvh * G;
  if (lo >= hi) {
    // Empty split: (lse, O) = (-inf, 0).
    for (int i = tid; i < G * D; i += kThreads) {
      const int j = i / D, d = i % D;
      publish<FUSED>(part_o + ((head0 + j) * max_splits + s) * D + d, 0.f);
      if (d == 0) publish<FUSED>(part_lse + (head0 + j) * max_splits + s, kNegInf);
    }
    if constexpr (FUSED) arrive_and_merge<D, kThreads>(smem, counters, part_o, part_lse, o, lse, b, kvh, Hkv, G, head0, n,
                                              max_splits);
    return;
  }

  const int w = tid >> 6, l = tid & 63;
  const int j16 = l & 15;     // query column of this lane
  const int qq = l >> 4;      // which 4-key group of each 16-key block
  const size_t kvoff = ((size_t)b * Hkv + kvh) * (size_t)S_cap * D;
  const bf16* kg = kc + kvoff;
  const bf16* vg = vc + kvoff;

  // Q^T B operand: lane holds Q[head j16][32 s + 8 qq .. +7], zero past G.
  bf16x8 qf[C::DS];
#pragma unroll
  for (int st = 0; st < C::DS; ++st) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (j16 < G) x = ld16(q + (head0 + j16) * D + 32 * st + 8 * qq);
    qf[st] = as_bf16x8(x);
  }

  // V staging map: chunk column vcol (d = 8 vcol .. +7), key groups vgrp[g].
  const int vcol = l / C::LQ;
  const int vsub = l % C::LQ;

  struct Regs {
    u32x4 k[2][C::DS];
    u32x4 v[C::NGRP][4];
  };

  // Keys past the split end are read clamped to its last key (finite data,
  // masked to -inf in the scores, so P = 0 for them); cache slots at or past
  // kv_len are never touched.  Unconditional loads let the next chunk's loads
  // stay in flight while the current one is processed.  K/V are streamed once,
  // so the loads are non-temporal.
  auto load_chunk = [&](Regs& R, int key0) {
    if constexpr (kKViaLds) {
      // Whole 16-byte columns of full rows per instruction: K_RPI rows each.
#pragma unroll
      for (int i = 0; i < 2 * C::DS; ++i) {
        const int key = min(key0 + l / C::CPR + C::K_RPI * i, hi - 1);
        R.k[i / C::DS][i % C::DS] = ld16_nt(kg + (size_t)key * D + 8 * (l % C::CPR));
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = min(key0 + 16 * kb + j16, hi - 1);
#pragma unroll
        for (int st = 0; st < C::DS; ++st) R.k[kb][st] = ld16_nt(kg + (size_t)key * D + 32 * st + 8 * qq);
      }
    }
#pragma unroll
    for (int g = 0; g < C::NGRP; ++g) {
      const int kgid = vsub + C::LQ * g;   // 4-key group index 0..7 inside the chunk
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(key0 + 4 * kgid + r, hi - 1);
        R.v[g][r] = ld16_nt(vg + (size_t)key * D + 8 * vcol);
      }
    }
  };

  bf16* VT = reinterpret_cast<bf16*>(smem) + w * (C::VT_ELEMS + C::K_ELEMS);
  bf16* KL = VT + C::VT_ELEMS;   // per-wave K rows (only with kKViaLds)

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = __builtin_amdgcn_readfirstlane((hi - lo + kChunk - 1) / kChunk);

  auto process = [&](const Regs& R, int ci) {
    const int key0 = lo + ci * kChunk;

    // S^T for keys key0 + 16 kb + (0..15).
    f32x4 sacc[2];
    if constexpr (kKViaLds) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 2 * C::DS; ++i)
        st16(KL + (l / C::CPR + C::K_RPI * i) * C::KP + 8 * (l % C::CPR), R.k[i / C::DS][i % C::DS]);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < C::DS; ++st) {
        bf16x8 a;
        if constexpr (kKViaLds)
          a = *reinterpret_cast<const bf16x8*>(KL + (16 * kb + j16) * C::KP + 32 * st + 8 * qq);
        else
          a = as_bf16x8(R.k[kb][st]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[st], sacc[kb], 0, 0, 0);
      }
    }
    if (key0 + kChunk > hi) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 16 * kb + 4 * qq + r;
          sacc[kb][r] = key < hi ? sacc[kb][r] : kNegInf;
        }
    }

    // V -> LDS, transposed: row d, key position 8 q + 4 kb + r.  The wave's
    // previous reads of this region must be complete before it is rewritten.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < C::NGRP; ++g) {
      const int kgid = vsub + C::LQ * g;
      const int p0 = 8 * (kgid & 3) + 4 * (kgid >> 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        uint32_t a, bq;
        if (e & 1) {
          a = pack_hi(R.v[g][0][dw], R.v[g][1][dw]);
          bq = pack_hi(R.v[g][2][dw], R.v[g][3][dw]);
        } else {
          a = pack_lo(R.v[g][0][dw], R.v[g][1][dw]);
          bq = pack_lo(R.v[g][2][dw], R.v[g][3][dw]);
        }
        u32x2 pr = {a, bq};
        *reinterpret_cast<u32x2*>(VT + (8 * vcol + e) * C::VTP + p0) = pr;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // Online softmax over the chunk (base 2), row reduction over the 4 lanes
    // that share this query column.
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float corr = exp2_hw(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2_hw(__builtin_fmaf(sacc[kb][r], c, -m_use));
        sacc[kb][r] = p;
        psum += p;
      }
    l_run = l_run * corr + psum;
    m_run = m_new;
    const bf16x8 pf = to_bf16x8(sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3], sacc[1][0], sacc[1][1],
                                sacc[1][2], sacc[1][3]);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      oacc[db] *= corr;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(VT + (16 * db + j16) * C::VTP + 8 * qq);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[db], 0, 0, 0);
    }
  };

  // Two register buffers in ping-pong, no copies between them, so the next
  // chunk's loads stay in flight while the current chunk is processed.
  Regs ra, rb;
  int ci = w;
  if (ci < nch) load_chunk(ra, lo + ci * kChunk);
  if (ci + NW < nch) load_chunk(rb, lo + (ci + NW) * kChunk);
  while (ci < nch) {
    process(ra, ci);
    if (ci + 2 * NW < nch) load_chunk(ra, lo + (ci + 2 * NW) * kChunk);
    ci += NW;
    if (ci >= nch) break;
    process(rb, ci);
    if (ci + 2 * NW < nch) load_chunk(rb, lo + (ci + 2 * NW) * kChunk);
    ci += NW;
  }

  // Row sum over the 4 lanes of the query column.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // Merge the 4 wave states through LDS.
  __syncthreads();
  float* Ow = reinterpret_cast<float*>(smem);       // [NW][16][D] unnormalised O
  float* mw = Ow + NW * 16 * D;                       // [NW][16]
  float* lw = mw + NW * 16;                           // [NW][16]
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) Ow[(w * 16 + j16) * D + 16 * db + 4 * qq + r] = oacc[db][r];
  if (l < 16) {
    mw[w * 16 + l] = m_run;
    lw[w * 16 + l] = l_run;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int j = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mw[ww * 16 + j]);
    float osum = 0.f, wsum = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float f = exp2_hw(mw[ww * 16 + j] - M);
        wsum += f * lw[ww * 16 + j];
        osum += f * Ow[(ww * 16 + j) * D + d];
      }
    }
    const bool has = wsum > 0.f;
    publish<FUSED>(part_o + ((head0 + j) * max_splits + s) * D + d, has ? osum / wsum : 0.f);
    if (d == 0) publish<FUSED>(part_lse + (head0 + j) * max_splits + s, has ? (M + __log2f(wsum)) * kLn2 : kNegInf);
  }
  if constexpr (FUSED) {
    __syncthreads();   // the merge below reuses the LDS staging area
    arrive_and_merge<D, kThreads>(smem, counters, part_o, part_lse, o, lse, b, kvh, Hkv, G, head0, n, max_splits);
  }
}

}  // namespace

hipError_t launch_decode_splitkv(const DecodeArgs& a, hipStream_t stream) {
  const long long grid = (long long)a.B * a.Hkv * a.max_splits;
  const float c = a.scale * kLog2e;
  const dim3 g((unsigned)grid), blk(64 * kWaves);
  const bool fused = a.counters != nullptr;
#define SA_LAUNCH(DD, FF)                                                                                   \
  hipLaunchKernelGGL((decode_splitkv_bf16_kernel<DD, FF, kWaves>), g, blk, 0, stream, (const bf16*)a.q,    \
                     (const bf16*)a.k, (const bf16*)a.v, a.kv_len, a.num_splits, a.Hq, a.Hkv, a.S_cap,      \
                     a.max_splits, c, a.part_o, a.part_lse, a.counters, (bf16*)a.o, a.lse)
  if (a.d == 128) {
    if (fused) SA_LAUNCH(128, true); else SA_LAUNCH(128, false);
  } else {
    if (fused) SA_LAUNCH(64, true); else SA_LAUNCH(64, false);
  }
#undef SA_LAUNCH
  return hipGetLastError();
}

}  // namespace sa
