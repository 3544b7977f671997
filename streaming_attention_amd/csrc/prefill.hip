// Fused streaming attention forward (prefill) for gfx950.
//
// Method: "ADR-0060: AHBM GQA Fused Attention kernel (Llama3-70B)", section 3
// (per KV tile: scores, boundary mask, tile max, new running max, P = exp(S - m),
// correction exp(m_old - m_new), l = l*corr + rowsum P, O = O*corr + P V),
// section 5.2 (the G query heads of one KV head stacked into the GEMM M
// dimension, so one K/V tile serves all of them) and section 5.4 (tiles wholly
// after the query block skipped, straddling tiles masked).  "AttentionRegion
// Transformation" sections 6-8 give the same loop: Q tile resident, K/V tiles
// streamed HBM -> shared memory -> registers, S and P never written out.
//
// MI355X mapping (bf16 path)
//   * One workgroup = 8 waves = 256 stacked query rows of one (batch, KV head)
//     when there are enough such blocks to give every CU one, else 4 waves =
//     128 rows (two workgroups per CU); each wave owns 32 rows.  In the 8-wave
//     launch with G a multiple of 8 the 256 rows are the same 32 positions of
//     8 query heads, so all waves see the same causal extent.  KV tiles of
//     64 keys go from global memory straight into LDS (buffer loads with the
//     LDS destination, no register staging) while earlier tiles are computed.
//     The 8-wave launches run the two-team kernel (prefill_pp_kernel below):
//     the two waves of every SIMD alternate between the MFMA work and the
//     softmax work of their tiles, in step through workgroup barriers.  The
//     4-wave and paged launches run prefill_bf16_kernel, in which each wave
//     interleaves both kinds of work itself and one barrier per tile orders
//     a double-buffered ring.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K (from LDS) is the A operand and Q (held in VGPRs for the whole sweep)
//     the B operand.  In the accumulator layout every lane then owns ONE query
//     row (column l % 32) and 32 of the tile's 64 keys; its partner lane l ^ 32
//     holds the other 32.  Running max, running sum and the output rescale are
//     therefore per-lane scalars, and a row reduction is a local reduction plus
//     one exchange with the partner lane.
//   * The output is accumulated transposed too, O^T += V^T P^T: V^T is the A
//     operand, P^T the B operand.  The B operand of an MFMA needs, per lane, 8
//     reduction (key) indices of one query -- 8 accumulator registers of S^T,
//     so P goes from the score accumulators to the P V operand with no data
//     movement.  V stays row-major in LDS; the transposing LDS read of gfx950
//     (ds_read_b64_tr_b16) delivers the matching V^T fragments.
//   * Softmax runs in base 2: c = scale * log2(e) is folded into one FMA before
//     v_exp_f32, against a fixed exponent base per row (the first tile's max,
//     raised only when a tile's probabilities grow large).  Masks are selects
//     to -inf, never additions, on straddling and tail tiles only.
//   * Work order: heaviest causal tiles first, and when the number of
//     (batch, KV head) groups is a multiple of 8, every group's tiles go to one
//     XCD (workgroups are dealt to the 8 XCDs round robin) so its K/V stays in
//     that XCD's L2.  Split-KV mode (a key range per workgroup, fp32 partials)
//     and paged mode (multi-token decode over a page pool, longest sequences
//     first) reuse the same loop; see the notes above the kernel.
//
// fp32 path: the same loop with v_mfma_f32_32x32x2_f32 (one K value per lane
// per step, so V needs no transpose) and 32-key tiles, P kept in fp32.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kBM = 128;   // stacked query rows per workgroup (fp32 path)
constexpr int kBN = 64;    // keys per KV tile (bf16 path)
constexpr int kThreads = 256;
constexpr int kNumCUs = 256;          // MI355X compute units
constexpr float kSumCap = 16777216.f;  // 2^24: largest partial row sum of P accepted without
                                      // raising the exponent base (P <= 2^24 keeps O far from fp32 overflow)
constexpr int kLdsAhead = 4;          // LDS operand reads issued ahead of their MFMA

struct TileCoord {
  int b, kvh, mt, split;
};

// Workgroup index -> (batch, KV head, KV split, M tile).  A (batch, KV head,
// split) triple is a "group" here.  Heaviest M tiles (latest query positions)
// are dealt first; with n_groups % 8 == 0 each group is pinned to XCD
// (group % 8), so the workgroups that stream the same K/V range share an L2.
template <int BM>
__device__ __forceinline__ TileCoord map_tile(int wg, int n_groups, int n_splits, int Hkv, int n_mt, int G,
                                              int Sq) {
  int group, rk;
  if ((n_groups & 7) == 0) {
    const int xcd = wg & 7, slot = wg >> 3, gpx = n_groups >> 3;
    group = (slot % gpx) * 8 + xcd;
    rk = slot / gpx;
  } else {
    group = wg % n_groups;
    rk = wg / n_groups;
  }
  int mt;
  if (Sq % BM == 0) {
    const int n_pb = Sq / BM;          // position blocks per query head
    const int pb = n_pb - 1 - rk / G;  // latest positions first
    const int g = rk % G;
    mt = g * n_pb + pb;
  } else {
    mt = n_mt - 1 - rk;
  }
  TileCoord t;
  t.split = group % n_splits;
  group /= n_splits;
  t.b = group / Hkv;
  t.kvh = group % Hkv;
  t.mt = mt;
  return t;
}

// The same dealing for the two-team kernel's head-interleaved blocks (G a
// multiple of 8): block (hb, pb) holds positions 32 pb .. 32 pb + 31 of query
// heads 8 hb .. 8 hb + 7; the latest positions are dealt first.
__device__ __forceinline__ TileCoord map_tile_heads8(int wg, int n_groups, int n_splits, int Hkv, int n_hb,
                                                     int n_pb) {
  int group, rk;
  if ((n_groups & 7) == 0) {
    const int xcd = wg & 7, slot = wg >> 3, gpx = n_groups >> 3;
    group = (slot % gpx) * 8 + xcd;
    rk = slot / gpx;
  } else {
    group = wg % n_groups;
    rk = wg / n_groups;
  }
  TileCoord t;
  t.mt = (rk % n_hb) * n_pb + (n_pb - 1 - rk / n_hb);
  t.split = group % n_splits;
  group /= n_splits;
  t.b = group / Hkv;
  t.kvh = group % Hkv;
  return t;
}

// First / last valid stacked row of a row range and the smallest / largest
// query position t (row % Sq) inside it.
__device__ __forceinline__ void row_range_positions(int rA, int rB, int Sq, int& t_min, int& t_max) {
  if (rA / Sq == rB / Sq) {
    t_min = rA % Sq;
    t_max = rB % Sq;
  } else {
    t_min = 0;
    t_max = Sq - 1;
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel
//
// LDS tiles.  A K or V tile is kBN key rows of D bf16 values, row-major (2 D
// bytes a row, no padding), filled by direct global -> LDS buffer loads: one
// such load stores the 16 bytes fetched by lane l at byte 16 l of a 1 KB
// chunk, so which global bytes a lane fetches decides where they land.  Two
// XOR swizzles, applied through that choice, keep the operand reads free of
// bank conflicts on the 64 banks (256 bytes per clock) of the LDS:
//   K  16-byte unit u of row r is stored at unit u ^ sk(r), with sk(r) = r % 16
//      at D = 128 (256-byte rows) and (r / 2) % 8 at D = 64 (128-byte rows).
//      The score A-operand read (rows 32 kb .. 32 kb + 31, one unit each,
//      16 lanes per clock) then touches 16 different bank groups.
//   V  32-byte unit h of row r is stored at unit h ^ sv(r), with
//      sv(r) = 2 (r % 4) at D = 128 and 2 ((r / 2) % 2) at D = 64.  The P V
//      A-operand is read with ds_read_b64_tr_b16; 32 lanes (two 16-lane
//      groups) per clock read 4 rows x 2 adjacent 32-byte units, which then
//      fall on 8 different units.
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives
// as its element e (e = 0..3) element i % 4 of the 8 bytes addressed by lane
// 4 e + i / 4 of the group.  When the addressing lanes point at 4 consecutive
// d values of 4 key rows, every lane receives one d column over 4 keys: the
// transposed V operand, read straight from the row-major tile.
//
// QB = 32-row query blocks per wave, NW = waves per workgroup (32 * QB * NW
// stacked rows).  QB = 2 would halve the LDS bytes per MFMA (every K and V
// fragment read from LDS would feed two MFMAs) at one wave per SIMD, but it
// spills under the compiler's register allocation; the launches use QB = 1.
// ---------------------------------------------------------------------------
// 16 bytes per lane, global (buffer, byte offset voff + soff) -> LDS chunk dst
// (wave-uniform; lane l writes dst + 16 l).  Out-of-range bytes arrive as zero.
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, lds_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, reinterpret_cast<__attribute__((address_space(3))) void*>(dst), 16,
                                           voff, soff, 0, 0);
}
// Completion of this wave's direct-to-LDS loads (they count as vector memory
// loads); a workgroup barrier after it publishes the tiles to all waves.
__device__ __forceinline__ void wait_lds_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same wait as a compiler builtin (vmcnt 0, other counters unchanged:
// gfx9 encoding expcnt 7, lgkmcnt 15), so that the compiler's own wait
// insertion knows that every earlier vector memory load has completed.
__device__ __forceinline__ void wait_vm_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

template <int P>
using Parity = std::integral_constant<int, P>;

// Split-KV mode (part_o != nullptr): the workgroup covers only KV split
// tc.split -- tiles [s T, min((s + 1) T, all tiles)) with T = ceil(tiles /
// n_splits), intersected with the causal extent -- and writes the normalised
// fp32 partial (O over those keys, their LSE) in place of O and LSE.
//
// Paged mode (PAGED): multi-token decode over a paged cache.  k and v are page
// pools [num_pages, Hkv, kBN, D]; key tile kt of sequence b is pool page
// block_table[b * max_pages + kt] (clamped into the pool); the sequence holds
// kv_len[b] keys (clamped to [0, kBN * max_pages]) and its Sq query tokens are
// its last Sq positions, so q_start = kv_len[b] - Sq may be negative (rows
// before the first key see nothing).  Skv is unused.  Each tile gets its own
// buffer resource over the page's valid rows, so rows past kv_len read zero.
// seq_splits (paged mode, may be null): sequence b uses only its first
// seq_splits[b] (clamped to [1, n_splits]) splits, with the tile plan of that
// count; workgroups of its other splits exit at once.
template <int D, bool CAUSAL, int QB, int NW, bool PAGED>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 3 - QB : 1) void prefill_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int Sq, int Skv,
    float c, int n_splits, float* __restrict__ part_o, float* __restrict__ part_lse,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_len, int max_pages, int num_pages,
    const int32_t* __restrict__ seq_splits) {
  constexpr int NT = 64 * NW;               // threads per workgroup
  constexpr int BM = 32 * QB * NW;          // stacked query rows per workgroup
  constexpr int RW = 32 * QB;               // rows per wave
  constexpr int RB = 2 * D;                 // bytes per K / V row
  constexpr int U = D / 8;                  // 16-byte units per row
  constexpr int TB = kBN * RB;              // bytes per tile
  constexpr int NLD = kBN * U / NT;         // direct loads per thread per tile
  constexpr int DS = D / 16;                // MFMA k-steps over d for S^T
  constexpr int DB = D / 32;                // 32-row d blocks of O^T
  static_assert(NLD * NT == kBN * U, "a tile is a whole number of wave loads");
  auto sk = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto sv = [](int r) { return D == 128 ? 2 * (r & 3) : 2 * ((r >> 1) & 1); };

  // One array per ring slot: the compiler's wait-count analysis can then tell
  // a direct load in flight into one slot from reads of another.
  __shared__ __attribute__((aligned(1024))) char k_slot0[TB];
  __shared__ __attribute__((aligned(1024))) char k_slot1[TB];
  __shared__ __attribute__((aligned(1024))) char v_slot0[TB];
  __shared__ __attribute__((aligned(1024))) char v_slot1[TB];
  lds_t* const kbuf[2] = {(lds_t*)k_slot0, (lds_t*)k_slot1};
  lds_t* const vbuf[2] = {(lds_t*)v_slot0, (lds_t*)v_slot1};

  const int G = Hq / Hkv;
  const int rows_total = G * Sq;
  const int n_mt = (rows_total + BM - 1) / BM;
  const int n_groups = B * Hkv;
  TileCoord tc = map_tile<BM>(blockIdx.x, n_groups * n_splits, n_splits, Hkv, n_mt, G, Sq);
  const int r0 = tc.mt * BM;
  if constexpr (PAGED) {
    // map_tile deals the sequence slots in launch order; slot r is the
    // sequence of rank r by length, longest first.
    __shared__ int len_s[kRankMax];
    __shared__ int pick;
    const int cap = kBN * max_pages;
    tc.b = seq_of_rank<NT>(kv_len, B, cap, tc.b, len_s, &pick);
    const int len = kv_len[tc.b];
    Skv = len < 0 ? 0 : (len > cap ? cap : len);   // keys of this workgroup's sequence
  }
  const int q_start = Skv - Sq;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lr = l & 31;   // query column owned by this lane inside each row block
  const int hf = l >> 5;   // which half of the key set / d chunk the lane holds

  const size_t head0 = (size_t)tc.b * Hq + (size_t)tc.kvh * G;   // first query head of group
  const bf16* qg = q + head0 * Sq * D;
  const size_t kvoff = PAGED ? 0 : ((size_t)tc.b * Hkv + tc.kvh) * (size_t)Skv * D;

  // This lane's query rows (one per row block) and their global positions.
  int row[QB], pos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    row[qb] = r0 + RW * w + 32 * qb + lr;
    pos[qb] = q_start + (row[qb] < rows_total ? row[qb] % Sq : 0);
  }

  // Tile range of this workgroup (its KV split, cut at the causal extent) and
  // the mask-free bound per wave.
  int n_sp = n_splits;
  if (PAGED && seq_splits != nullptr) {
    n_sp = seq_splits[tc.b];
    n_sp = n_sp < 1 ? 1 : (n_sp > n_splits ? n_splits : n_sp);
    if (tc.split >= n_sp) return;   // uniform over the workgroup: before any barrier
  }
  const int tiles_all = (Skv + kBN - 1) / kBN;
  const int tiles_per_split = (tiles_all + n_sp - 1) / n_sp;
  int kt_lo = tc.split * tiles_per_split;
  int kt_hi = min(tiles_all, kt_lo + tiles_per_split);
  int wave_tmin = 0x3fffffff;
  // A wave whose rows all lie past the group's last row (small query blocks,
  // e.g. a few decode tokens) only helps load the tiles.
  const bool wave_active = r0 + RW * w < rows_total;
  // Causal: the workgroup sweeps to the last tile its latest row sees, but a
  // wave with earlier rows needs only tiles [kt_lo, wave_end): from step
  // wave_end + 1 on it only helps load tiles (step wave_end still runs: it
  // adds the P V product of tile wave_end - 1).
  int wave_end = 0x3fffffff;
  if (CAUSAL) {
    int tmin, tmax;
    row_range_positions(r0, min(r0 + BM - 1, rows_total - 1), Sq, tmin, tmax);
    const int vis_end = q_start + tmax + 1;   // keys seen by the block's last position
    kt_hi = min(kt_hi, vis_end > 0 ? (vis_end + kBN - 1) / kBN : 0);
    const int wA = r0 + RW * w, wB = min(r0 + RW * w + RW - 1, rows_total - 1);
    if (wA <= wB) {
      int a, bb;
      row_range_positions(wA, wB, Sq, a, bb);
      wave_tmin = a;
      const int wv_end = q_start + bb + 1;
      wave_end = wv_end > 0 ? (wv_end + kBN - 1) / kBN : 0;
    }
  }

  // Q^T B operands: lane holds Q[row][16 s + 8 hf .. +7] for s = 0 .. DS-1.
  // Buffer loads: rows past the group's last stacked row read as zero.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg, (uint32_t)rows_total * D * 2);
  bf16x8 qf[QB][DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[qb][s] = as_bf16x8(buf_ld16(rq, (uint32_t)row[qb] * D * 2 + 16 * hf + 32 * s, 0));

  // Direct loads: load j of this thread fills 16-byte unit p = 64 (4 j + w) + l
  // of the tile, i.e. row p / U, stored unit p % U; the source offsets undo the
  // swizzles.  Rows at or past Skv read as zero (their scores are masked to
  // -inf, so P = 0, and the zero V rows add nothing).  The tile advances through
  // the wave-uniform offset, so the loop spends no VALU on load addresses.
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kvoff, PAGED ? 0u : (uint32_t)Skv * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kvoff, PAGED ? 0u : (uint32_t)Skv * RB);
  // Paged mode: a resource over the valid rows of tile kt's page (none past
  // the sequence's last key, so such loads read zero).
  auto page_rsrc = [&](const bf16* pool, int kt) {
    int rows_v = Skv - kt * kBN;
    rows_v = rows_v < 0 ? 0 : (rows_v > kBN ? kBN : rows_v);
    int pg = kt < max_pages ? block_table[(size_t)tc.b * max_pages + kt] : 0;
    pg = pg < 0 ? 0 : (pg >= num_pages ? num_pages - 1 : pg);
    return make_rsrc(pool + ((size_t)pg * Hkv + tc.kvh) * kBN * D, (uint32_t)(rows_v * RB));
  };
  uint32_t k_src[NLD], v_src[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int p = 64 * (NW * j + w) + l;
    const int r = p / U, u = p % U;
    k_src[j] = (uint32_t)(r * RB + 16 * (u ^ sk(r)));
    v_src[j] = (uint32_t)(r * RB + 32 * ((u >> 1) ^ sv(r)) + 16 * (u & 1));
  }
  auto load_k = [&](int kt, lds_t* dst) {
    if constexpr (PAGED) {
      const __amdgpu_buffer_rsrc_t r = page_rsrc(k, kt);
#pragma unroll
      for (int j = 0; j < NLD; ++j) load_to_lds16(r, dst + 1024 * (NW * j + w), k_src[j], 0);
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j) load_to_lds16(rk, dst + 1024 * (NW * j + w), k_src[j], (uint32_t)kt * TB);
    }
  };
  auto load_v = [&](int kt, lds_t* dst) {
    if constexpr (PAGED) {
      const __amdgpu_buffer_rsrc_t r = page_rsrc(v, kt);
#pragma unroll
      for (int j = 0; j < NLD; ++j) load_to_lds16(r, dst + 1024 * (NW * j + w), v_src[j], 0);
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j) load_to_lds16(rv, dst + 1024 * (NW * j + w), v_src[j], (uint32_t)kt * TB);
    }
  };

  // Operand read offsets.  Score A operand (K): row 32 kb + lr, logical unit
  // 2 s + hf.  P V A operand (V^T, transposing read r of key chunk (kb, cc)):
  // this lane addresses row 32 kb + 16 cc + 8 r + 4 (g / 2) + jj / 4 at
  // d = 32 db + 16 (g % 2) + 4 (jj % 4), with g = l / 16, jj = l % 16, and so
  // receives V[32 kb + 16 cc + 8 r + 4 hf + e][32 db + lr], e = 0..3: the keys
  // of B-operand slots 4 r + e of P^T chunk (kb, cc) (see pack below).
  uint32_t k_rd[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) k_rd[s] = (uint32_t)(lr * RB + 16 * ((2 * s + hf) ^ sk(lr)));
  const int g4 = l >> 4, jj = l & 15;
  const int vrow = 4 * (g4 >> 1) + (jj >> 2);   // row offset inside an 8-row read (chunk starts are multiples of 8)
  uint32_t v_rd[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    v_rd[db] = (uint32_t)(vrow * RB + 32 * ((2 * db + (g4 & 1)) ^ sv(vrow)) + 8 * (jj & 3));

  // Running state per row block (per lane = per query row; l is this lane's
  // partial over its half of the keys).
  float m_run[QB], l_run[QB];
  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[qb][i][j] = 0.f;
  }

  // Row max of a score tile, scaled to log2 units (c > 0), combined with the
  // partner lane that holds the other half of the tile's keys.
  auto tile_max = [&](const f32x16 (&S)[2]) { return max_xor32(max_of32(S[0], S[1])) * c; };

  // Online softmax in base 2 with a fixed exponent base.  The base m (per
  // row) is the row max of the first tile; a later tile is exponentiated
  // against the same m without computing its max: P = 2^(S c - m) may then
  // exceed 1 (fp32 and bf16 keep their relative precision at any exponent),
  // and O and l share the base, so O / l and LSE = (m + log2 l) ln 2 are
  // unchanged.  Only when a row's partial sum of P over this lane's 32 keys
  // exceeds kSumCap (so some P could be large enough to threaten fp32 range
  // in O) is the tile redone: its scores are recomputed, its max taken, m
  // raised, O and l rescaled by 2^(m_old - m_new) and P recomputed.  Data
  // whose scores never climb far above the first tile's maximum never takes
  // that path.
  // Key kt kBN + 4 hf + o (o = 32 kb + 8 (r / 4) + r % 4, at most 59) is
  // visible when o <= lim: one compare of a lane value with a small constant
  // per element.
  auto mask_tile = [&](int kt, f32x16 (&S)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int last = CAUSAL ? min(pos[qb], Skv - 1) : Skv - 1;
      const int lim = last - kt * kBN - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
          S[qb][kb][r] = (o <= lim) ? S[qb][kb][r] : kNegInf;
        }
    }
  };
  auto exponentiate = [&](f32x16 (&S)[QB][2], float (&psum)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_use = (m_run[qb] == kNegInf) ? 0.f : m_run[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[qb][kb][r] = exp2_hw(__builtin_fmaf(S[qb][kb][r], c, -m_use));
      psum[qb] = sum_tree32(S[qb][0], S[qb][1]);
    }
  };
  auto raise_base = [&](const f32x16 (&S)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = fmaxf(m_run[qb], tile_max(S[qb]));
      const float corr = (m_new == kNegInf) ? 1.f : exp2_hw(m_run[qb] - m_new);   // 0 from m = -inf
      l_run[qb] *= corr;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[qb][i][j] *= corr;
      m_run[qb] = m_new;
    }
  };
  // P^T B operand of key chunk (kb, cc): P registers 8 cc .. 8 cc + 7 of block
  // kb, i.e. slot e' holds key 32 kb + 16 cc + 8 (e' / 4) + 4 hf + e' % 4.
  auto pack = [&](const f32x16 (&Pv)[QB][2], bf16x8 (&pf)[QB][2][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int r8 = 8 * cc;
          pf[qb][kb][cc] = to_bf16x8(Pv[qb][kb][r8 + 0], Pv[qb][kb][r8 + 1], Pv[qb][kb][r8 + 2], Pv[qb][kb][r8 + 3],
                                     Pv[qb][kb][r8 + 4], Pv[qb][kb][r8 + 5], Pv[qb][kb][r8 + 6], Pv[qb][kb][r8 + 7]);
        }
  };
  // MFMA i (0..15) of the P V product of one tile: key chunk (i / 8, (i / 4) % 2)
  // of V slot Vs, d block i % 4 (D = 128; D = 64 has 8 MFMAs, d block i % 2).
  auto pv_mfma = [&](const lds_t* Vs, const bf16x8 (&pf)[QB][2][2], int i) {
    const int kb = i / (2 * DB), cc = (i / DB) & 1, db = i % DB;
    const lds_t* vp = Vs + (32 * kb + 16 * cc) * RB + v_rd[db];
    const s16x4 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * RB);
    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kb][cc], oacc[qb][db], 0, 0, 0);
  };
  // MFMA i (0 .. 2 DS - 1) of the scores of one tile: d step i / 2, key block i % 2.
  auto score_mfma = [&](const lds_t* Ks, f32x16 (&S)[QB][2], int i) {
    const int s = i >> 1, kb = i & 1;
    const bf16x8 a = lds_read16(Ks + 32 * kb * RB + k_rd[s]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      S[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][s], S[qb][kb], 0, 0, 0);
  };
  // Rare path: the scores of tile kt again, with K read from global memory
  // (its LDS slot is being refilled by then).
  auto rescore_from_global = [&](int kt, f32x16 (&S)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) S[qb][kb][j] = 0.f;
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 a;
        if constexpr (PAGED)
          a = as_bf16x8(buf_ld16(page_rsrc(k, kt), (uint32_t)((32 * kb + lr) * RB + 32 * s + 16 * hf), 0));
        else
          a = as_bf16x8(buf_ld16(rk, (uint32_t)((kt * kBN + 32 * kb + lr) * RB + 32 * s + 16 * hf), 0));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][s], S[qb][kb], 0, 0, 0);
      }
  };

  // One pipelined step, three tiles deep:
  //   P1  tile kt: mask (straddling / tail tiles only);
  //   P2  the score MFMAs of tile kt + 1 (K slot Kn) and the P V MFMAs of tile
  //       kt - 1 (V slot Vp, operand pf_prev) alternate, interleaved with the
  //       exponentials, row sums and bf16 packing of tile kt;
  //   P3  the range check of tile kt (rare redo), row sums into l.
  // After the last tile the score MFMAs run on an idle slot and are discarded,
  // which keeps them in the same basic block as the work they interleave with.
  auto step = [&](int kt, f32x16 (&S)[QB][2], f32x16 (&Snext)[QB][2], const bf16x8 (&pf_prev)[QB][2][2],
                  bf16x8 (&pf_new)[QB][2][2], const lds_t* Kn, const lds_t* Vp) {
    const int key_end = kt * kBN + kBN - 1;
    const bool need_mask = (key_end >= Skv) || (CAUSAL && key_end > q_start + wave_tmin);
    // A real branch (most tiles need no mask): without the hint the compiler
    // turns the rare mask into selects executed on every tile.
    if (__builtin_expect(need_mask, 0)) mask_tile(kt, S);

    // P2.  The wave raises its issue priority while it feeds the matrix core,
    // so the arbiter prefers its MFMAs over the other wave's VALU.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) Snext[qb][kb][j] = 0.f;
#pragma unroll
    for (int i = 0; i < 2 * DS; ++i) {
      score_mfma(Kn, Snext, i);
      if (i < 4 * DB) pv_mfma(Vp, pf_prev, i);
    }
    float psum[QB];
    exponentiate(S, psum);
    pack(S, pf_new);
    // Schedule: LDS reads run ahead of their MFMAs; ~3.5 VALU per MFMA.
    __builtin_amdgcn_sched_group_barrier(0x100, 3 * kLdsAhead / 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * DS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);       // score MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3 * QB, 0);   // VALU
      if (i < 4 * DB) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);       // P V MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * QB, 0);   // VALU
      }
      if (2 * i + kLdsAhead < 4 * DS) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // next LDS reads
    }
    __builtin_amdgcn_s_setprio(0);

    // P3.
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) over |= !(psum[qb] <= kSumCap);   // also catches inf / NaN
    if (__builtin_amdgcn_ballot_w64(over)) {
      rescore_from_global(kt, S);
      if (need_mask) mask_tile(kt, S);
      raise_base(S);
      exponentiate(S, psum);
      pack(S, pf_new);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += psum[qb];
  };

  // Software pipeline (ADR-0060 section 5.6, option 3: the next tile's score
  // GEMM is started before this tile's softmax; here one stage deeper):
  // iteration kt (parity P = kt % 2) loads K tile kt + 2 into K slot P and V
  // tile kt into V slot P -- slots iteration kt - 1 finished reading -- while
  // it computes the scores of tile kt + 1 from K slot 1 - P, the softmax of
  // tile kt, and the P V product of tile kt - 1 from V slot 1 - P.  One barrier per tile, after this wave's loads have landed,
  // orders the rings.  The P V product of the last tile follows the loop.
  kt_lo = __builtin_amdgcn_readfirstlane(kt_lo);
  kt_hi = __builtin_amdgcn_readfirstlane(kt_hi);
  wave_tmin = __builtin_amdgcn_readfirstlane(wave_tmin);
  wave_end = __builtin_amdgcn_readfirstlane(min(wave_end, kt_hi));
  f32x16 sA[QB][2], sB[QB][2];
  bf16x8 pfA[QB][2][2], pfB[QB][2][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) pfB[qb][kb][cc] = bf16x8{};   // "tile -1": P = 0
  if (kt_hi > kt_lo) {
    load_k(kt_lo, kbuf[0]);
    load_k(kt_lo + 1, kbuf[1]);
    // V slot 1 plays tile -1 in iteration 0: zero it, so 0 * V stays 0.
#pragma unroll
    for (int i = 0; i < TB / (16 * NT); ++i)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(vbuf[1] + 16 * (tid + NT * i)) =
          u32x4{0u, 0u, 0u, 0u};
    wait_lds_loads();
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sA[qb][kb][j] = 0.f;
    if (wave_active) {
#pragma unroll
      for (int i = 0; i < 2 * DS; ++i) score_mfma(kbuf[0], sA, i);
      // The exponent base: the first tile's row max, taken here, outside the
      // loop, so that the steady-state step carries no max and no rescale.
      const int key_end = kt_lo * kBN + kBN - 1;
      if ((key_end >= Skv) || (CAUSAL && key_end > q_start + wave_tmin)) mask_tile(kt_lo, sA);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) m_run[qb] = tile_max(sA[qb]);
    }
    __syncthreads();   // K slot 0 is reloaded in iteration 0
  }
  auto iteration = [&](auto parity, int kt, f32x16 (&Scur)[QB][2], f32x16 (&Snext)[QB][2],
                       const bf16x8 (&pf_prev)[QB][2][2], bf16x8 (&pf_new)[QB][2][2]) {
    constexpr int P = decltype(parity)::value;
    load_k(kt + 2, kbuf[P]);    // past the range these fill idle slots (zeros past Skv)
    load_v(kt, vbuf[P]);
    if (wave_active && kt <= wave_end) step(kt, Scur, Snext, pf_prev, pf_new, kbuf[1 - P], vbuf[1 - P]);
    wait_lds_loads();
    __syncthreads();
  };
  for (int kt = kt_lo; kt < kt_hi; kt += 2) {
    iteration(Parity<0>{}, kt, sA, sB, pfB, pfA);
    if (kt + 1 < kt_hi) iteration(Parity<1>{}, kt + 1, sB, sA, pfA, pfB);
  }
  // P V of the last tile (V slot and P registers by its parity), unless this
  // wave stopped early: then that tile is wholly masked for it and step
  // wave_end has already added its last real tile.
  if (kt_hi > kt_lo && wave_active && wave_end >= kt_hi) {
    if ((kt_hi - kt_lo) & 1) {
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i) pv_mfma(vbuf[0], pfA, i);
    } else {
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i) pv_mfma(vbuf[1], pfB, i);
    }
  }

  // Epilogue: O = O^T / l per row, LSE = (m + log2 l) ln 2; in split-KV mode
  // the same pair in fp32 into this split's partial slot.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_xor32(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_row = l_tot > 0.f ? (m_run[qb] + __log2f(l_tot)) * kLn2 : kNegInf;
    if (row[qb] < rows_total) {
      const size_t flat = head0 * Sq + row[qb];   // row of [B, Hq, Sq]
      if (part_o != nullptr) {
        const size_t slot = flat * n_splits + tc.split;
        float* prow = part_o + slot * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * db + 8 * q4 + 4 * hf;
            f32x4 val = {oacc[qb][db][4 * q4 + 0] * inv, oacc[qb][db][4 * q4 + 1] * inv,
                         oacc[qb][db][4 * q4 + 2] * inv, oacc[qb][db][4 * q4 + 3] * inv};
            *reinterpret_cast<f32x4*>(prow + d0) = val;
          }
        if (hf == 0) part_lse[slot] = lse_row;
      } else {
        bf16* orow = o + flat * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * db + 8 * q4 + 4 * hf;
            const uint32_t lo = pack_lo(__builtin_bit_cast(uint16_t, (bf16)(oacc[qb][db][4 * q4 + 0] * inv)),
                                        __builtin_bit_cast(uint16_t, (bf16)(oacc[qb][db][4 * q4 + 1] * inv)));
            const uint32_t hi = pack_lo(__builtin_bit_cast(uint16_t, (bf16)(oacc[qb][db][4 * q4 + 2] * inv)),
                                        __builtin_bit_cast(uint16_t, (bf16)(oacc[qb][db][4 * q4 + 3] * inv)));
            u32x2 pr = {lo, hi};
            *reinterpret_cast<u32x2*>(orow + d0) = pr;
          }
        if (lse != nullptr && hf == 0) lse[flat] = lse_row;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel, two-team form (8 waves, 256 stacked rows, one workgroup per CU)
//
// Waves w and w + 4 of a workgroup run on the same SIMD.  The waves are two
// teams -- team 0 = waves 0-3, team 1 = waves 4-7, one wave of each on every
// SIMD -- that take turns between two phases, with one workgroup barrier
// between phases ("half-steps"):
//   matrix phase of tile j: S(j+1) = K(j+1) Q^T and O^T += V(j)^T P(j)^T,
//                           32 MFMAs per wave at d = 128, operands from LDS;
//   vector phase of tile j: P(j) = 2^(S(j) c - m), its row sums and bf16
//                           packing (plus the mask on straddling tiles).
// Team 0 runs the matrix phase of tile j in half-step 2j and the vector phase
// of tile j + 1 in half-step 2j + 1; team 1 runs the same one half-step
// later.  In every half-step each SIMD therefore holds one wave that issues
// MFMAs back to back and one that does the softmax arithmetic beside them, so
// the matrix core is fed while the exponentials run, whatever the order the
// SIMD picks instructions in.  This is the pages' idea of starting the next
// tile's score GEMM before the current tile's softmax, carried across waves.
//
// K and V tiles go through three-slot LDS rings (tile x in slot x % 3).  The
// loads ride in the vector phases, so a matrix phase issues only LDS reads
// and MFMAs: team 0 loads K(j+3) during its vector phase of tile j + 1, team
// 1 loads V(j+2) during its vector phase of tile j, and each team waits for
// its loads at the end of its next matrix phase, so the barrier that closes
// that half-step publishes the tile.  Every slot is reloaded only after the
// barrier that follows its last read (K(j) stays until both teams have run
// the vector phase of tile j, which may recompute its scores), and a V tile
// is published one half-step before the first wave that reads it starts its
// matrix phase: the vector phase reads the first V^T fragment of the wave's
// next matrix phase ahead, so that phase starts with an MFMA, not with an LDS
// round trip.  The tile loop is unrolled three times so that every slot index
// is a compile-time constant: the compiler then tells a read of one slot from
// a direct load in flight into another and adds no wait for it.
// ---------------------------------------------------------------------------
template <int I>
using IC = std::integral_constant<int, I>;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int Sq, int Skv,
    float c, int n_splits, float* __restrict__ part_o, float* __restrict__ part_lse) {
  constexpr int NW = 8, NT = 64 * NW, BM = 32 * NW;
  constexpr int RB = 2 * D;                 // bytes per K / V row
  constexpr int U = D / 8;                  // 16-byte units per row
  constexpr int TB = kBN * RB;              // bytes per tile
  constexpr int NLD = kBN * U / NT;         // direct loads per thread per tile (all 8 waves)
  constexpr int NLT = kBN * U / (NT / 2);   // the same when one team of 4 waves loads a tile
  constexpr int DS = D / 16;                // MFMA k-steps over d for S^T
  constexpr int DB = D / 32;                // 32-row d blocks of O^T
  constexpr int NM = 2 * DS;                // score MFMAs per tile (= P V MFMAs)
  constexpr int PF = 1;                     // V^T fragments read ahead across the barrier
  constexpr int LA = 4;                     // MFMAs whose LDS operands are in flight
  static_assert(NLD * NT == kBN * U && NLT * NT == 2 * kBN * U && NM == 4 * DB && PF <= LA && LA < NM,
                "tile shape");
  auto sk = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto sv = [](int r) { return D == 128 ? 2 * (r & 3) : 2 * ((r >> 1) & 1); };

  // V slots first: the transposing V reads (two per MFMA) then all fit the
  // 16-bit offset field of the LDS instructions, and only the K reads of two
  // slots need an address add.
  __shared__ __attribute__((aligned(1024))) char lds_a_v0[TB];
  __shared__ __attribute__((aligned(1024))) char lds_a_v1[TB];
  __shared__ __attribute__((aligned(1024))) char lds_a_v2[TB];
  __shared__ __attribute__((aligned(1024))) char lds_b_k0[TB];
  __shared__ __attribute__((aligned(1024))) char lds_b_k1[TB];
  __shared__ __attribute__((aligned(1024))) char lds_b_k2[TB];
  auto kslot = [&](auto s) __attribute__((always_inline)) -> lds_t* {
    constexpr int i = decltype(s)::value;
    return i == 0 ? (lds_t*)lds_b_k0 : (i == 1 ? (lds_t*)lds_b_k1 : (lds_t*)lds_b_k2);
  };
  auto vslot = [&](auto s) __attribute__((always_inline)) -> lds_t* {
    constexpr int i = decltype(s)::value;
    return i == 0 ? (lds_t*)lds_a_v0 : (i == 1 ? (lds_t*)lds_a_v1 : (lds_t*)lds_a_v2);
  };

  const int G = Hq / Hkv;
  const int rows_total = G * Sq;
  // Row blocks.  With G a multiple of 8 a block is 32 positions of 8 query
  // heads, wave w taking head 8 hb + w: every wave then has the same causal
  // extent, so no SIMD idles through the block's last tiles while another
  // finishes.  Otherwise a block is 256 consecutive stacked rows (g-major).
  const bool heads8 = (G & 7) == 0;
  const int n_pb = (Sq + 31) >> 5;
  const TileCoord tc =
      heads8 ? map_tile_heads8(blockIdx.x, B * Hkv * n_splits, n_splits, Hkv, G >> 3, n_pb)
             : map_tile<BM>(blockIdx.x, B * Hkv * n_splits, n_splits, Hkv, (rows_total + BM - 1) / BM, G, Sq);
  const int q_start = Skv - Sq;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = w >> 2;
  const int l = tid & 63;
  const int lr = l & 31;
  const int hf = l >> 5;

  const size_t head0 = (size_t)tc.b * Hq + (size_t)tc.kvh * G;
  const bf16* qg = q + head0 * Sq * D;
  const size_t kvoff = ((size_t)tc.b * Hkv + tc.kvh) * (size_t)Skv * D;

  // This wave's first stacked row (g Sq + t) and its number of valid rows, and
  // the smallest and largest position t of the whole block.
  int wrow0, wrows, blk_tmin, blk_tmax;
  if (heads8) {
    const int t0 = 32 * (tc.mt % n_pb);
    wrow0 = (8 * (tc.mt / n_pb) + w) * Sq + t0;
    wrows = min(32, Sq - t0);
    blk_tmin = t0;
    blk_tmax = t0 + wrows - 1;
  } else {
    const int r0 = tc.mt * BM;
    wrow0 = r0 + 32 * w;
    wrows = max(0, min(32, rows_total - wrow0));
    row_range_positions(r0, min(r0 + BM - 1, rows_total - 1), Sq, blk_tmin, blk_tmax);
  }
  const int row = wrow0 + lr;
  const bool row_ok = lr < wrows;
  const int pos = q_start + (row_ok ? row % Sq : 0);

  // Tile range of the workgroup (its key split, cut at the causal extent),
  // and the last tile this wave needs (relative to the first, -1 for none).
  const int tiles_all = (Skv + kBN - 1) / kBN;
  const int tiles_per_split = (tiles_all + n_splits - 1) / n_splits;
  int kt_lo = tc.split * tiles_per_split;
  int kt_hi = min(tiles_all, kt_lo + tiles_per_split);
  int wave_tmin = 0x3fffffff;
  int wave_end = 0x3fffffff;
  if (CAUSAL) {
    const int vis_end = q_start + blk_tmax + 1;
    kt_hi = min(kt_hi, vis_end > 0 ? (vis_end + kBN - 1) / kBN : 0);
    if (wrows > 0) {
      int a, bb;
      row_range_positions(wrow0, wrow0 + wrows - 1, Sq, a, bb);
      wave_tmin = a;
      const int wv_end = q_start + bb + 1;
      wave_end = wv_end > 0 ? (wv_end + kBN - 1) / kBN : 0;
    }
  }
  kt_lo = __builtin_amdgcn_readfirstlane(kt_lo);
  kt_hi = __builtin_amdgcn_readfirstlane(kt_hi);
  wave_tmin = __builtin_amdgcn_readfirstlane(wave_tmin);
  const int T = max(kt_hi - kt_lo, 0);
  const int jw_last = __builtin_amdgcn_readfirstlane(wrows > 0 ? min(min(wave_end, kt_hi) - kt_lo, T) - 1 : -1);

  // Q^T B operands: lane holds Q[row][16 s + 8 hf .. +7]; invalid rows read
  // as zero (their offset lies past the buffer).  Waited for together with the
  // first tiles' loads below.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg, (uint32_t)rows_total * D * 2);
  const uint32_t q_off = (uint32_t)(row_ok ? row : rows_total) * D * 2 + 16 * hf;
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) qf[s] = as_bf16x8(buf_ld16(rq, q_off + 32 * s, 0));

  // Direct loads (same unit map and swizzles as the kernel above).
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kvoff, (uint32_t)Skv * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kvoff, (uint32_t)Skv * RB);
  // Prologue tiles: all 8 waves load, unit p = 64 (8 j + w) + l.  In the loop
  // one team loads a tile (team 0 the K tiles, team 1 the V tiles): unit
  // p = 64 (4 j + w % 4) + l.  The source offsets undo the swizzles.
  auto k_src_of = [&](int p) __attribute__((always_inline)) {
    const int r = p / U, u = p % U;
    return (uint32_t)(r * RB + 16 * (u ^ sk(r)));
  };
  auto v_src_of = [&](int p) __attribute__((always_inline)) {
    const int r = p / U, u = p % U;
    return (uint32_t)(r * RB + 32 * ((u >> 1) ^ sv(r)) + 16 * (u & 1));
  };
  auto load_k = [&](int kt, lds_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NLD; ++j)
      load_to_lds16(rk, dst + 1024 * (NW * j + w), k_src_of(64 * (NW * j + w) + l), (uint32_t)kt * TB);
  };
  auto load_v = [&](int kt, lds_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NLD; ++j)
      load_to_lds16(rv, dst + 1024 * (NW * j + w), v_src_of(64 * (NW * j + w) + l), (uint32_t)kt * TB);
  };
  const int wt = w & 3;   // wave index inside its team
  uint32_t t_src[NLT];    // this wave's source offsets for its team's tile (K for team 0, V for team 1)
#pragma unroll
  for (int j = 0; j < NLT; ++j) {
    const int p = 64 * (4 * j + wt) + l;
    t_src[j] = team == 0 ? k_src_of(p) : v_src_of(p);
  }
  auto load_team = [&](int kt, lds_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = team == 0 ? rk : rv;
#pragma unroll
    for (int j = 0; j < NLT; ++j) load_to_lds16(r, dst + 1024 * (4 * j + wt), t_src[j], (uint32_t)kt * TB);
  };

  // Operand read offsets (as in the kernel above).
  // K read offsets carry a bias of kKBias that the reads take back in their
  // constant part: the K slots then sit within the 16-bit offset field of the
  // LDS reads from a per-lane base, with no address add per read.  (The empty
  // asm hides the bias from the compiler, which would fold it back.)
  constexpr uint32_t kKBias = 32768;
  uint32_t k_rd[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    k_rd[s] = kKBias + (uint32_t)(lr * RB + 16 * ((2 * s + hf) ^ sk(lr)));
    asm("" : "+v"(k_rd[s]));
  }
  const int g4 = l >> 4, jj = l & 15;
  const int vrow = 4 * (g4 >> 1) + (jj >> 2);
  uint32_t v_rd[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    v_rd[db] = (uint32_t)(vrow * RB + 32 * ((2 * db + (g4 & 1)) ^ sv(vrow)) + 8 * (jj & 3));

  float m_run = kNegInf, l_run = 0.f;
  float m_use = 0.f;   // the exponent base as applied: m_run, or 0 while no key was seen
  // Rescale of O owed by a raised exponent base, applied at the start of the
  // next matrix phase (rescaling in the vector phase costs the compiler's
  // register allocation more than the loop has).
  float o_corr = 1.f;
  bool o_pending = false;
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
  f32x16 S[2];
  bf16x8 pf[2][2];
  bf16x8 pre_v[PF];   // operands of the first PF MFMAs of the next matrix phase

  // Operand fragments: score MFMA i is d step i / 2, key block i % 2; P V
  // MFMA i is key chunk (i / (2 DB), (i / DB) % 2), d block i % DB.
  auto k_frag = [&](const lds_t* Ks, int i) __attribute__((always_inline)) {
    return lds_read16(Ks + ((int)(32 * (i & 1) * RB) - (int)kKBias) + k_rd[i >> 1]);
  };
  auto v_frag = [&](const lds_t* Vs, int i) __attribute__((always_inline)) {
    const int kb = i / (2 * DB), cc = (i / DB) & 1, db = i % DB;
    const lds_t* vp = Vs + (32 * kb + 16 * cc) * RB + v_rd[db];
    const s16x4 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * RB);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto mfma_s = [&](const bf16x8& a, int i) __attribute__((always_inline)) {
    const int kb = i & 1;
    S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i >> 1], (i >> 1) == 0 ? f32x16{} : S[kb], 0, 0, 0);
  };
  auto mfma_pv = [&](const bf16x8& a, int i) __attribute__((always_inline)) {
    const int kb = i / (2 * DB), cc = (i / DB) & 1, db = i % DB;
    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][cc], oacc[db], 0, 0, 0);
  };
  // Operand of MFMA t of a matrix phase: t < NM the P V MFMA t (V slot Vs),
  // else the score MFMA t - NM (K slot Ks).
  auto frag = [&](const lds_t* Ks, const lds_t* Vs, int t) __attribute__((always_inline)) {
    return t < NM ? v_frag(Vs, t) : k_frag(Ks, t - NM);
  };
  auto prefetch = [&](const lds_t* Vs) __attribute__((always_inline)) {
    // Issued after the vector work, not hoisted into it: the fragments then
    // hold registers only across the barrier.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < PF; ++i) pre_v[i] = v_frag(Vs, i);
  };
  // Matrix phase: the P V MFMAs of the current tile (V slot Vs, P in pf),
  // then, unless this is the wave's last tile (scores == false), the score
  // MFMAs of the next tile (K slot Ks) into S.  P is dead before S is
  // written, so the two never hold registers at once; the LDS reads run LA
  // MFMAs ahead of their use (on the last tile the first LA - PF K reads are
  // issued and left unused).  The two parts are scheduled as two regions.
  auto matrix_phase = [&](const lds_t* Ks, const lds_t* Vs, bool scores) __attribute__((always_inline)) {
    if (o_pending) {   // rare: the vector phase raised the exponent base
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[i][j] *= o_corr;
      o_corr = 1.f;
      o_pending = false;
    }
    __builtin_amdgcn_s_setprio(1);
    constexpr int NT2 = 2 * NM;
    bf16x8 fr[NT2];
#pragma unroll
    for (int t = 0; t < PF; ++t) fr[t] = pre_v[t];
#pragma unroll
    for (int t = PF; t < LA; ++t) fr[t] = frag(Ks, Vs, t);
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      fr[t + LA] = frag(Ks, Vs, t + LA);
      mfma_pv(fr[t], t);
    }
    // Schedule of each region: the reads of MFMAs PF .. LA - 1 first (two
    // LDS reads for a V^T fragment, one for a K fragment), then each MFMA
    // after the reads of the MFMA LA places later.
    constexpr int lead = 2 * (LA - PF);
    if (lead > 0) __builtin_amdgcn_sched_group_barrier(0x100, lead, 0);
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      if (t + LA < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if (scores) {
#pragma unroll
      for (int t = NM; t < NT2; ++t) {
        if (t + LA < NT2) fr[t + LA] = frag(Ks, Vs, t + LA);
        mfma_s(fr[t], t - NM);
      }
#pragma unroll
      for (int t = NM; t < NT2; ++t) {
        if (t + LA < NT2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Key kt kBN + 4 hf + o (o = 32 kb + 8 (r / 4) + r % 4, at most 59) is
  // visible when o <= lim: one compare of a lane value with a small constant
  // per element.
  auto mask_tile = [&](int kt) __attribute__((always_inline)) {
    const int last = CAUSAL ? min(pos, Skv - 1) : Skv - 1;
    const int lim = last - kt * kBN - 4 * hf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
        S[kb][r] = (o <= lim) ? S[kb][r] : kNegInf;
      }
  };
  auto tile_needs_mask = [&](int kt) __attribute__((always_inline)) {
    const int key_end = kt * kBN + kBN - 1;
    return (key_end >= Skv) || (CAUSAL && key_end > q_start + wave_tmin);
  };
  // P = 2^(S c - m) in place, this lane's partial row sum, and the bf16 P^T
  // operands (slot e' of chunk (kb, cc) is key 32 kb + 16 cc + 8 (e' / 4) +
  // 4 hf + e' % 4, i.e. accumulator register 8 cc + e').
  auto exponentiate = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kb][r] = exp2_hw(__builtin_fmaf(S[kb][r], c, -m_use));
    return sum_tree32(S[0], S[1]);
  };
  auto pack = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int r8 = 8 * cc;
        pf[kb][cc] = to_bf16x8(S[kb][r8 + 0], S[kb][r8 + 1], S[kb][r8 + 2], S[kb][r8 + 3], S[kb][r8 + 4],
                               S[kb][r8 + 5], S[kb][r8 + 6], S[kb][r8 + 7]);
      }
  };
  // Rare path (the fixed exponent base of the kernel above): the row sums of
  // the tile grew past kSumCap, so the scores are recomputed from K, still in
  // its LDS slot Ks, the base is raised to the tile's max and l rescaled (O
  // when the matrix phase next runs).
  auto redo_tile = [&](int kt, const lds_t* Ks) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NM; ++i) mfma_s(k_frag(Ks, i), i);
    if (tile_needs_mask(kt)) mask_tile(kt);
    const float m_new = fmaxf(m_run, max_xor32(max_of32(S[0], S[1])) * c);
    const float corr = (m_new == kNegInf) ? 1.f : exp2_hw(m_run - m_new);
    l_run *= corr;
    o_corr *= corr;   // O is rescaled before its next P V product
    o_pending = true;
    m_run = m_new;
    m_use = (m_run == kNegInf) ? 0.f : m_run;
  };
  auto vector_phase = [&](int kt, const lds_t* Ks) __attribute__((always_inline)) {
    if (__builtin_expect(tile_needs_mask(kt), 0)) mask_tile(kt);
    float psum = exponentiate();
    // Packed before the range check, so that the packing overlaps the row-sum
    // tree instead of waiting for the check; the rare redo packs again.  (The
    // empty asm takes the packed operands, which keeps the compiler from
    // moving the packing past the branch.)
    pack();
    asm volatile("" ::"v"(pf[0][0]), "v"(pf[0][1]), "v"(pf[1][0]), "v"(pf[1][1]));
    if (__builtin_amdgcn_ballot_w64(!(psum <= kSumCap))) {   // also catches inf / NaN
      redo_tile(kt, Ks);
      psum = exponentiate();
      pack();
    }
    l_run += psum;
  };
  // Workgroup barrier that the compiler may not move memory operations across
  // (s_barrier alone does not order them), with no wait on loads in flight.
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Loads of one ring tile by this wave's team: team 0 fills the K ring,
  // team 1 the V ring (a uniform branch, so that each load names its slot).
  auto load_ring = [&](auto slot, int kt) __attribute__((always_inline)) {
    if (team == 0) load_team(kt, kslot(slot));
    else load_team(kt, vslot(slot));
  };

  // Prologue: K(0..2) and V(0..1) in flight together with Q, one wait for
  // all of them on every path (the compiler's wait insertion then never sees
  // the Q loads pending inside the loop, where a wait on them would also wait
  // for the tile loads in flight); S(0) and the exponent base (its row max)
  // for every wave, then the softmax of tile 0.  Team 1 runs that softmax as
  // its first half-step (beside team 0's first matrix phase) and loads V(2) in
  // it; team 0 runs it before its first half-step.
  if (T > 0) {
    load_k(kt_lo, kslot(IC<0>{}));
    if (T > 1) load_k(kt_lo + 1, kslot(IC<1>{}));
    if (T > 2) load_k(kt_lo + 2, kslot(IC<2>{}));
    load_v(kt_lo, vslot(IC<0>{}));
    if (T > 1) load_v(kt_lo + 1, vslot(IC<1>{}));
  }
  wait_vm_loads();
  if (T > 0) {
    barrier();
    if (team == 1 && T > 2) load_team(kt_lo + 2, vslot(IC<2>{}));
    if (jw_last >= 0) {
#pragma unroll
      for (int i = 0; i < NM; ++i) mfma_s(k_frag(kslot(IC<0>{}), i), i);
      if (tile_needs_mask(kt_lo)) mask_tile(kt_lo);
      m_run = max_xor32(max_of32(S[0], S[1])) * c;
      m_use = (m_run == kNegInf) ? 0.f : m_run;
      vector_phase(kt_lo, kslot(IC<0>{}));
      prefetch(vslot(IC<0>{}));
    }
    if (team == 1) barrier();
  }

  // One tile j of the loop, the same code for both teams: the matrix phase of
  // tile j, then the vector phase of tile j + 1, one half-step each.  Team 1
  // runs one half-step behind team 0, so in every half-step one team is in a
  // matrix phase and the other in a vector phase.  The loads ride in the
  // vector phases, so the matrix phases issue nothing but LDS reads and
  // MFMAs: in its vector phase of tile j + 1 a team loads tile j + 3 of its
  // ring into slot j % 3, and it waits for those loads at the end of its next
  // matrix phase, so the barrier that closes that half-step publishes the
  // tile.  JM = j % 3 names the slots.
  auto tile = [&](auto jm, int j) __attribute__((always_inline)) {
    constexpr int JM = decltype(jm)::value;
    if (j <= jw_last) matrix_phase(kslot(IC<(JM + 1) % 3>{}), vslot(IC<JM>{}), j < jw_last);
    wait_vm_loads();
    barrier();
    if (j + 3 < T) load_ring(IC<JM>{}, kt_lo + j + 3);
    if (j + 1 <= jw_last) {
      vector_phase(kt_lo + j + 1, kslot(IC<(JM + 1) % 3>{}));
      prefetch(vslot(IC<(JM + 1) % 3>{}));
    }
    barrier();
  };
  // The loop runs a whole number of 3-tile rounds: tiles past the last do
  // nothing but keep the barriers in step.  Team 0 ends with one barrier
  // more, matching team 1's first half-step.
  for (int j = 0; j < T; j += 3) {
    tile(IC<0>{}, j);
    tile(IC<1>{}, j + 1);
    tile(IC<2>{}, j + 2);
  }
  if (team == 0 && T > 0) barrier();

  // Epilogue (as in the kernel above).
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_row = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  if (row_ok) {
    const size_t flat = head0 * Sq + row;
    if (part_o != nullptr) {
      const size_t slot = flat * n_splits + tc.split;
      float* prow = part_o + slot * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * db + 8 * q4 + 4 * hf;
          f32x4 val = {oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                       oacc[db][4 * q4 + 3] * inv};
          *reinterpret_cast<f32x4*>(prow + d0) = val;
        }
      if (hf == 0) part_lse[slot] = lse_row;
    } else {
      bf16* orow = o + flat * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * db + 8 * q4 + 4 * hf;
          const uint32_t lo = pack_lo(__builtin_bit_cast(uint16_t, (bf16)(oacc[db][4 * q4 + 0] * inv)),
                                      __builtin_bit_cast(uint16_t, (bf16)(oacc[db][4 * q4 + 1] * inv)));
          const uint32_t hi = pack_lo(__builtin_bit_cast(uint16_t, (bf16)(oacc[db][4 * q4 + 2] * inv)),
                                      __builtin_bit_cast(uint16_t, (bf16)(oacc[db][4 * q4 + 3] * inv)));
          u32x2 pr = {lo, hi};
          *reinterpret_cast<u32x2*>(orow + d0) = pr;
        }
      if (lse != nullptr && hf == 0) lse[flat] = lse_row;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel
// ---------------------------------------------------------------------------
constexpr int kBN32 = 32;   // keys per KV tile (fp32 path)

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int Sq, int Skv,
    float c) {
  constexpr int KP = D + 1;       // odd pitch: the 32 rows of a K read hit 32 banks
  constexpr int VP = D + 4;
  constexpr int CPR = D / 4;      // 16-byte chunks per row
  constexpr int RPI = kThreads / CPR;
  constexpr int NL = kBN32 / RPI; // loads per thread per tensor
  constexpr int DB = D / 32;
  constexpr int DS = D / 2;

  __shared__ __attribute__((aligned(16))) float Ks[kBN32 * KP];
  __shared__ __attribute__((aligned(16))) float Vs[kBN32 * VP];

  const int G = Hq / Hkv;
  const int rows_total = G * Sq;
  const int n_mt = (rows_total + kBM - 1) / kBM;
  const TileCoord tc = map_tile<kBM>(blockIdx.x, B * Hkv, 1, Hkv, n_mt, G, Sq);
  const int r0 = tc.mt * kBM;
  const int q_start = Skv - Sq;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 31, hf = l >> 5;
  const size_t head0 = (size_t)tc.b * Hq + (size_t)tc.kvh * G;
  const float* qg = q + head0 * Sq * D;
  const size_t kvoff = ((size_t)tc.b * Hkv + tc.kvh) * (size_t)Skv * D;
  const float* kg = k + kvoff;
  const float* vg = v + kvoff;

  const int row = r0 + 32 * w + lr;
  const bool row_ok = row < rows_total;
  const int pos = q_start + (row_ok ? row % Sq : 0);

  int n_tiles = (Skv + kBN32 - 1) / kBN32;
  int wave_tmin = 0x3fffffff;
  if (CAUSAL) {
    int tmin, tmax;
    row_range_positions(r0, min(r0 + kBM - 1, rows_total - 1), Sq, tmin, tmax);
    n_tiles = min(n_tiles, (q_start + tmax) / kBN32 + 1);
    const int wA = r0 + 32 * w, wB = min(r0 + 32 * w + 31, rows_total - 1);
    if (wA <= wB) {
      int a, bb;
      row_range_positions(wA, wB, Sq, a, bb);
      wave_tmin = a;
    }
  }

  float qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) qf[s] = row_ok ? qg[(size_t)row * D + 2 * s + hf] : 0.f;

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;

  const int ch = tid % CPR, rg = tid / CPR;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int key0 = kt * kBN32;
    u32x4 kx[NL], vx[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int key = key0 + rg + RPI * i;
      u32x4 a = {0u, 0u, 0u, 0u}, b2 = {0u, 0u, 0u, 0u};
      if (key < Skv) {
        a = ld16(kg + (size_t)key * D + 4 * ch);
        b2 = ld16(vg + (size_t)key * D + 4 * ch);
      }
      kx[i] = a;
      vx[i] = b2;
    }
    __syncthreads();   // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      // Bit-cast copies of the elements: clang lowers a bit-cast of a vector
      // element lvalue as a read of element 0.
      float* kd = Ks + (rg + RPI * i) * KP + 4 * ch;
      const f32x4 kf = __builtin_bit_cast(f32x4, kx[i]);
      kd[0] = kf[0];
      kd[1] = kf[1];
      kd[2] = kf[2];
      kd[3] = kf[3];
      st16(Vs + (rg + RPI * i) * VP + 4 * ch, vx[i]);
    }
    __syncthreads();

    f32x16 sacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[lr * KP + 2 * s + hf], qf[s], sacc, 0, 0, 0);

    const int key_end = key0 + kBN32 - 1;
    if ((key_end >= Skv) || (CAUSAL && key_end > q_start + wave_tmin)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        const bool vis = (key < Skv) && (!CAUSAL || key <= pos);
        sacc[r] = vis ? sacc[r] : kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float corr = exp2_hw(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_hw(__builtin_fmaf(sacc[r], c, -m_use));
      sacc[r] = p;
      psum += p;
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[i][j] *= corr;

    // O^T += V^T P^T, two keys per step: k-slot hf of step st = 4 q + s' is
    // key 8 q + 4 hf + s', i.e. this lane's accumulator st.
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = 8 * (st >> 2) + 4 * hf + (st & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VP + 32 * db + lr], sacc[st], oacc[db], 0, 0, 0);
    }
  }

  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    float* orow = o + (head0 * Sq + row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hf;
        f32x4 val = {oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                     oacc[db][4 * q4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + d0) = val;
      }
    if (lse != nullptr && hf == 0)
      lse[head0 * Sq + row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const long long rows = (long long)(a.Hq / a.Hkv) * a.Sq;   // stacked rows per (batch, KV head)
  const long long groups = (long long)a.B * a.Hkv;
  const float c = a.scale * kLog2e;
  const dim3 blk(kThreads);
  if (a.bf16) {
    // One 32-row block per wave.  (Two blocks per wave halve the LDS bytes per
    // MFMA but spill at one wave per SIMD: the compiler shuttles the output
    // accumulators between AGPRs and VGPRs.)  8 waves (256 rows) per
    // workgroup, one workgroup per CU, whenever that still gives every CU a
    // workgroup: each K/V tile brought into LDS then serves twice the rows,
    // and the two-team kernel runs (paged mode keeps the one-team kernel).
    // Smaller problems take 4-wave workgroups, two per CU.
    const long long wg8 = (rows + 255) / 256 * groups * a.n_splits;
    const bool eight = rows > 128 && wg8 >= kNumCUs;
    const bool paged = a.block_table != nullptr;
    // The two-team kernel's blocks are 32 positions x 8 query heads when G is
    // a multiple of 8 (as many blocks as 256-row blocks whenever Sq % 32 == 0).
    const int G = a.Hq / a.Hkv;
    const long long wg_pp = (G % 8 == 0) ? (long long)(G / 8) * ((a.Sq + 31) / 32) * groups * a.n_splits : wg8;
    const long long nwg = eight ? (paged ? wg8 : wg_pp) : (rows + 127) / 128 * groups * a.n_splits;
    const dim3 g((unsigned)nwg), blk_w(eight ? 512 : 256);
#define SA_LAUNCH_ONE(DD, CC, WW, PG)                                                                    \
  hipLaunchKernelGGL((prefill_bf16_kernel<DD, CC, 1, WW, PG>), g, blk_w, 0, stream, (const bf16*)a.q,     \
                     (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Skv, c, \
                     a.n_splits, a.part_o, a.part_lse, a.block_table, a.kv_len, a.max_pages, a.num_pages, \
                     a.seq_splits)
#define SA_LAUNCH_PP(DD, CC)                                                                             \
  hipLaunchKernelGGL((prefill_pp_kernel<DD, CC>), g, blk_w, 0, stream, (const bf16*)a.q, (const bf16*)a.k, \
                     (const bf16*)a.v, (bf16*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Skv, c, a.n_splits,    \
                     a.part_o, a.part_lse)
#define SA_LAUNCH_BF16(DD, CC)                                                                           \
  do {                                                                                                   \
    if (paged) {                                                                                         \
      if (eight) SA_LAUNCH_ONE(DD, CC, 8, true); else SA_LAUNCH_ONE(DD, CC, 4, true);                   \
    } else {                                                                                             \
      if (eight) SA_LAUNCH_PP(DD, CC); else SA_LAUNCH_ONE(DD, CC, 4, false);                            \
    }                                                                                                    \
  } while (0)
    if (a.d == 128) {
      if (a.causal) SA_LAUNCH_BF16(128, true); else SA_LAUNCH_BF16(128, false);
    } else {
      if (a.causal) SA_LAUNCH_BF16(64, true); else SA_LAUNCH_BF16(64, false);
    }
#undef SA_LAUNCH_BF16
#undef SA_LAUNCH_PP
#undef SA_LAUNCH_ONE
  } else {
    const dim3 g((unsigned)((rows + kBM - 1) / kBM * groups));
#define SA_LAUNCH_F32(DD, CC)                                                                         \
  hipLaunchKernelGGL((prefill_f32_kernel<DD, CC>), g, blk, 0, stream, (const float*)a.q,            \
                     (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Sq, \
                     a.Skv, c)
    if (a.d == 128) {
      if (a.causal) SA_LAUNCH_F32(128, true); else SA_LAUNCH_F32(128, false);
    } else {
      if (a.causal) SA_LAUNCH_F32(64, true); else SA_LAUNCH_F32(64, false);
    }
#undef SA_LAUNCH_F32
  }
  return hipGetLastError();
}

}  // namespace sa
