// Device-side helpers shared by the streaming attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();

// Hardware base-2 exponential (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Non-temporal 16-byte load, for data streamed through exactly once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round 8 fp32 values to bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                           float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

// Low / high 16-bit halves of two dwords packed into one dword (one
// v_perm_b32 each: selector bytes 0-3 pick from the second operand, 4-7 from
// the first).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Raw buffer resource over [base, base + nbytes): loads at offsets at or past
// nbytes return zero, so tails need no clamping or predication.  Word 3 selects
// 32-bit data format, as raw (untyped, stride 0) buffer access requires on gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
// 16-byte buffer load at byte offset voff (per lane) + soff (wave-uniform).
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// Device-scope (sc1) 16-byte buffer load: misses any stale copy in this XCD's
// L2 and reads the device coherence point.
__device__ __forceinline__ f32x4 buf_ld16_dev(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 16));
}
// Device-scope (sc1) store and load of one float, relaxed.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Max of 32 values held in two 16-float accumulators with 3-input max ops.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float max_of32(const f32x16& a, const f32x16& b) {
  float t[11];
#pragma unroll
  for (int i = 0; i < 5; ++i) t[i] = max3f(a[3 * i], a[3 * i + 1], a[3 * i + 2]);
#pragma unroll
  for (int i = 0; i < 5; ++i) t[5 + i] = max3f(b[3 * i], b[3 * i + 1], b[3 * i + 2]);
  t[10] = fmaxf(a[15], b[15]);
  const float u0 = max3f(t[0], t[1], t[2]), u1 = max3f(t[3], t[4], t[5]), u2 = max3f(t[6], t[7], t[8]);
  return max3f(max3f(u0, u1, u2), t[9], t[10]);
}

// Pairwise (tree) max / sum of the 32 values of two 16-float accumulators:
// depth 5 instead of a 32-long dependent chain.
__device__ __forceinline__ float max_tree32(const f32x16& a, const f32x16& b) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = fmaxf(a[i], b[i]);
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
  return t[0];
}
__device__ __forceinline__ float sum_tree32(const f32x16& a, const f32x16& b) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = a[i] + b[i];
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[i] + t[i + w];
  return t[0];
}

// Combine a value with the one in lane l ^ 32 through v_permlane32_swap (a
// VALU op; no LDS round trip).  Swapping the upper half of one copy with the
// lower half of another leaves, in every lane, its own value in one result
// and its partner's in the other.
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// LDS pointers and 16-byte / transposing LDS reads.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;

__device__ __forceinline__ bf16x8 lds_read16(const lds_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}
// ds_read_b64_tr_b16: in every 16-lane group, lane i receives element i % 4 of
// the 8 bytes addressed by lane 4 e + i / 4, as its element e.
__device__ __forceinline__ s16x4 lds_read_tr16(const lds_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(const_cast<lds_t*>(p)));
}

// Longest sequences first (paged decode): slot r of the launch goes to the
// sequence of rank r by valid length, longest first, ties by index, so the
// workgroups with the most keys start first and the short ones fill the tail.
// The B <= kRankMax clamped lengths are staged in LDS (len_s) and every thread
// ranks its sequences against all of them; beyond kRankMax sequences, launch
// order.  Every thread of the workgroup calls it (it synchronises).
constexpr int kRankMax = 256;
template <int NT>
__device__ __forceinline__ int seq_of_rank(const int32_t* kv_len, int B, int cap, int r, int* len_s, int* pick) {
  if (B > kRankMax) return r;
  auto clamp_len = [&](int len) { return len < 0 ? 0 : (len > cap ? cap : len); };
  for (int j = threadIdx.x; j < B; j += NT) len_s[j] = clamp_len(kv_len[j]);
  __syncthreads();
  for (int j = threadIdx.x; j < B; j += NT) {
    const int lj = len_s[j];
    int rank = 0;
    for (int i = 0; i < B; ++i) rank += (len_s[i] > lj) || (len_s[i] == lj && i < j);
    if (rank == r) *pick = j;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*pick);
}

}  // namespace sa
