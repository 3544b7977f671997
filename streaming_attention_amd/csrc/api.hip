// C ABI of the streaming attention library: argument validation on the host,
// then one enqueue on the caller's stream.  See include/attn.h for the
// contract of every entry point.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "launch.h"

namespace {

constexpr long long kMaxGrid = (1LL << 24) - 1;   // workgroups per launch (x 256 threads < 2^32)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool good_scale(float s) { return isfinite(s) && s > 0.f; }

// Shared validation of attn_prefill / attn_prefill_splitkv.  Buffer offsets
// inside one (batch, KV head) slice are 32-bit on the GPU, so each such slice
// of Q, K and V must stay under 2 GiB.
int check_prefill(const void* q, const void* k, const void* v, int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq,
                  int32_t Skv, int32_t d, attn_dtype_t dtype, int32_t causal, float scale, long long n_splits) {
  if (B < 0 || Sq < 0 || Skv < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (causal && Sq > Skv) return ATTN_ERR_SHAPE;
  if (!good_scale(scale)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;
  const long long G = Hq / Hkv;
  if (G * (long long)Sq > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const long long n_mt = (G * Sq + 127) / 128;
  if (n_mt * (long long)B * Hkv * n_splits > kMaxGrid) return ATTN_ERR_SHAPE;
  const long long esize = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
  if (G * Sq * d * esize > 0x7fffffffLL || (long long)Skv * d * esize > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) return ATTN_OK;
  if (q == nullptr) return ATTN_ERR_NULL;
  if (Skv > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || (Skv > 0 && (!aligned16(k) || !aligned16(v)))) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Fixed workspace of attn_decode_noalloc: the split partials of one call,
// part_o [B, Hq, max_splits, d] fp32 at the start and part_lse
// [B, Hq, max_splits] fp32 at kNoallocLseOffset, for at most
// ATTN_NOALLOC_MAX_PARTIALS (batch, head, split) entries at d <= 128.  Every
// GPU the library runs on holds its own copy until the process ends.  The
// array's name is a host-side stand-in: host code uses only the per-device
// address that hipGetSymbolAddress returns.
constexpr size_t kNoallocPartialBytes = (size_t)ATTN_NOALLOC_MAX_PARTIALS * 128 * sizeof(float);
constexpr size_t kNoallocLseOffset = kNoallocPartialBytes;
constexpr size_t kNoallocBytes = kNoallocPartialBytes + (size_t)ATTN_NOALLOC_MAX_PARTIALS * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream), looked up once per device with that
// device current.
int scratch_address(hipStream_t stream, unsigned char** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_LAUNCH;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (e != hipSuccess || p == nullptr) return ATTN_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return ATTN_OK;
}

// Shared validation of the split-KV decode entry points (pointer checks
// excluded).
int check_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t S_cap, int32_t d, int32_t max_splits,
                 attn_dtype_t dtype, float scale) {
  if (B < 0 || S_cap < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (max_splits < 1 || max_splits > 256) return ATTN_ERR_SHAPE;
  if (!good_scale(scale)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * Hkv * max_splits > kMaxGrid) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid size, scale or causal/size relation";
    case ATTN_ERR_UNSUPPORTED: return "unsupported dtype, head dim or head grouping";
    case ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case ATTN_ERR_WORKSPACE:
      return "request exceeds the fixed workspace of attn_decode_noalloc (B * Hq * max_splits > 65536)";
    default: return "unknown status";
  }
}

int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t Hq,
                 int32_t Hkv, int32_t Sq, int32_t Skv, int32_t d, attn_dtype_t dtype, int32_t causal, float scale,
                 hipStream_t stream) {
  const int st = check_prefill(q, k, v, B, Hq, Hkv, Sq, Skv, d, dtype, causal, scale, 1);
  if (st != ATTN_OK || B == 0 || Sq == 0) return st;
  if (o == nullptr) return ATTN_ERR_NULL;
  if (!aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;

  sa::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Skv = Skv; a.d = d;
  a.bf16 = dtype == ATTN_DTYPE_BF16;
  a.causal = causal != 0;
  a.scale = scale;
  return sa::launch_prefill(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_prefill_splitkv(const void* q, const void* k, const void* v, float* part_o, float* part_lse, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Skv, int32_t d, int32_t num_splits,
                         attn_dtype_t dtype, int32_t causal, float scale, hipStream_t stream) {
  if (num_splits < 1 || num_splits > 256) return ATTN_ERR_SHAPE;
  const int st = check_prefill(q, k, v, B, Hq, Hkv, Sq, Skv, d, dtype, causal, scale, num_splits);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) return ATTN_OK;
  if (part_o == nullptr || part_lse == nullptr) return ATTN_ERR_NULL;
  if (!aligned16(part_o) || !aligned16(part_lse)) return ATTN_ERR_ALIGN;

  sa::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.o = nullptr; a.lse = nullptr;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Skv = Skv; a.d = d;
  a.bf16 = true;
  a.causal = causal != 0;
  a.scale = scale;
  a.n_splits = num_splits; a.part_o = part_o; a.part_lse = part_lse;
  return sa::launch_prefill(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* kv_len, const int32_t* num_splits_seq, int32_t B, int32_t Hq, int32_t Hkv,
                      int32_t T_q, int32_t num_pages, int32_t max_pages, int32_t d, int32_t num_splits,
                      attn_dtype_t dtype, float scale, float* part_o, float* part_lse, void* o, float* lse,
                      hipStream_t stream) {
  if (B < 0 || T_q < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || num_pages < 1 || max_pages < 1)
    return ATTN_ERR_SHAPE;
  if (num_splits < 1 || num_splits > 256) return ATTN_ERR_SHAPE;
  if (!good_scale(scale)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  const long long G = Hq / Hkv;
  if ((long long)max_pages * 64 > 0x7fffffffLL || G * T_q * d * 2 > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  const long long n_mt = (G * T_q + 127) / 128;
  if (n_mt * (long long)B * Hkv * num_splits > kMaxGrid) return ATTN_ERR_SHAPE;
  if (B == 0 || T_q == 0) return ATTN_OK;
  if (q == nullptr || k_pages == nullptr || v_pages == nullptr || block_table == nullptr || kv_len == nullptr)
    return ATTN_ERR_NULL;
  if (num_splits > 1 ? (part_o == nullptr || part_lse == nullptr) : o == nullptr) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) ||
      (num_splits > 1 ? (!aligned16(part_o) || !aligned16(part_lse)) : (!aligned16(o) || !aligned16(lse))))
    return ATTN_ERR_ALIGN;

  sa::PrefillArgs a;
  a.q = q; a.k = k_pages; a.v = v_pages;
  a.o = num_splits > 1 ? nullptr : o;
  a.lse = num_splits > 1 ? nullptr : lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = T_q; a.Skv = 0; a.d = d;
  a.bf16 = true;
  a.causal = true;
  a.scale = scale;
  a.n_splits = num_splits;
  a.part_o = num_splits > 1 ? part_o : nullptr;
  a.part_lse = num_splits > 1 ? part_lse : nullptr;
  a.block_table = block_table; a.kv_len = kv_len; a.max_pages = max_pages; a.num_pages = num_pages;
  a.seq_splits = num_splits > 1 ? num_splits_seq : nullptr;
  const hipError_t e = sa::decode_paged_fits(Hq, Hkv, T_q, d) ? sa::launch_decode_paged(a, stream)
                                                               : sa::launch_prefill(a, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                        const int32_t* num_splits, int32_t B, int32_t Hq, int32_t Hkv, int32_t S_cap, int32_t d,
                        int32_t max_splits, attn_dtype_t dtype, float scale, float* part_o, float* part_lse,
                        hipStream_t stream) {
  if (B < 0 || S_cap < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (max_splits < 1 || max_splits > 256) return ATTN_ERR_SHAPE;
  if (!good_scale(scale)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * Hkv * max_splits > kMaxGrid) return ATTN_ERR_SHAPE;
  if (B == 0) return ATTN_OK;
  if (q == nullptr || part_o == nullptr || part_lse == nullptr) return ATTN_ERR_NULL;
  if (S_cap > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(part_o) || !aligned16(part_lse) ||
      (S_cap > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return ATTN_ERR_ALIGN;

  sa::DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.kv_len = kv_len; a.num_splits = num_splits;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S_cap = S_cap; a.d = d; a.max_splits = max_splits;
  a.scale = scale; a.part_o = part_o; a.part_lse = part_lse;
  a.counters = nullptr; a.o = nullptr; a.lse = nullptr;
  return sa::launch_decode_splitkv(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                const int32_t* num_splits, int32_t B, int32_t Hq, int32_t Hkv, int32_t S_cap, int32_t d,
                int32_t max_splits, attn_dtype_t dtype, float scale, float* part_o, float* part_lse, int32_t* counters,
                void* o, float* lse, hipStream_t stream) {
  if (B < 0 || S_cap < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (max_splits < 1 || max_splits > 256) return ATTN_ERR_SHAPE;
  if (!good_scale(scale)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * Hkv * max_splits > kMaxGrid) return ATTN_ERR_SHAPE;
  if (B == 0) return ATTN_OK;
  if (q == nullptr || part_o == nullptr || part_lse == nullptr || counters == nullptr || o == nullptr)
    return ATTN_ERR_NULL;
  if (S_cap > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(part_o) || !aligned16(part_lse) || !aligned16(counters) || !aligned16(o) ||
      !aligned16(lse) || (S_cap > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return ATTN_ERR_ALIGN;

  sa::DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.kv_len = kv_len; a.num_splits = num_splits;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S_cap = S_cap; a.d = d; a.max_splits = max_splits;
  a.scale = scale; a.part_o = part_o; a.part_lse = part_lse;
  a.counters = counters; a.o = o; a.lse = lse;
  return sa::launch_decode_splitkv(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                        const int32_t* num_splits, int32_t B, int32_t Hq, int32_t Hkv, int32_t S_cap, int32_t d,
                        int32_t max_splits, attn_dtype_t dtype, float scale, void* o, float* lse,
                        hipStream_t stream) {
  const int st = check_decode(B, Hq, Hkv, S_cap, d, max_splits, dtype, scale);
  if (st != ATTN_OK) return st;
  if ((long long)B * Hq * max_splits > ATTN_NOALLOC_MAX_PARTIALS) return ATTN_ERR_WORKSPACE;
  if (B == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (S_cap > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(o) || !aligned16(lse) || (S_cap > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return ATTN_ERR_ALIGN;
  unsigned char* ws = nullptr;
  const int sst = scratch_address(stream, &ws);
  if (sst != ATTN_OK) return sst;
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(ws + kNoallocLseOffset);

  // The split sweep writes every partial the merge reads (splits s < n_b of
  // each row), so nothing in the workspace has to start at zero.
  sa::DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.kv_len = kv_len; a.num_splits = num_splits;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S_cap = S_cap; a.d = d; a.max_splits = max_splits;
  a.scale = scale; a.part_o = part_o; a.part_lse = part_lse;
  a.counters = nullptr; a.o = nullptr; a.lse = nullptr;
  if (sa::launch_decode_splitkv(a, stream) != hipSuccess) return ATTN_ERR_LAUNCH;
  sa::CombineArgs c;
  c.part_o = part_o; c.part_lse = part_lse; c.num_splits = num_splits;
  c.B = B; c.Hq = Hq; c.max_splits = max_splits; c.d = d;
  c.o = o; c.lse = lse; c.out_bf16 = true;
  return sa::launch_combine_lse(c, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_combine_lse(const float* part_o, const float* part_lse, const int32_t* num_splits, int32_t B,
                     int32_t Hq, int32_t max_splits, int32_t d, void* o, float* lse, attn_dtype_t out_dtype,
                     hipStream_t stream) {
  if (B < 0 || Hq < 1) return ATTN_ERR_SHAPE;
  if (max_splits < 1 || max_splits > 256) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (out_dtype != ATTN_DTYPE_BF16 && out_dtype != ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * Hq > kMaxGrid) return ATTN_ERR_SHAPE;
  if (B == 0) return ATTN_OK;
  if (part_o == nullptr || part_lse == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (!aligned16(part_o) || !aligned16(part_lse) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;

  sa::CombineArgs a;
  a.part_o = part_o; a.part_lse = part_lse; a.num_splits = num_splits;
  a.B = B; a.Hq = Hq; a.max_splits = max_splits; a.d = d;
  a.o = o; a.lse = lse; a.out_bf16 = out_dtype == ATTN_DTYPE_BF16;
  return sa::launch_combine_lse(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
