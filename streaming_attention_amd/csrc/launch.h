// Host-side launch interfaces between the C ABI layer and the kernel files.
// Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Sq, Skv, d;
  bool bf16;
  bool causal;
  float scale;
  // Split-KV mode (bf16 only) when part_o is non-null: fp32 partials
  // [B, Hq, Sq, n_splits, d] and [B, Hq, Sq, n_splits] instead of o / lse.
  int n_splits = 1;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  // Paged multi-token decode when block_table is non-null: k / v are page
  // pools [num_pages, Hkv, 64, d], block_table [B, max_pages], kv_len [B].
  const int32_t* block_table = nullptr;
  const int32_t* kv_len = nullptr;
  int max_pages = 0;
  int num_pages = 0;
  const int32_t* seq_splits = nullptr;   // per-sequence split counts (paged), or null
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* kv_len;
  const int32_t* num_splits;
  int B, Hq, Hkv, S_cap, d, max_splits;
  float scale;
  float* part_o;
  float* part_lse;
  // Fused merge (attn_decode) when counters is non-null.
  int32_t* counters;
  void* o;
  float* lse;
};

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* num_splits;
  int B, Hq, max_splits, d;
  void* o;
  float* lse;
  bool out_bf16;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode_splitkv(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_combine_lse(const CombineArgs& a, hipStream_t stream);
// Paged multi-token decode for small query blocks (G * T_q <= 32, d 64 or 128):
// the streaming decode kernel; other paged shapes run the prefill kernel's
// paged mode (launch_prefill with block_table set).
bool decode_paged_fits(int Hq, int Hkv, int T_q, int d);
hipError_t launch_decode_paged(const PrefillArgs& a, hipStream_t stream);

}  // namespace sa
