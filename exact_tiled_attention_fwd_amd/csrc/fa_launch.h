// fa_launch.h - internal interface between the C ABI (fa_api.cpp) and the
// kernel translation units. Not installed; callers use include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Element strides of (batch, head, row) for q, k, v and o; the head-dim
// stride is 1. A packed batch uses the head and row (token) strides only.
struct Layout {
  long long q[3], k[3], v[3], o[3];
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int dtype;
  // Packed variable-length batch (cu_q != nullptr): q, o hold total_q tokens
  // per head, k, v total_k per kv-head (addressed through `layout`), lse
  // [Hq, total_q]; Nq / Nk unused; query tiles cover max_seqlen_q rows per
  // sequence.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k, max_seqlen_q;
  Layout layout;
};

// Decode key split: chunk keys per workgroup, n_split chunks cover Lcap rows.
// Decode split plan. The split kernel gives every wave an equal share of the
// cached rows (at least `chunk` of them), so one (sequence, kv-head) pair
// yields at most n_split + 1 partial results ("slots").
struct DecodePlan {
  int chunk;
  int n_split;
  int slots;             // partial results per (sequence, q-head): n_split + 1
  size_t ws_lse_offset;  // bytes from workspace start to the LSE partials
  size_t ws_hdr_offset;  // bytes from workspace start to the split header
  size_t ws_bytes;       // total workspace bytes
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* seqlens;
  void* o;
  float* lse;
  void* workspace;
  size_t ws_lse_offset, ws_hdr_offset;
  int B, Hq, Hkv, Lcap, d;
  float scale;
  int chunk, slots;
  int dtype;
  // Paged cache (block_table != nullptr): k_cache / v_cache are
  // [num_pages, Hkv, page_size, d] and Lcap = max_pages * page_size.
  const int32_t* block_table;
  int page_size, max_pages, num_pages;
};

constexpr int kDecodeTileRows = 128;
constexpr int kFwdBlockRows = 256;  // query rows per prefill workgroup

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
int set_fwd_schedule(int mode);  // FA_SCHEDULE_*; previous mode or -1
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// The static decode workspace behind fa_decode_noalloc (fa.h): its size and
// its device address on the current device (looked up on the first call
// per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace fa
