// fa_api.cpp - the C ABI of include/fa.h: argument validation, the decode
// split plan, per-device capability check and kernel dispatch. Nothing here
// allocates device memory or synchronises; every check runs before any
// launch, so a rejected call writes nothing.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "fa_launch.h"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [p, p+n) and [q, q+m) overlap?
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || !n || !m) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

// Product of positive ints into bytes, false on overflow past 2^62.
bool mul_bytes(size_t& out, std::initializer_list<long long> xs) {
  unsigned __int128 acc = 1;
  for (long long x : xs) {
    acc *= (unsigned __int128)x;
    if (acc > ((unsigned __int128)1 << 62)) return false;
  }
  out = (size_t)acc;
  return true;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
std::mutex g_dev_mu;
int g_dev_ok[256];

fa_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 256) return fail(FA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (g_dev_ok[dev] == 2) return fail(FA_ERR_UNSUPPORTED, "device %d is %s, this library targets gfx950", dev, prop.gcnArchName);
  }
  if (g_dev_ok[dev] != 1) return fail(FA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return FA_OK;
}

fa_status check_common(int d, int dtype, float scale, int Hq, int Hkv) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return fail(FA_ERR_UNSUPPORTED, "dtype %d is not bf16 (0) or fp16 (1)", dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head width d=%d is not 64 or 128", d);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  return FA_OK;
}

fa::DecodePlan make_plan(int B, int Hkv, int Lcap, int num_splits, int Hq, int d) {
  const int R = fa::kDecodeTileRows;
  long long chunk;
  if (num_splits > 0) {
    chunk = ((long long)Lcap + num_splits - 1) / num_splits;
  } else {
    // Enough workgroups to cover the GPU several times over, chunks of at
    // least one tile; long caches get 512-key chunks.
    chunk = 512;
    while (chunk > R && (long long)B * Hkv * (((long long)Lcap + chunk - 1) / chunk) < 4096) chunk /= 2;
  }
  chunk = ((chunk + R - 1) / R) * R;
  if (chunk > (1LL << 30)) chunk = 1LL << 30;
  fa::DecodePlan p;
  p.chunk = (int)chunk;
  p.n_split = (int)(((long long)Lcap + chunk - 1) / chunk);
  const size_t rows = (size_t)B * Hq * p.n_split;
  const size_t o_bytes = ((rows * d * sizeof(float)) + 255) & ~(size_t)255;
  const size_t l_bytes = ((rows * sizeof(float)) + 255) & ~(size_t)255;
  p.ws_lse_offset = o_bytes;
  p.ws_bytes = o_bytes + l_bytes;
  return p;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return 1; }

const char* fa_status_string(int s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d)", B, Hq, Hkv, Nq, Nk, d);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  fa_status st = check_common(d, dtype, scale, Hq, Hkv);
  if (st != FA_OK) return st;
  if (causal && Nq > Nk) return fail(FA_ERR_INVALID_ARG, "causal attention needs Nq <= Nk (Nq=%d Nk=%d)", Nq, Nk);
  size_t qb, kb, lb;
  if (!mul_bytes(qb, {B, Hq, Nq, d, 2}) || !mul_bytes(kb, {B, Hkv, Nk, d, 2}) || !mul_bytes(lb, {B, Hq, Nq, 4}))
    return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  if ((long long)((Nq + fa::kFwdBlockRows - 1) / fa::kFwdBlockRows) * B * Hq > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse && (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) || overlap(lse, lb, o, qb)))
    return fail(FA_ERR_INVALID_ARG, "lse overlaps another tensor");
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, nullptr, nullptr, 0, 0, 0};
  hipError_t e = fa::launch_fwd(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd launch: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k,
                         int max_seqlen_q, int d, float scale, int causal, int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k)
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o, cu_seqlens_q and cu_seqlens_k must be non-null");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be 4-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || total_q <= 0 || total_k <= 0 || max_seqlen_q <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG,
                "sizes must be positive (B=%d Hq=%d Hkv=%d total_q=%d total_k=%d max_seqlen_q=%d d=%d)", B, Hq, Hkv,
                total_q, total_k, max_seqlen_q, d);
  if (max_seqlen_q > total_q) return fail(FA_ERR_INVALID_ARG, "max_seqlen_q=%d exceeds total_q=%d", max_seqlen_q, total_q);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  fa_status st = check_common(d, dtype, scale, Hq, Hkv);
  if (st != FA_OK) return st;
  size_t qb, kb, lb;
  if (!mul_bytes(qb, {Hq, total_q, d, 2}) || !mul_bytes(kb, {Hkv, total_k, d, 2}) || !mul_bytes(lb, {Hq, total_q, 4}))
    return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  if ((long long)((max_seqlen_q + fa::kFwdBlockRows - 1) / fa::kFwdBlockRows) * B * Hq > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse && (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) || overlap(lse, lb, o, qb)))
    return fail(FA_ERR_INVALID_ARG, "lse overlaps another tensor");
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, 0, 0, d, scale, causal, dtype,
                cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q};
  hipError_t e = fa::launch_fwd(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_varlen launch: %s", hipGetErrorString(e));
  return FA_OK;
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Lcap, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lcap <= 0 || (d != 64 && d != 128) || num_splits < 0 || Hq % Hkv) return 0;
  return make_plan(B, Hkv, Lcap, num_splits, Hq, d).ws_bytes;
}

}  // extern "C"

namespace {

// Shared by fa_decode and fa_decode_paged: cache_elems is the element count
// of each of k_cache / v_cache; table != nullptr selects the paged layout.
fa_status decode_impl(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* table, const int32_t* seqlens, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, int B, int Hq, int Hkv, int Lcap, int d, float scale, int num_splits,
                      int dtype, void* stream, size_t cache_bytes, int page_size, int max_pages, int num_pages) {
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", fn);
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "%s: num_splits must be >= 0", fn);
  fa_status st = check_common(d, dtype, scale, Hq, Hkv);
  if (st != FA_OK) return st;
  if (Hq / Hkv > 32) return fail(FA_ERR_UNSUPPORTED, "at most 32 q-heads per kv-head (got %d)", Hq / Hkv);
  if (B > 65535 || Hkv > 65535) return fail(FA_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  size_t qb;
  if (!mul_bytes(qb, {B, Hq, d, 2})) return fail(FA_ERR_INVALID_ARG, "%s: tensor sizes overflow", fn);
  const fa::DecodePlan p = make_plan(B, Hkv, Lcap, num_splits, Hq, d);
  if (workspace_bytes < p.ws_bytes)
    return fail(FA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, p.ws_bytes);
  const size_t cb = cache_bytes;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k_cache, cb) || overlap(o, qb, v_cache, cb) ||
      overlap(workspace, p.ws_bytes, q, qb) || overlap(workspace, p.ws_bytes, k_cache, cb) ||
      overlap(workspace, p.ws_bytes, v_cache, cb) || overlap(workspace, p.ws_bytes, o, qb))
    return fail(FA_ERR_INVALID_ARG, "o or workspace overlaps another tensor");
  st = check_device();
  if (st != FA_OK) return st;
  fa::DecodeArgs a{q, k_cache, v_cache, seqlens, o, lse, workspace, p.ws_lse_offset, B, Hq, Hkv, Lcap, d, scale,
                   p.chunk, p.n_split, dtype, table, page_size, max_pages, num_pages};
  hipError_t e = fa::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens, void* o,
                    float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Lcap, int d,
                    float scale, int num_splits, int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !k_cache || !v_cache || !seqlens || !o || !workspace)
    return fail(FA_ERR_INVALID_ARG, "q, k_cache, v_cache, seqlens, o and workspace must be non-null");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  if (!aligned(seqlens, 4)) return fail(FA_ERR_INVALID_ARG, "seqlens must be 4-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lcap <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d Lcap=%d d=%d)", B, Hq, Hkv, Lcap, d);
  size_t cb;
  if (!mul_bytes(cb, {B, Hkv, Lcap, d, 2})) return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  return decode_impl("fa_decode", q, k_cache, v_cache, nullptr, seqlens, o, lse, workspace, workspace_bytes, B, Hq,
                     Hkv, Lcap, d, scale, num_splits, dtype, stream, cb, 0, 0, 0);
}

fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                          const int32_t* seqlens, void* o, float* lse, void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d, float scale,
                          int num_splits, int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !k_pages || !v_pages || !block_table || !seqlens || !o || !workspace)
    return fail(FA_ERR_INVALID_ARG, "q, k_pages, v_pages, block_table, seqlens, o and workspace must be non-null");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k_pages, v_pages and o must be 16-byte aligned");
  if (!aligned(seqlens, 4) || !aligned(block_table, 4))
    return fail(FA_ERR_INVALID_ARG, "seqlens and block_table must be 4-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || num_pages <= 0 || page_size <= 0 || max_pages <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d num_pages=%d page_size=%d max_pages=%d d=%d)",
                B, Hq, Hkv, num_pages, page_size, max_pages, d);
  if (page_size % 32 != 0) return fail(FA_ERR_UNSUPPORTED, "page_size must be a multiple of 32 (got %d)", page_size);
  const long long Lcap = (long long)max_pages * page_size;
  if (Lcap > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "max_pages * page_size overflows int");
  size_t cb, tb;
  if (!mul_bytes(cb, {num_pages, Hkv, page_size, d, 2}) || !mul_bytes(tb, {B, max_pages, 4}))
    return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  return decode_impl("fa_decode_paged", q, k_pages, v_pages, block_table, seqlens, o, lse, workspace,
                     workspace_bytes, B, Hq, Hkv, (int)Lcap, d, scale, num_splits, dtype, stream, cb, page_size,
                     max_pages, num_pages);
}

}  // extern "C"
