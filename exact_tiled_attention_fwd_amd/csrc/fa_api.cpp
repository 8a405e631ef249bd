// fa_api.cpp - the C ABI of include/fa.h: argument validation, the decode
// split plan, per-device capability check and kernel dispatch. Nothing here
// allocates device memory or synchronises; every check runs before any
// launch, so a rejected call writes nothing.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "fa_bwd_launch.h"
#include "fa_fp8_launch.h"
#include "fa_launch.h"

static_assert(fa::kNoAllocScratchBytes == FA_NOALLOC_SCRATCH_BYTES, "static decode workspace size");

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

// A byte range of one argument (ptr may be null, then it overlaps nothing).
struct Span {
  const void* p;
  size_t n;
};

// Does any output range overlap an input range or another output range?
bool outputs_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (const Span* a = outs.begin(); a != outs.end(); ++a) {
    for (const Span& b : ins)
      if (overlap(a->p, a->n, b.p, b.n)) return true;
    for (const Span* b = a + 1; b != outs.end(); ++b)
      if (overlap(a->p, a->n, b->p, b->n)) return true;
  }
  return false;
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
    // The smallest share of rows a split wave takes: 512 keys for long
    // caches, less (down to one 128-row tile) when there are few rows in
    // all, so that small batches still spread over many waves.
    chunk = 512;
    while (chunk > R && (long long)B * Hkv * (((long long)Lcap + chunk - 1) / chunk) < 4096) chunk /= 2;
  }
  chunk = ((chunk + R - 1) / R) * R;
  if (chunk > (1LL << 30)) chunk = 1LL << 30;
  fa::DecodePlan p;
  p.chunk = (int)chunk;
  p.n_split = (int)(((long long)Lcap + chunk - 1) / chunk);
  p.slots = p.n_split + 1;
  const size_t rows = (size_t)B * Hq * p.slots;
  const size_t o_bytes = ((rows * d * sizeof(float)) + 255) & ~(size_t)255;
  const size_t l_bytes = ((rows * sizeof(float)) + 255) & ~(size_t)255;
  const size_t h_bytes = (((size_t)B + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
  p.ws_lse_offset = o_bytes;
  p.ws_hdr_offset = o_bytes + l_bytes;
  p.ws_bytes = o_bytes + l_bytes + h_bytes;
  return p;
}

// Element strides of one tensor dimension.
struct Dim {
  long long size, stride;
};

// Largest element offset any index reaches (strides >= 0), or -1 on overflow
// past 2^61.
long long max_offset(std::initializer_list<Dim> dims, int d) {
  __int128 acc = d - 1;
  for (const Dim& x : dims) acc += (__int128)(x.size - 1) * x.stride;
  return acc > ((__int128)1 << 61) ? -1 : (long long)acc;
}

// No two indices of the tensor share an element: with the dimensions of more
// than one index sorted by stride, each stride exceeds the largest offset the
// smaller ones reach (the head-dim has stride 1 and d entries).
bool rows_disjoint(std::initializer_list<Dim> dims, int d) {
  Dim ds[4];
  int n = 0;
  ds[n++] = Dim{d, 1};
  for (const Dim& x : dims)
    if (x.size > 1) ds[n++] = x;
  std::sort(ds, ds + n, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
  __int128 reach = 0;
  for (int i = 0; i < n; ++i) {
    if ((__int128)ds[i].stride <= reach) return false;
    reach += (__int128)(ds[i].size - 1) * ds[i].stride;
  }
  return true;
}

// Shared by fa_fwd, fa_fwd_strided, fa_fwd_varlen and fa_fwd_varlen_strided.
// cu_q != nullptr selects the packed layout (Nq, Nk unused; batch strides
// ignored).
fa_status fwd_impl(const char* fn, const void* q, const void* k, const void* v, void* o, float* lse,
                   const fa::Layout& ly, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, void* stream, const int32_t* cu_q, const int32_t* cu_k, int total_q, int total_k,
                   int max_seqlen_q) {
  const bool packed = cu_q != nullptr || cu_k != nullptr;
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "%s: q, k, v and o must be non-null", fn);
  if (packed && (!cu_q || !cu_k))
    return fail(FA_ERR_INVALID_ARG, "%s: cu_seqlens_q and cu_seqlens_k must be non-null", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
  if (packed && (!aligned(cu_q, 4) || !aligned(cu_k, 4)))
    return fail(FA_ERR_INVALID_ARG, "%s: cu_seqlens_q and cu_seqlens_k must be 4-byte aligned", fn);
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", fn);
  if (packed) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || total_q <= 0 || total_k <= 0 || max_seqlen_q <= 0 || d <= 0)
      return fail(FA_ERR_INVALID_ARG,
                  "%s: sizes must be positive (B=%d Hq=%d Hkv=%d total_q=%d total_k=%d max_seqlen_q=%d d=%d)", fn, B,
                  Hq, Hkv, total_q, total_k, max_seqlen_q, d);
    if (max_seqlen_q > total_q)
      return fail(FA_ERR_INVALID_ARG, "%s: max_seqlen_q=%d exceeds total_q=%d", fn, max_seqlen_q, total_q);
  } else if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) {
    return fail(FA_ERR_INVALID_ARG, "%s: sizes must be positive (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d)", fn, B, Hq, Hkv,
                Nq, Nk, d);
  }
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "%s: causal must be 0 or 1", fn);
  fa_status st = check_common(d, dtype, scale, Hq, Hkv);
  if (st != FA_OK) return st;
  if (!packed && causal && Nq > Nk)
    return fail(FA_ERR_INVALID_ARG, "%s: causal attention needs Nq <= Nk (Nq=%d Nk=%d)", fn, Nq, Nk);
  // Strides: non-negative multiples of 8 elements (16-byte rows); row strides
  // below 2^24 elements (32-bit offsets within a key tile), others below 2^40.
  const long long* all[4] = {ly.q, ly.k, ly.v, ly.o};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t)
    for (int i = packed ? 1 : 0; i < 3; ++i) {
      const long long x = all[t][i];
      if (x < 0 || (x & 7) || x >= (i == 2 ? (1LL << 24) : (1LL << 40)))
        return fail(FA_ERR_INVALID_ARG,
                    "%s: stride %d of %s is %lld; strides must be non-negative multiples of 8 elements, row strides "
                    "below 2^24 and the others below 2^40",
                    fn, i, names[t], x);
    }
  const long long bq = packed ? 1 : B, rq = packed ? total_q : Nq, rk = packed ? total_k : Nk;
  const long long oq = max_offset({{bq, ly.q[0]}, {Hq, ly.q[1]}, {rq, ly.q[2]}}, d);
  const long long ok = max_offset({{bq, ly.k[0]}, {Hkv, ly.k[1]}, {rk, ly.k[2]}}, d);
  const long long ov = max_offset({{bq, ly.v[0]}, {Hkv, ly.v[1]}, {rk, ly.v[2]}}, d);
  const long long oo = max_offset({{bq, ly.o[0]}, {Hq, ly.o[1]}, {rq, ly.o[2]}}, d);
  size_t lb;
  if (oq < 0 || ok < 0 || ov < 0 || oo < 0 || !mul_bytes(lb, {bq, Hq, rq, 4}))
    return fail(FA_ERR_INVALID_ARG, "%s: tensor sizes overflow", fn);
  if (!rows_disjoint({{bq, ly.o[0]}, {Hq, ly.o[1]}, {rq, ly.o[2]}}, d))
    return fail(FA_ERR_INVALID_ARG, "%s: the strides of o make two of its elements share memory", fn);
  const int rows = packed ? max_seqlen_q : Nq;
  if ((long long)((rows + fa::kFwdBlockRows - 1) / fa::kFwdBlockRows) * B * Hq > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  const size_t qb = 2 * (size_t)(oq + 1), kb = 2 * (size_t)(ok + 1), vb = 2 * (size_t)(ov + 1),
               obb = 2 * (size_t)(oo + 1);
  const size_t cub = packed ? ((size_t)B + 1) * sizeof(int32_t) : 0;
  if (outputs_overlap({{o, obb}}, {{q, qb}, {k, kb}, {v, vb}, {cu_q, cub}, {cu_k, cub}}))
    return fail(FA_ERR_INVALID_ARG, "%s: o overlaps an input", fn);
  if (lse && outputs_overlap({{lse, lb}, {o, obb}}, {{q, qb}, {k, kb}, {v, vb}, {cu_q, cub}, {cu_k, cub}}))
    return fail(FA_ERR_INVALID_ARG, "%s: lse overlaps another tensor", fn);
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, cu_q, cu_k, total_q, total_k,
                max_seqlen_q, ly};
  hipError_t e = fa::launch_fwd(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return FA_OK;
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

int fa_set_prefill_schedule(int mode) { return fa::set_fwd_schedule(mode); }

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, int dtype, void* stream) {
  g_last_error.clear();
  const long long qh = (long long)Nq * d, kh = (long long)Nk * d;
  const fa::Layout ly{{(long long)Hq * qh, qh, d}, {(long long)Hkv * kh, kh, d}, {(long long)Hkv * kh, kh, d},
                      {(long long)Hq * qh, qh, d}};
  return fwd_impl("fa_fwd", q, k, v, o, lse, ly, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream, nullptr,
                  nullptr, 0, 0, 0);
}

fa_status fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, const int64_t* strides,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                         void* stream) {
  g_last_error.clear();
  if (!strides) return fail(FA_ERR_INVALID_ARG, "fa_fwd_strided: strides must be non-null");
  fa::Layout ly;
  for (int i = 0; i < 3; ++i) {
    ly.q[i] = strides[i];
    ly.k[i] = strides[3 + i];
    ly.v[i] = strides[6 + i];
    ly.o[i] = strides[9 + i];
  }
  return fwd_impl("fa_fwd_strided", q, k, v, o, lse, ly, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream, nullptr,
                  nullptr, 0, 0, 0);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k,
                         int max_seqlen_q, int d, float scale, int causal, int dtype, void* stream) {
  g_last_error.clear();
  const long long qh = (long long)total_q * d, kh = (long long)total_k * d;
  const fa::Layout ly{{0, qh, d}, {0, kh, d}, {0, kh, d}, {0, qh, d}};
  return fwd_impl("fa_fwd_varlen", q, k, v, o, lse, ly, B, Hq, Hkv, 0, 0, d, scale, causal, dtype, stream,
                  cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q);
}

fa_status fa_fwd_varlen_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int64_t* strides, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int d,
                                float scale, int causal, int dtype, void* stream) {
  g_last_error.clear();
  if (!strides) return fail(FA_ERR_INVALID_ARG, "fa_fwd_varlen_strided: strides must be non-null");
  const fa::Layout ly{{0, strides[0], strides[1]}, {0, strides[2], strides[3]}, {0, strides[4], strides[5]},
                      {0, strides[6], strides[7]}};
  return fwd_impl("fa_fwd_varlen_strided", q, k, v, o, lse, ly, B, Hq, Hkv, 0, 0, d, scale, causal, dtype, stream,
                  cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q);
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
                      int dtype, void* stream, size_t cache_bytes, size_t table_bytes, int page_size, int max_pages,
                      int num_pages) {
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", fn);
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "%s: num_splits must be >= 0", fn);
  fa_status st = check_common(d, dtype, scale, Hq, Hkv);
  if (st != FA_OK) return st;
  if (Hq / Hkv > 32) return fail(FA_ERR_UNSUPPORTED, "at most 32 q-heads per kv-head (got %d)", Hq / Hkv);
  if (B > 65535 || Hkv > 65535) return fail(FA_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  if ((long long)B * Hkv * (((long long)Lcap + 31) / 32) > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "%s: B * Hkv * ceil(Lcap / 32) must fit in int32", fn);
  size_t qb;
  if (!mul_bytes(qb, {B, Hq, d, 2})) return fail(FA_ERR_INVALID_ARG, "%s: tensor sizes overflow", fn);
  const fa::DecodePlan p = make_plan(B, Hkv, Lcap, num_splits, Hq, d);
  if (workspace_bytes < p.ws_bytes)
    return fail(FA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, p.ws_bytes);
  const size_t cb = cache_bytes, lb = lse ? (size_t)B * Hq * sizeof(float) : 0, sb = (size_t)B * sizeof(int32_t);
  if (outputs_overlap({{o, qb}, {lse, lb}, {workspace, p.ws_bytes}},
                      {{q, qb}, {k_cache, cb}, {v_cache, cb}, {seqlens, sb}, {table, table_bytes}}))
    return fail(FA_ERR_INVALID_ARG, "%s: o, lse or the workspace overlaps another argument", fn);
  st = check_device();
  if (st != FA_OK) return st;
  fa::DecodeArgs a{q, k_cache, v_cache, seqlens, o, lse, workspace, p.ws_lse_offset, p.ws_hdr_offset, B, Hq, Hkv,
                   Lcap, d, scale, p.chunk, p.slots, dtype, table, page_size, max_pages, num_pages};
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
                     Hkv, Lcap, d, scale, num_splits, dtype, stream, cb, 0, 0, 0, 0);
}

fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                            void* o, float* lse, int B, int Hq, int Hkv, int Lcap, int d, float scale, int num_splits,
                            int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !k_cache || !v_cache || !seqlens || !o)
    return fail(FA_ERR_INVALID_ARG, "q, k_cache, v_cache, seqlens and o must be non-null");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  if (!aligned(seqlens, 4)) return fail(FA_ERR_INVALID_ARG, "seqlens must be 4-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lcap <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d Lcap=%d d=%d)", B, Hq, Hkv, Lcap, d);
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "fa_decode_noalloc: num_splits must be >= 0");
  fa_status st = check_common(d, dtype, scale, Hq, Hkv);
  if (st != FA_OK) return st;
  size_t cb;
  if (!mul_bytes(cb, {B, Hkv, Lcap, d, 2})) return fail(FA_ERR_INVALID_ARG, "tensor sizes overflow");
  const size_t need = make_plan(B, Hkv, Lcap, num_splits, Hq, d).ws_bytes;
  if (need > fa::kNoAllocScratchBytes)
    return fail(FA_ERR_INVALID_ARG,
                "fa_decode_noalloc: this decode needs a %zu-byte workspace, more than the %zu-byte static one "
                "(use fa_decode with a caller-owned workspace)", need, fa::kNoAllocScratchBytes);
  st = check_device();
  if (st != FA_OK) return st;
  void* ws = nullptr;
  const hipError_t e = fa::noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_decode_noalloc: scratch address: %s", hipGetErrorString(e));
  return decode_impl("fa_decode_noalloc", q, k_cache, v_cache, nullptr, seqlens, o, lse, ws, fa::kNoAllocScratchBytes,
                     B, Hq, Hkv, Lcap, d, scale, num_splits, dtype, stream, cb, 0, 0, 0, 0);
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
                     workspace_bytes, B, Hq, Hkv, (int)Lcap, d, scale, num_splits, dtype, stream, cb, tb,
                     page_size, max_pages, num_pages);
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, const float* q_descale,
                     const float* k_descale, const float* v_descale, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !q_descale || !k_descale || !v_descale)
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: q, k, v, o and the three descale arrays must be non-null");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: q, k, v and o must be 16-byte aligned");
  if (!aligned(q_descale, 4) || !aligned(k_descale, 4) || !aligned(v_descale, 4) || (lse && !aligned(lse, 4)))
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: descales and lse must be 4-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: sizes must be positive (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d)", B, Hq,
                Hkv, Nq, Nk, d);
  if (d != 128) return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: head width d=%d is not 128", d);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: causal must be 0 or 1");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: scale must be finite and > 0 (got %g)", (double)scale);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (causal && Nq > Nk)
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: causal attention needs Nq <= Nk (Nq=%d Nk=%d)", Nq, Nk);
  size_t qb, kb, ob, lb, dqb, dkb;
  if (!mul_bytes(qb, {B, Hq, Nq, d}) || !mul_bytes(kb, {B, Hkv, Nk, d}) || !mul_bytes(ob, {B, Hq, Nq, d, 2}) ||
      !mul_bytes(lb, {B, Hq, Nq, 4}) || !mul_bytes(dqb, {B, Hq, 4}) || !mul_bytes(dkb, {B, Hkv, 4}))
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: tensor sizes overflow");
  if ((long long)((Nq + fa::kFp8BlockRows - 1) / fa::kFp8BlockRows) * B * Hq > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: grid too large");
  if (overlap(o, ob, q, qb) || overlap(o, ob, k, kb) || overlap(o, ob, v, kb) || overlap(o, ob, q_descale, dqb) ||
      overlap(o, ob, k_descale, dkb) || overlap(o, ob, v_descale, dkb))
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: o overlaps an input");
  if (lse && outputs_overlap({{lse, lb}, {o, ob}},
                             {{q, qb}, {k, kb}, {v, kb}, {q_descale, dqb}, {k_descale, dkb}, {v_descale, dkb}}))
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: lse overlaps another tensor");
  fa_status st = check_device();
  if (st != FA_OK) return st;
  fa::Fp8Args a{static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), o,
                lse, q_descale, k_descale, v_descale, B, Hq, Hkv, Nq, Nk, scale, causal};
  hipError_t e = fa::launch_fwd_fp8(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_fp8 launch: %s", hipGetErrorString(e));
  return FA_OK;
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq) {
  size_t n;
  if (B <= 0 || Hq <= 0 || Nq <= 0 || !mul_bytes(n, {B, Hq, Nq, 4})) return 0;
  return (n + 255) & ~(size_t)255;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                 int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return fail(FA_ERR_INVALID_ARG, "fa_bwd: q, k, v, o, lse, dout, dq, dk, dv and workspace must be non-null");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(FA_ERR_INVALID_ARG, "fa_bwd: q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(workspace, 256))
    return fail(FA_ERR_INVALID_ARG, "fa_bwd: lse must be 4-byte and workspace 256-byte aligned");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "fa_bwd: sizes must be positive (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d)", B, Hq, Hkv,
                Nq, Nk, d);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "fa_bwd: causal must be 0 or 1");
  fa_status st = check_common(d, dtype, scale, Hq, Hkv);
  if (st != FA_OK) return st;
  if (causal && Nq > Nk)
    return fail(FA_ERR_INVALID_ARG, "fa_bwd: causal attention needs Nq <= Nk (Nq=%d Nk=%d)", Nq, Nk);
  size_t qb, kb, lb;
  if (!mul_bytes(qb, {B, Hq, Nq, d, 2}) || !mul_bytes(kb, {B, Hkv, Nk, d, 2}) || !mul_bytes(lb, {B, Hq, Nq, 4}))
    return fail(FA_ERR_INVALID_ARG, "fa_bwd: tensor sizes overflow");
  const size_t need = fa_bwd_workspace_bytes(B, Hq, Nq);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "fa_bwd: workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  if ((long long)((Nq + fa::kBwdQueryRows - 1) / fa::kBwdQueryRows) * B * Hq > 0x7fffffffLL ||
      (long long)((Nk + fa::kBwdKeyRows - 1) / fa::kBwdKeyRows) * B * Hkv > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: grid too large");
  // outputs and the workspace may overlap nothing else
  const void* ins[6] = {q, k, v, o, lse, dout};
  const size_t in_b[6] = {qb, kb, kb, qb, lb, qb};
  void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_b[4] = {qb, kb, kb, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], out_b[i], ins[j], in_b[j]))
        return fail(FA_ERR_INVALID_ARG, "fa_bwd: an output or the workspace overlaps an input");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], out_b[i], outs[j], out_b[j]))
        return fail(FA_ERR_INVALID_ARG, "fa_bwd: two outputs (or an output and the workspace) overlap");
  }
  st = check_device();
  if (st != FA_OK) return st;
  fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, Hq, Hkv, Nq, Nk, d,
                scale, causal, dtype};
  hipError_t e = fa::launch_bwd(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_bwd launch: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // extern "C"
