// fa_bwd_launch.h - internal interface between the C ABI (fa_api.cpp) and the
// backward kernels (fa_bwd.hip). Not installed; callers use include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Contiguous layouts: q, o, dout, dq [B, Hq, Nq, d]; k, v, dk, dv
// [B, Hkv, Nk, d]; lse [B, Hq, Nq] fp32 (natural log, from the forward);
// delta [B, Hq, Nq] fp32 scratch (row sums of dout * o).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int dtype;
};

constexpr int kBwdKeyRows = 128;    // keys per dK/dV workgroup
constexpr int kBwdQueryRows = 128;  // query rows per dQ workgroup

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace fa
