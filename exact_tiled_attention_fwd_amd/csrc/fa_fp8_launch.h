// fa_fp8_launch.h - internal interface between the C ABI (fa_api.cpp) and the
// FP8 prefill kernel (fa_fwd_fp8.hip). Not installed; callers use include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// q [B, Hq, Nq, 128], k, v [B, Hkv, Nk, 128] as OCP E4M3 bytes; o [B, Hq, Nq,
// 128] bf16; lse [B, Hq, Nq] fp32 or null; descales fp32 [B, Hq] (q) and
// [B, Hkv] (k, v): element x of a (b, head) slab stands for x * descale.
struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  void* o;
  float* lse;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  int B, Hq, Hkv, Nq, Nk;
  float scale;
  int causal;
};

constexpr int kFp8BlockRows = 256;  // query rows per FP8 workgroup

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);

}  // namespace fa
