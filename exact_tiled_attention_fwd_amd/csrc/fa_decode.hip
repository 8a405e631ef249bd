// fa_decode.hip - one query token per sequence against its KV cache (gfx950).
//
// Decode reads every cached K/V row once and does little arithmetic per byte,
// so its time is set by memory traffic ("Advanced techniques for enhancing LLM
// throughput", cabseo.com, "Autoregressive and memory-bound operations"). The
// keys of each (sequence, kv-head) are cut into chunks; one workgroup streams
// one chunk through LDS and serves all q-heads of the group from that single
// read (grouped-query attention, SDPA page, devhandbook.co.kr, Example 5).
//
// Split kernel: workgroup (b, g, chunk s). Each tile of 128 keys is shared by
// 4 waves, wave w taking keys [32w, 32w+32). The q-heads of group g are the
// columns of the MFMA B operand (up to 32; unused columns are zero). Each wave
// keeps its own running max/sum; the four are merged in LDS at the end and
// the chunk's normalised output and LSE go to the workspace.
// Combine kernel: per (b, h), merge the chunks of sequence b with the LSE form
// of the softmax-merge identity ("The math of Flash Attention", unite.ai).
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;  // keys per tile

template <int DT, int D>
__global__ __launch_bounds__(kThreads, 1) void fa_decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hq, int Hkv,
    int Lcap, int chunk, int n_split, float scale_log2) {
  using T = Tile<D, kRows>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE_BYTES];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = min(max(seqlens[b], 0), Lcap);
  const int k0 = s * chunk;
  if (k0 >= L) return;  // whole workgroup: this chunk holds no cached rows
  const int k1 = min(k0 + chunk, L);
  const int grp = Hq / Hkv;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int col = lane & 31;  // q-head within the group (B-operand column)
  const size_t bg = (size_t)b * Hkv + g;
  const uint16_t* kp = kc + (bg * Lcap + k0) * D;
  const uint16_t* vp = vc + (bg * Lcap + k0) * D;

  u32x4 qop[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    if (col < grp)
      qop[ks] = *reinterpret_cast<const u32x4*>(q + ((size_t)b * Hq + g * grp + col) * D + 16 * ks + 8 * half);
    else
      qop[ks] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 acc_o[T::MT];
#pragma unroll
  for (int mt = 0; mt < T::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const int n = k1 - k0;
  const int n_t = (n + kRows - 1) / kRows;
  TileRegs<D, kRows> regs;
  load_tile<D, kRows>(kp, vp, min(kRows, n), regs);
  store_tile<D, kRows>(smem, regs);
  __syncthreads();

  for (int jt = 0; jt < n_t; ++jt) {
    const int j0 = jt * kRows;
    const bool more = jt + 1 < n_t;
    if (more) {
      const int jn = j0 + kRows;
      load_tile<D, kRows>(kp + (size_t)jn * D, vp + (size_t)jn * D, min(kRows, n - jn), regs);
    }
    const char* st = smem + (jt & 1) * T::STAGE_BYTES;
    const int jw = j0 + 32 * wave;  // first key of this wave's block (chunk-relative)
    if (jw < n) {
      f32x16 s_acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) s_acc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) s_acc = mfma32<DT>(k_operand<D, kRows>(st, wave, ks, lane), qop[ks], s_acc);
      if (jw + 32 > n) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (jw + acc_key(r, half) >= n) s_acc[r] = -__builtin_inff();
      }
      f32x16 s1[1] = {s_acc};
      uint32_t pk1[1][8];
      softmax_step<DT, 1, T::MT>(s1, scale_log2, m_run, l_run, acc_o, pk1);
      const uint32_t* pk = pk1[0];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 bop = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
#pragma unroll
        for (int mt = 0; mt < T::MT; ++mt)
          acc_o[mt] = mfma32<DT>(vt_operand<D, kRows>(st + T::K_BYTES, mt, 2 * wave + u, lane), bop, acc_o[mt]);
      }
    }
    if (more) store_tile<D, kRows>(smem + ((jt + 1) & 1) * T::STAGE_BYTES, regs);
    __syncthreads();
  }

  // ---- merge the 4 waves' partial states in LDS (stage buffers are free now)
  const float l_tot = halves_sum(l_run);
  float* red_o = reinterpret_cast<float*>(smem);             // [4][grp][D]
  float* red_m = red_o + 4 * 32 * D;                          // [4][32]
  float* red_l = red_m + 4 * 32;                              // [4][32]
  if (col < grp) {
#pragma unroll
    for (int mt = 0; mt < T::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * mt + acc_key(r, half);
        red_o[(wave * 32 + col) * D + d] = acc_o[mt][r];
      }
    if (half == 0) {
      red_m[wave * 32 + col] = m_run;
      red_l[wave * 32 + col] = l_tot;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < grp * D; idx += kThreads) {
    const int c = idx / D, d = idx % D;
    float mstar = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) mstar = fmaxf(mstar, red_m[w * 32 + c]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = red_m[w * 32 + c];
      const float f = (mw == -__builtin_inff()) ? 0.f : exp2_fast(mw - mstar);
      lsum += f * red_l[w * 32 + c];
      osum += f * red_o[(w * 32 + c) * D + d];
    }
    const size_t row = ((size_t)b * Hq + g * grp + c) * n_split + s;
    ws_o[row * D + d] = osum / lsum;
    if (d == 0) ws_lse[row] = (mstar + __builtin_log2f(lsum)) * kLn2;
  }
}

// Merge the chunk results of (b, h): LSE = log sum_s exp(LSE_s),
// O = sum_s exp(LSE_s - LSE) O_s. One workgroup of 64 threads per (b, h).
template <int DT, int D>
__global__ __launch_bounds__(64) void fa_decode_combine_kernel(const float* __restrict__ ws_o,
                                                               const float* __restrict__ ws_lse,
                                                               const int32_t* __restrict__ seqlens,
                                                               uint16_t* __restrict__ o, float* __restrict__ lse,
                                                               int Hq, int Lcap, int chunk, int n_split) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int L = min(max(seqlens[b], 0), Lcap);
  const int ns = (L + chunk - 1) / chunk;
  const float* lp = ws_lse + (size_t)bh * n_split;
  const float* op = ws_o + (size_t)bh * n_split * D;
  float mstar = -__builtin_inff();
  for (int s = 0; s < ns; ++s) mstar = fmaxf(mstar, lp[s]);
  float sum = 0.f;
  for (int s = 0; s < ns; ++s) sum += __expf(lp[s] - mstar);
  const float lse_all = (ns > 0) ? mstar + __logf(sum) : -__builtin_inff();
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float wgt = __expf(lp[s] - lse_all);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += wgt * op[(size_t)s * D + threadIdx.x * PER + i];
  }
  uint16_t* orow = o + (size_t)bh * D;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow + threadIdx.x * 2) = pack2<DT>(acc[0], acc[1]);
  } else {
    const uint32_t w = pack2<DT>(acc[0], 0.f);
    orow[threadIdx.x] = (uint16_t)(w & 0xFFFFu);
  }
  if (lse != nullptr && threadIdx.x == 0) lse[bh] = lse_all;
}

template <int DT, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  float* ws_o = reinterpret_cast<float*>(a.workspace);
  float* ws_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + a.ws_lse_offset);
  hipLaunchKernelGGL((fa_decode_split_kernel<DT, D>), dim3(a.n_split, a.Hkv, a.B), dim3(kThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.seqlens, ws_o,
                     ws_lse, a.Hq, a.Hkv, a.Lcap, a.chunk, a.n_split, a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_decode_combine_kernel<DT, D>), dim3(a.B * a.Hq), dim3(64), 0, stream, ws_o, ws_lse,
                     a.seqlens, (uint16_t*)a.o, a.lse, a.Hq, a.Lcap, a.chunk, a.n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == DT_BF16) return a.d == 128 ? launch_decode_t<DT_BF16, 128>(a, stream) : launch_decode_t<DT_BF16, 64>(a, stream);
  return a.d == 128 ? launch_decode_t<DT_FP16, 128>(a, stream) : launch_decode_t<DT_FP16, 64>(a, stream);
}

}  // namespace fa
