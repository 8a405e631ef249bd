// fa_fwd.hip - prefill attention forward for gfx950.
//
// One workgroup (4 waves) owns BM = 128 query rows of one (batch, q-head); each
// wave owns 32 of them. The workgroup walks the key/value tiles of its kv-head
// (an outer loop over query blocks and an inner loop over key/value blocks, as
// in "Implementation details" of "Flash Attention: Revolutionizing Transformer
// Efficiency", unite.ai), streaming each tile HBM -> registers -> LDS with a
// double buffer so the next tile's loads are in flight while the current tile
// is multiplied. Per tile and wave:
//   S^T = K Q^T on the matrix cores (fp32 accumulate),
//   online softmax in base 2 (running max m, running sum l; the merge identity
//   of "The math of Flash Attention" on the same page),
//   O^T += V^T P^T with P rounded to the input type.
// O is divided by l once after the last tile and written once, with the
// natural-log LSE. Causal key tiles entirely above the diagonal are never
// loaded (SDPA page, devhandbook.co.kr, Example 3, is_causal).
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kThreads = 256; // 4 waves

// Work item of a workgroup: (b, kv-head g, q-head h, query tile qt).
struct Work {
  int b, g, h, qt;
};

// Heavy query tiles first (causal: later tiles see more keys), and when the
// (batch, kv-head) pairs divide evenly over the 8 XCDs, each XCD's share of
// workgroup ids maps to a fixed set of kv-heads so their K/V stay in that
// XCD's L2. Workgroup id L runs on XCD L % 8.
__device__ inline Work map_work(int L, int B, int Hq, int Hkv, int n_qt) {
  const int grp = Hq / Hkv;
  const int nbg = B * Hkv;
  int qt, bg, hh;
  if ((nbg & 7) == 0) {
    const int x = L & 7, s = L >> 3;
    const int nbx = nbg >> 3;
    const int per = nbx * grp;
    qt = n_qt - 1 - s / per;
    const int r = s % per;
    bg = x * nbx + r / grp;
    hh = r % grp;
  } else {
    const int per = nbg * grp;
    qt = n_qt - 1 - L / per;
    const int r = L % per;
    bg = r / grp;
    hh = r % grp;
  }
  Work w;
  w.b = bg / Hkv;
  w.g = bg % Hkv;
  w.h = w.g * grp + hh;
  w.qt = qt;
  return w;
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int Nq, int Nk,
    float scale_log2, int n_qt) {
  constexpr int ROWS = 8192 / D;  // keys per tile: 64 (d=128) or 128 (d=64)
  using T = Tile<D, ROWS>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE_BYTES];

  const Work wk = map_work(blockIdx.x, B, Hq, Hkv, n_qt);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int q0 = wk.qt * kBM;
  const int q0w = q0 + 32 * wave;  // first query row of this wave
  const int off = Nk - Nq;         // causal: key j visible to query i iff j <= i + off

  const size_t bh = (size_t)wk.b * Hq + wk.h;
  const size_t bg = (size_t)wk.b * Hkv + wk.g;
  const uint16_t* qp = q + bh * Nq * D;
  const uint16_t* kp = k + bg * Nk * D;
  const uint16_t* vp = v + bg * Nk * D;

  // Key tiles this workgroup visits.
  int n_kv = (Nk + ROWS - 1) / ROWS;
  if (CAUSAL) {
    const int last_key = min(q0 + kBM, Nq) - 1 + off;
    n_kv = min(n_kv, last_key / ROWS + 1);
  }
  // Key tiles this wave computes on.
  const bool wave_active = q0w < Nq;
  int wave_tiles = n_kv;
  if (CAUSAL && wave_active) wave_tiles = min(n_kv, (min(q0w + 31, Nq - 1) + off) / ROWS + 1);

  // Q^T operand (B operand of S^T = K Q^T), held for the whole loop.
  const int qrow = q0w + (lane & 31);
  u32x4 qop[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    if (wave_active && qrow < Nq)
      qop[ks] = *reinterpret_cast<const u32x4*>(qp + (size_t)qrow * D + 16 * ks + 8 * half);
    else
      qop[ks] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 acc_o[T::MT];
#pragma unroll
  for (int mt = 0; mt < T::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;
  float m_run = -__builtin_inff();  // running max of scaled scores, log2 units
  float l_run = 0.f;                // this lane's share of the running sum

  TileRegs<D, ROWS> regs;
  load_tile<D, ROWS>(kp, vp, min(ROWS, Nk), regs);
  store_tile<D, ROWS>(smem, regs);
  __syncthreads();

  for (int jt = 0; jt < n_kv; ++jt) {
    const int j0 = jt * ROWS;
    const bool more = jt + 1 < n_kv;
    if (more) {
      const int jn = j0 + ROWS;
      load_tile<D, ROWS>(kp + (size_t)jn * D, vp + (size_t)jn * D, min(ROWS, Nk - jn), regs);
    }
    const char* st = smem + (jt & 1) * T::STAGE_BYTES;

    if (wave_active && jt < wave_tiles) {
      // ---- S^T = K Q^T (the two 32-key blocks interleaved: independent chains)
      f32x16 s[T::KB];
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) s[kb] = mfma32<DT>(k_operand<D, ROWS>(st, kb, ks, lane), qop[ks], s[kb]);
      // ---- mask: ragged key tail, causal diagonal
      const bool need_mask = (j0 + ROWS > Nk) || (CAUSAL && j0 + ROWS - 1 > q0w + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(Nk, qrow + off + 1) : Nk;  // keys < lim are visible
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (j0 + 32 * kb + acc_key(r, half) >= lim) s[kb][r] = -__builtin_inff();
      }
      // ---- online softmax (base 2)
      uint32_t pk[T::KB][8];
      softmax_step<DT, T::KB, T::MT>(s, scale_log2, m_run, l_run, acc_o, pk);
      // ---- O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 b = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
#pragma unroll
          for (int mt = 0; mt < T::MT; ++mt)
            acc_o[mt] = mfma32<DT>(vt_operand<D, ROWS>(st, mt, 2 * kb + u, lane), b, acc_o[mt]);
        }
    }

    if (more) store_tile<D, ROWS>(smem + ((jt + 1) & 1) * T::STAGE_BYTES, regs);
    __syncthreads();
  }

  if (!wave_active) return;
  // ---- epilogue: normalise once, write O and LSE
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < Nq) {
    uint16_t* orow = o + bh * Nq * D + (size_t)qrow * D;
#pragma unroll
    for (int mt = 0; mt < T::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * mt + 8 * i + 4 * half;
        const u32x2 w = {pack2<DT>(acc_o[mt][4 * i] * inv, acc_o[mt][4 * i + 1] * inv),
                         pack2<DT>(acc_o[mt][4 * i + 2] * inv, acc_o[mt][4 * i + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (lse != nullptr && half == 0)
      lse[bh * Nq + qrow] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
  }
}

template <int DT, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long long nblocks = (long long)n_qt * a.B * a.Hq;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_fwd_kernel<DT, D, CAUSAL>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const bool c = a.causal != 0;
  if (a.dtype == DT_BF16) {
    if (a.d == 128) return c ? launch_fwd_t<DT_BF16, 128, true>(a, stream) : launch_fwd_t<DT_BF16, 128, false>(a, stream);
    return c ? launch_fwd_t<DT_BF16, 64, true>(a, stream) : launch_fwd_t<DT_BF16, 64, false>(a, stream);
  }
  if (a.d == 128) return c ? launch_fwd_t<DT_FP16, 128, true>(a, stream) : launch_fwd_t<DT_FP16, 128, false>(a, stream);
  return c ? launch_fwd_t<DT_FP16, 64, true>(a, stream) : launch_fwd_t<DT_FP16, 64, false>(a, stream);
}

}  // namespace fa
