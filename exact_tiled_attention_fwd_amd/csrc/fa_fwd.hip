// fa_fwd.hip - prefill attention forward for gfx950.
//
// One workgroup owns BM = 256 query rows of one (batch, q-head): 8 waves of 32
// rows each, in two groups of 4. The workgroup walks the key/value tiles of
// its kv-head (an outer loop over query blocks and an inner loop over
// key/value blocks, as in "Implementation details" of "Flash Attention:
// Revolutionizing Transformer Efficiency", unite.ai). Per tile and wave:
//   MA: S^T = K Q^T on the matrix cores (fp32 accumulate),
//   SM: online softmax in base 2 (running max m, running sum l; the merge
//       identity of "The math of Flash Attention" on the same page),
//   MB: O^T += V^T P^T with P rounded to the input type.
// The two groups run out of phase: while one group's waves issue matrix-core
// work (MB of the previous tile and MA of the current one), the other group's
// waves, which share the same SIMDs, run their softmax on the vector ALUs.
// Each phase ends at a workgroup barrier. Group 0 streams the V tiles and
// group 1 the K tiles HBM -> registers -> LDS, one tile ahead, into a 2-deep
// ring for each. O is divided by l once after the last tile and written
// once, with the natural-log LSE. Causal key tiles entirely above the
// diagonal are never loaded (SDPA page, devhandbook.co.kr, Example 3).
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

constexpr int kBM = kFwdBlockRows;  // query rows per workgroup
constexpr int kThreads = 512;  // 8 waves = 2 groups of 4

template <int DT, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int Nq_all, int Nk_all,
    float scale_log2, int n_qt, Varlen vlen, Layout ly) {
  constexpr int ROWS = 8192 / D;  // keys per tile: 64 (d=128) or 128 (d=64)
  using T = Tile<D, ROWS>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::K_BYTES + 2 * T::VT_BYTES];
  char* const kring = smem;                    // K tiles, slot = tile & 1
  char* const vring = smem + 2 * T::K_BYTES;   // V^T tiles, slot = tile & 1

  const Work wk = VARLEN ? map_work_packed(blockIdx.x, B, Hq, Hkv, n_qt) : map_work(blockIdx.x, B, Hq, Hkv, n_qt);
  const Slabs sl = slabs_of<VARLEN>(wk, q, k, v, o, lse, Hq, Nq_all, Nk_all, vlen, ly);
  const int Nq = sl.Nq, Nk = sl.Nk;
  const int q0 = wk.qt * kBM;
  if (VARLEN && q0 >= Nq) return;  // past this sequence's rows (the whole workgroup)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int grp = wave >> 2;                // 0: V loader, MFMA first; 1: K loader
  const int gtid = threadIdx.x & 255;       // thread index within the group
  const int q0w = q0 + 32 * wave;  // first query row of this wave
  const int off = Nk - Nq;         // causal: key j visible to query i iff j <= i + off

  const uint16_t* qp = sl.q;
  const uint16_t* kp = sl.k;
  const uint16_t* vp = sl.v;

  // Key tiles this workgroup visits.
  int n_kv = (Nk + ROWS - 1) / ROWS;
  if (CAUSAL) {
    const int last_key = min(q0 + kBM, Nq) - 1 + off;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / ROWS + 1);
  }
  // Key tiles this wave computes on (0 if the wave has no valid query row).
  const bool wave_active = q0w < Nq;
  int wave_tiles = wave_active ? n_kv : 0;
  if (CAUSAL && wave_active) {
    const int last = min(q0w + 31, Nq - 1) + off;
    wave_tiles = last < 0 ? 0 : min(n_kv, last / ROWS + 1);
  }

  // Q^T operand (B operand of S^T = K Q^T), held for the whole loop.
  const int qrow = q0w + (lane & 31);
  u32x4 qop[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    if (qrow < Nq)
      qop[ks] = *reinterpret_cast<const u32x4*>(qp + (size_t)qrow * sl.qs + 16 * ks + 8 * half);
    else
      qop[ks] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 acc_o[T::MT];
#pragma unroll
  for (int mt = 0; mt < T::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;
  float m_run = -__builtin_inff();  // row reference point, log2 units
  float l_run = 0.f;                // this lane's share of the running sum
  f32x16 s[T::KB];                  // S^T of the tile last multiplied
  uint32_t pk[T::KB][8];            // P of the tile last softmaxed

  // SM(j): mask the ragged key tail / causal diagonal, online softmax -> pk.
  auto softmax = [&](int j) {
    const int j0 = j * ROWS;
    const bool need_mask = (j0 + ROWS > Nk) || (CAUSAL && j0 + ROWS - 1 > q0w + off);
    if (need_mask) {
      const int lim = CAUSAL ? min(Nk, qrow + off + 1) : Nk;  // keys < lim are visible
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j0 + 32 * kb + acc_key(r, half) >= lim) s[kb][r] = -__builtin_inff();
    }
    softmax_step<DT, T::KB, T::MT>(s, scale_log2, m_run, l_run, acc_o, pk);
  };
  // Matrix-core phase: MB(jo) = O^T += V^T_jo P^T (if do_o), MA(js) = S^T = K_js Q^T (if do_s).
  // mma_pre issues the first operand reads; mma finishes the phase.
  u32x4 obuf[kPF];
  auto mma_pre = [&](bool do_o, int jo, bool do_s, int js) {
    const char* vl = vring + (jo & 1) * T::VT_BYTES;
    const char* kl = kring + (js & 1) * T::K_BYTES;
    if (do_o && do_s)
      mma_prefetch<D, ROWS, true, true>(obuf, vl, kl, lane);
    else if (do_o)
      mma_prefetch<D, ROWS, true, false>(obuf, vl, kl, lane);
    else if (do_s)
      mma_prefetch<D, ROWS, false, true>(obuf, vl, kl, lane);
  };
  auto mma = [&](bool do_o, int jo, bool do_s, int js) {
    const char* vl = vring + (jo & 1) * T::VT_BYTES;
    const char* kl = kring + (js & 1) * T::K_BYTES;
    if (do_o && do_s)
      mma_run<DT, D, ROWS, true, true>(obuf, vl, kl, pk, qop, acc_o, s, lane);
    else if (do_o)
      mma_run<DT, D, ROWS, true, false>(obuf, vl, kl, pk, qop, acc_o, s, lane);
    else if (do_s)
      mma_run<DT, D, ROWS, false, true>(obuf, vl, kl, pk, qop, acc_o, s, lane);
  };
  auto tile_rows = [&](int j) { return min(ROWS, Nk - j * ROWS); };

  // Each group runs its own loop (both execute the same number of barriers):
  // macro-step i is phase A then phase B, each closed by a barrier.
  //   group 0: A = store V_i, load V_{i+1}, MB(i-1), MA(i)   B = SM(i)
  //   group 1: A = load K_{i+1}, SM(i-1)                     B = MB(i-1), MA(i), store K_{i+1}
  // V_i / K_i live in ring slot i & 1; a slot is rewritten only after the
  // barrier that ends the last phase reading its previous tile.
  if (grp == 0) {
    u32x4 rv[T::U][4];
    load_v<D, ROWS>(vp, sl.vs, tile_rows(0), gtid, rv);
    store_v<D, ROWS>(vring, gtid, rv);
    if (n_kv > 1) load_v<D, ROWS>(vp + (size_t)ROWS * sl.vs, sl.vs, tile_rows(1), gtid, rv);
    __syncthreads();
    mma_pre(false, -1, 0 < wave_tiles, 0);
    for (int i = 0; i <= n_kv; ++i) {
      if (i >= 1 && i < n_kv) {
        store_v<D, ROWS>(vring + (i & 1) * T::VT_BYTES, gtid, rv);
        if (i + 1 < n_kv) load_v<D, ROWS>(vp + (size_t)(i + 1) * ROWS * sl.vs, sl.vs, tile_rows(i + 1), gtid, rv);
      }
      mma(i >= 1 && i - 1 < wave_tiles, i - 1, i < wave_tiles, i);
      __syncthreads();
      if (i < wave_tiles) softmax(i);
      // V_i (stored in phase A) is complete: start the next phase's reads.
      mma_pre(i < wave_tiles, i, i + 1 < wave_tiles, i + 1);
      __syncthreads();
    }
  } else {
    u32x4 rk[TileRegs<D, ROWS>::KU];
    load_k<D, ROWS>(kp, sl.ks, tile_rows(0), gtid, rk);
    store_k<D, ROWS>(kring, gtid, rk);
    __syncthreads();
    for (int i = 0; i <= n_kv; ++i) {
      if (i + 1 < n_kv) load_k<D, ROWS>(kp + (size_t)(i + 1) * ROWS * sl.ks, sl.ks, tile_rows(i + 1), gtid, rk);
      if (i >= 1 && i - 1 < wave_tiles) softmax(i - 1);
      // V_{i-1} and K_i were completed before the last barrier.
      mma_pre(i >= 1 && i - 1 < wave_tiles, i - 1, i < wave_tiles, i);
      __syncthreads();
      mma(i >= 1 && i - 1 < wave_tiles, i - 1, i < wave_tiles, i);
      if (i + 1 < n_kv) store_k<D, ROWS>(kring + ((i + 1) & 1) * T::K_BYTES, gtid, rk);
      __syncthreads();
    }
  }

  if (!wave_active) return;
  // ---- epilogue: normalise once, write O and LSE
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < Nq) {
    uint16_t* orow = sl.o + (size_t)qrow * sl.os;
#pragma unroll
    for (int mt = 0; mt < T::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * mt + 8 * i + 4 * half;
        const u32x2 w = {pack2<DT>(acc_o[mt][4 * i] * inv, acc_o[mt][4 * i + 1] * inv),
                         pack2<DT>(acc_o[mt][4 * i + 2] * inv, acc_o[mt][4 * i + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (sl.lse != nullptr && half == 0)
      sl.lse[qrow] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
  }
}

template <int DT, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int rows = VARLEN ? a.max_seqlen_q : a.Nq;
  const int n_qt = (rows + kBM - 1) / kBM;
  const long long nblocks = (long long)n_qt * a.B * a.Hq;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (nblocks == 0) return hipSuccess;
  const Varlen vl{a.cu_q, a.cu_k, a.total_q, a.total_k};
  hipLaunchKernelGGL((fa_fwd_kernel<DT, D, CAUSAL, VARLEN>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_qt, vl, a.layout);
  return hipGetLastError();
}

template <int DT, bool CAUSAL>
hipError_t launch_fwd_v(const FwdArgs& a, hipStream_t stream) {
  return a.cu_q != nullptr ? launch_fwd_t<DT, 64, CAUSAL, true>(a, stream)
                           : launch_fwd_t<DT, 64, CAUSAL, false>(a, stream);
}

}  // namespace

// d = 128 runs the direct-to-LDS kernel; d = 64 the register-staged one.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_fwd_d128(a, stream);
  const bool c = a.causal != 0;
  if (a.dtype == DT_BF16) return c ? launch_fwd_v<DT_BF16, true>(a, stream) : launch_fwd_v<DT_BF16, false>(a, stream);
  return c ? launch_fwd_v<DT_FP16, true>(a, stream) : launch_fwd_v<DT_FP16, false>(a, stream);
}

}  // namespace fa
