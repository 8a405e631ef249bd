// fa_fwd_fp8.hip - prefill attention forward with 8-bit float inputs (OCP E4M3)
// for gfx950, head width 128.
//
// The FP8 computation that "Flash Attention: Revolutionizing Transformer
// Efficiency" (unite.ai) lists for FlashAttention-3 (that section, point 2),
// on the CDNA4 matrix cores: both products run on
// v_mfma_f32_32x32x64_f8f6f4 (E4M3 operands, fp32 accumulation), at twice the
// 16-bit rate. The page gives no scaling method, so each (batch, head) slab of
// q, k, v carries one fp32 descale: element x stands for x * descale. The
// score scale folds the q and k descales in; the v descale is applied once in
// the epilogue.
//
// Structure: one workgroup of 8 waves owns 256 query rows of one (b, q-head)
// (32 rows per wave) and walks 64-key tiles of its kv-head. As in the 16-bit
// kernels, two groups of 4 waves alternate on the same SIMDs, one issuing
// matrix-core work while the other runs its softmax; group 0 stages V and
// group 1 stages K through registers into 2-slot LDS rings:
//   S^T = K Q^T             A = K rows from LDS, B = Q^T held in registers
//   online softmax          p = 2^(s c - m + 4) against the running
//                           reference m; the row maximum is taken only on a
//                           row's first tile or when some lane's sum exceeds
//                           448 (E4M3's largest value, which then bounds
//                           every p); the 2^4 keeps small values normal and
//                           cancels against the running sum
//   O^T += V^T P^T          A = V^T from LDS, B = P rounded to E4M3 (RNE)
// V is transposed on its way into LDS (4x4 byte blocks, v_perm_b32), with the
// keys of each row stored in the order a lane holds its 32 P values, so every
// operand is two 16-byte LDS reads and no lane exchanges are needed.
#include <type_traits>

#include "fa_fp8_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;                 // 8 waves = 2 groups of 4
constexpr int kBM = kFp8BlockRows;            // 256 query rows
constexpr int kD = 128;                       // head width (bytes per row in fp8)
constexpr int kRows = 64;                     // keys per tile
constexpr int kKStride = kD;                  // K tile row: 128 bytes
constexpr int kVtStride = kRows + 16;         // V^T tile row: 64 keys + 16 bytes of padding
constexpr int kKBytes = kRows * kKStride;     // 8 KiB
constexpr int kVtBytes = kD * kVtStride;      // 10 KiB
constexpr int kStage = kKBytes + kVtBytes;
constexpr float kPOffset = 4.f;               // P is scaled by 2^4 before rounding
constexpr float kSumLimit8 = 448.f;           // largest finite E4M3 value

__device__ inline f32x16 mfma_f8(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ inline i32x8 cat(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// K tile: row r, 16-byte chunk c (0..7) stored at chunk position c ^ (r & 7).
__device__ inline int kpos(int r, int c) { return c ^ (r & 7); }

// Position of key k (0..63) in a V^T row. A lane in half h holds, in its P
// accumulator registers r of key block kb, keys 32 kb + 8 (r/4) + 4 h + r%4;
// packed in register order those are bytes 16 kb + r of the lane's operand,
// and V^T stores key k at 32 h + that byte index.
__device__ inline int vt_pos(int k) {
  return 32 * ((k >> 2) & 1) + 16 * (k >> 5) + 4 * ((k >> 3) & 3) + (k & 3);
}

// A operand of S^T = K Q^T: key 32 kb + lane % 32, head-dim bytes 64 ks + 32 h .. +31.
__device__ inline i32x8 k_op(const char* __restrict__ kl, int kb, int ks, int lane) {
  const int r = 32 * kb + (lane & 31), c = 4 * ks + 2 * (lane >> 5);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(kl + r * kKStride + kpos(r, c) * 16);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(kl + r * kKStride + kpos(r, c + 1) * 16);
  return cat(lo, hi);
}

// A operand of O^T += V^T P^T: head-dim row 32 mt + lane % 32, key bytes 32 h .. +31.
__device__ inline i32x8 vt_op(const char* __restrict__ vl, int mt, int lane) {
  const char* p = vl + (32 * mt + (lane & 31)) * kVtStride + 32 * (lane >> 5);
  return cat(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
}

// 4x4 byte transpose: rows a, b, c, d (4 bytes each) -> columns.
__device__ inline void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t (&out)[4]) {
  const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  out[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);        // a0 b0 c0 d0
  out[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);        // a1 b1 c1 d1
  out[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

// Global -> register staging of one tile by the 256 threads of one group
// (t = thread index in the group). Rows at or beyond nvalid re-read row
// nvalid - 1; their scores are masked. K: two 16-byte chunks per thread.
// V: two blocks of 4 keys x 4 bytes per thread (for each key row a wave
// covers 128 contiguous bytes of 2 rows per load).
__device__ inline void load_k8(const uint8_t* __restrict__ kb, int nvalid, int t, u32x4 (&r)[2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = t + 256 * p;
    const int row = min(idx >> 3, nvalid - 1), c = idx & 7;
    r[p] = *reinterpret_cast<const u32x4*>(kb + (size_t)row * kD + 16 * c);
  }
}
__device__ inline void store_k8(char* __restrict__ kl, int t, const u32x4 (&r)[2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = t + 256 * p;
    const int row = idx >> 3, c = idx & 7;
    *reinterpret_cast<u32x4*>(kl + row * kKStride + kpos(row, c) * 16) = r[p];
  }
}
__device__ inline void load_v8(const uint8_t* __restrict__ vb, int nvalid, int t, uint32_t (&r)[2][4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = t + 256 * p;
    const int dq = idx & 31, kq = idx >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = min(4 * kq + i, nvalid - 1);
      r[p][i] = *reinterpret_cast<const uint32_t*>(vb + (size_t)vr * kD + 4 * dq);
    }
  }
}
__device__ inline void store_v8(char* __restrict__ vl, int t, const uint32_t (&r)[2][4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = t + 256 * p;
    const int dq = idx & 31, kq = idx >> 5;
    uint32_t cols[4];
    transpose4(r[p][0], r[p][1], r[p][2], r[p][3], cols);
    const int pos = vt_pos(4 * kq);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(vl + (4 * dq + j) * kVtStride + pos) = cols[j];
  }
}

// Exponentials of one tile against reference m (log2 units): p = 2^(s c -
// m + kPOffset), packed four per register as E4M3 in the order of vt_pos.
// Returns this lane's sum of the unrounded values.
__device__ __attribute__((always_inline)) inline float exp_pack8(const f32x16 (&s)[2], float c, float m,
                                                                  uint32_t (&pk)[8]) {
  const float sub = m - kPOffset;
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * mm + i], c, -sub));
        psum += p[i];
      }
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      pk[4 * kb + mm] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
    }
  return psum;
}

// Online softmax step of one tile. The tile is first exponentiated against
// the current reference m_run; every value is at most its lane's sum, so if
// every lane's sum is at most kSumLimit the values fit E4M3 and are kept.
// Otherwise (or on a row's first tile) the tile's row maximum is taken, m_run
// moves to it, the running sum and accumulator are rescaled, and the tile is
// exponentiated again (then every value is at most 2^kPOffset).
__device__ __attribute__((always_inline)) inline void softmax8(const f32x16 (&s)[2], float c, float& m_run,
                                                                float& l_run, f32x16 (&acc_o)[4], uint32_t (&pk)[8]) {
  float psum = 0.f;
  bool slow = __builtin_amdgcn_ballot_w64(m_run == -__builtin_inff()) != 0;
  if (!slow) {
    psum = exp_pack8(s, c, m_run, pk);
    slow = __builtin_amdgcn_ballot_w64(!(psum <= kSumLimit8)) != 0;
  }
  if (slow) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    const float m_new = fmaxf(m_run, halves_max(mx) * c);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;
    m_run = m_new;
    psum = exp_pack8(s, c, m_use, pk);
  }
  l_run += psum;
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, const float* __restrict__ q_ds,
    const float* __restrict__ k_ds, const float* __restrict__ v_ds, int B, int Hq, int Hkv, int Nq, int Nk,
    float scale_log2, int n_qt) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kKBytes + 2 * kVtBytes];
  char* const kring = smem;                // K tile t in slot t & 1
  char* const vring = smem + 2 * kKBytes;  // V^T tile t in slot t & 1
  const Work wk = map_work(blockIdx.x, B, Hq, Hkv, n_qt);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int grp = wave >> 2;           // 0: matrix cores first, stages V; 1: softmax first, stages K
  const int gtid = threadIdx.x & 255;  // thread index within the group
  const int q0 = wk.qt * kBM;
  const int q0w = q0 + 32 * wave;
  const int qrow = q0w + (lane & 31);
  const int off = Nk - Nq;
  const size_t bh = (size_t)wk.b * Hq + wk.h, bg = (size_t)wk.b * Hkv + wk.g;
  const uint8_t* qp = q + bh * Nq * kD;
  const uint8_t* kp = k + bg * Nk * kD;
  const uint8_t* vp = v + bg * Nk * kD;
  // scores in log2 units: raw dot product times scale * log2(e) * q and k descales
  const float c = scale_log2 * q_ds[bh] * k_ds[bg];
  const float vd = v_ds[bg];

  // key tiles this workgroup visits, and those this wave computes on
  int n_kv = (Nk + kRows - 1) / kRows;
  if (CAUSAL) {
    const int last_key = min(q0 + kBM, Nq) - 1 + off;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kRows + 1);
  }
  const bool wave_active = q0w < Nq;
  int wt = wave_active ? n_kv : 0;
  if (CAUSAL && wave_active) {
    const int last = min(q0w + 31, Nq - 1) + off;
    wt = last < 0 ? 0 : min(n_kv, last / kRows + 1);
  }

  // Q^T operand: row qrow, head-dim bytes 64 ks + 32 h .. +31.
  const int qr = min(qrow, Nq - 1);
  i32x8 qop[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const uint8_t* p = qp + (size_t)qr * kD + 64 * ks + 32 * half;
    qop[ks] = cat(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
  }

  f32x16 acc_o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;
  float m_run = -__builtin_inff();  // running reference, log2 units
  float l_run = 0.f;                // this lane's share of the running sum
  f32x16 s[2];                      // S^T of the tile last multiplied
  uint32_t pk[8];                   // P of the tile last softmaxed (E4M3)

  auto softmax = [&](int j) {
    const int j0 = j * kRows;
    const bool need_mask = (j0 + kRows > Nk) || (CAUSAL && j0 + kRows - 1 > q0w + off);
    if (need_mask) {
      const int lim = CAUSAL ? min(Nk, qrow + off + 1) : Nk;  // keys < lim are visible
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j0 + 32 * kb + acc_key(r, half) >= lim) s[kb][r] = -__builtin_inff();
    }
    softmax8(s, c, m_run, l_run, acc_o, pk);
  };
  // Matrix-core phase: O^T += V^T_jo P^T (DO_O) and S^T = K_js Q^T (DO_S),
  // interleaved. All A operands of the phase are read from LDS first, so the
  // MFMAs wait for the reads once instead of each in turn.
  auto mma_t = [&](auto do_o_t, auto do_s_t, int jo, int js) {
    constexpr bool DO_O = decltype(do_o_t)::value, DO_S = decltype(do_s_t)::value;
    const char* vl = vring + (jo & 1) * kVtBytes;
    const char* kl = kring + (js & 1) * kKBytes;
    i32x8 ao[4], as[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (DO_O) ao[t] = vt_op(vl, t, lane);
      if constexpr (DO_S) as[t] = k_op(kl, t & 1, t >> 1, lane);
    }
    const i32x8 bp = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
    if constexpr (DO_S) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (DO_O) acc_o[t] = mfma_f8(ao[t], bp, acc_o[t]);
      if constexpr (DO_S) s[t & 1] = mfma_f8(as[t], qop[t >> 1], s[t & 1]);
    }
  };
  auto mma = [&](bool do_o, int jo, bool do_s, int js) {
    if (do_o && do_s)
      mma_t(std::true_type{}, std::true_type{}, jo, js);
    else if (do_o)
      mma_t(std::true_type{}, std::false_type{}, jo, js);
    else if (do_s)
      mma_t(std::false_type{}, std::true_type{}, jo, js);
  };
  auto tile_rows = [&](int j) { return min(kRows, Nk - j * kRows); };

  // Each group runs its own loop (both pass the same barriers):
  //   group 0: A = store V_i, load V_{i+1}, O(i-1), S(i)   B = softmax(i)
  //   group 1: A = load K_{i+1}, softmax(i-1)              B = O(i-1), S(i), store K_{i+1}
  // V_i / K_i live in ring slot i & 1; a slot is rewritten only after the
  // barrier that ends the last phase reading its previous tile.
  if (grp == 0) {
    uint32_t rv[2][4];
    if (n_kv > 0) {
      load_v8(vp, tile_rows(0), gtid, rv);
      store_v8(vring, gtid, rv);
      if (n_kv > 1) load_v8(vp + (size_t)kRows * kD, tile_rows(1), gtid, rv);
    }
    __syncthreads();
    for (int i = 0; i <= n_kv; ++i) {
      if (i >= 1 && i < n_kv) {
        store_v8(vring + (i & 1) * kVtBytes, gtid, rv);
        if (i + 1 < n_kv) load_v8(vp + (size_t)(i + 1) * kRows * kD, tile_rows(i + 1), gtid, rv);
      }
      mma(i >= 1 && i - 1 < wt, i - 1, i < wt, i);
      __syncthreads();
      if (i < wt) softmax(i);
      __syncthreads();
    }
  } else {
    u32x4 rk[2];
    if (n_kv > 0) {
      load_k8(kp, tile_rows(0), gtid, rk);
      store_k8(kring, gtid, rk);
    }
    __syncthreads();
    for (int i = 0; i <= n_kv; ++i) {
      if (i + 1 < n_kv) load_k8(kp + (size_t)(i + 1) * kRows * kD, tile_rows(i + 1), gtid, rk);
      if (i >= 1 && i - 1 < wt) softmax(i - 1);
      __syncthreads();
      mma(i >= 1 && i - 1 < wt, i - 1, i < wt, i);
      if (i + 1 < n_kv) store_k8(kring + ((i + 1) & 1) * kKBytes, gtid, rk);
      __syncthreads();
    }
  }

  if (!wave_active || qrow >= Nq) return;
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? vd / l_tot : 0.f;
  uint16_t* orow = o + (bh * Nq + qrow) * kD;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * mt + 8 * i + 4 * half;
      const u32x2 w = {pack2<DT_BF16>(acc_o[mt][4 * i] * inv, acc_o[mt][4 * i + 1] * inv),
                       pack2<DT_BF16>(acc_o[mt][4 * i + 2] * inv, acc_o[mt][4 * i + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d0) = w;
    }
  if (lse != nullptr && half == 0)
    lse[bh * Nq + qrow] = l_tot > 0.f ? (m_run - kPOffset + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
}

template <bool CAUSAL>
hipError_t launch_t(const Fp8Args& a, hipStream_t stream) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long long nblocks = (long long)n_qt * a.B * a.Hq;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<CAUSAL>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream, a.q, a.k, a.v,
                     (uint16_t*)a.o, a.lse, a.q_descale, a.k_descale, a.v_descale, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                     a.scale * kLog2e, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
  return a.causal ? launch_t<true>(a, stream) : launch_t<false>(a, stream);
}

}  // namespace fa
