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
// Structure: one workgroup of 4 waves owns 128 query rows of one (b, q-head)
// (32 rows per wave) and walks 64-key tiles of its kv-head, double-buffered in
// LDS through registers (one barrier per tile):
//   S^T = K Q^T             A = K rows from LDS, B = Q^T held in registers
//   online softmax          the tile's row maximum is taken every tile, and
//                           P is formed as exp2(s c - m + 8): every value lies
//                           in (0, 256], inside E4M3's range, and small ones
//                           keep normal precision; the 2^8 cancels against the
//                           running sum, which accumulates the same values
//   O^T += V^T P^T          A = V^T from LDS, B = P rounded to E4M3 (RNE)
// V is transposed on its way into LDS (4x4 byte blocks, v_perm_b32), with the
// keys of each row stored in the order a lane holds its 32 P values, so every
// operand is two 16-byte LDS reads and no lane exchanges are needed.
#include "fa_fp8_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;                 // 4 waves
constexpr int kBM = kFp8BlockRows;            // 128 query rows
constexpr int kD = 128;                       // head width (bytes per row in fp8)
constexpr int kRows = 64;                     // keys per tile
constexpr int kKStride = kD;                  // K tile row: 128 bytes
constexpr int kVtStride = kRows + 16;         // V^T tile row: 64 keys + 16 bytes of padding
constexpr int kKBytes = kRows * kKStride;     // 8 KiB
constexpr int kVtBytes = kD * kVtStride;      // 10 KiB
constexpr int kStage = kKBytes + kVtBytes;
constexpr float kPOffset = 8.f;               // P is scaled by 2^8 before rounding

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

// Global -> register staging of one tile (rows at or beyond nvalid re-read
// row nvalid - 1; their scores are masked). K: two 16-byte chunks per thread.
// V: two 4-key x 4-byte blocks per thread (a wave covers 128 contiguous bytes
// of 2 x 4 key rows per load).
struct TileRegs8 {
  u32x4 k[2];
  uint32_t v[2][4];
};

__device__ inline void load_tile8(const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb, int nvalid,
                                  TileRegs8& t) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = threadIdx.x + kThreads * p;
    const int row = min(idx >> 3, nvalid - 1), c = idx & 7;
    t.k[p] = *reinterpret_cast<const u32x4*>(kb + (size_t)row * kD + 16 * c);
    const int dq = idx & 31, kq = idx >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = min(4 * kq + i, nvalid - 1);
      t.v[p][i] = *reinterpret_cast<const uint32_t*>(vb + (size_t)vr * kD + 4 * dq);
    }
  }
}

__device__ inline void store_tile8(char* __restrict__ st, const TileRegs8& t) {
  char* kl = st;
  char* vl = st + kKBytes;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = threadIdx.x + kThreads * p;
    const int row = idx >> 3, c = idx & 7;
    *reinterpret_cast<u32x4*>(kl + row * kKStride + kpos(row, c) * 16) = t.k[p];
    const int dq = idx & 31, kq = idx >> 5;
    uint32_t cols[4];
    transpose4(t.v[p][0], t.v[p][1], t.v[p][2], t.v[p][3], cols);
    const int pos = vt_pos(4 * kq);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(vl + (4 * dq + j) * kVtStride + pos) = cols[j];
  }
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, const float* __restrict__ q_ds,
    const float* __restrict__ k_ds, const float* __restrict__ v_ds, int B, int Hq, int Hkv, int Nq, int Nk,
    float scale_log2, int n_qt) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  const Work wk = map_work(blockIdx.x, B, Hq, Hkv, n_qt);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
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

  int n_kv = (Nk + kRows - 1) / kRows;
  if (CAUSAL) {
    const int last_key = min(q0 + kBM, Nq) - 1 + off;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kRows + 1);
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
  float m_run = -__builtin_inff();  // running row maximum, log2 units
  float l_run = 0.f;                // this lane's share of the running sum of 2^8 P

  TileRegs8 tr;
  if (n_kv > 0) {
    load_tile8(kp, vp, min(kRows, Nk), tr);
    store_tile8(smem, tr);
  }
  __syncthreads();
  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv)
      load_tile8(kp + (size_t)(j + 1) * kRows * kD, vp + (size_t)(j + 1) * kRows * kD, min(kRows, Nk - (j + 1) * kRows),
                 tr);
    const char* kl = smem + (j & 1) * kStage;
    const char* vl = kl + kKBytes;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_f8(k_op(kl, kb, ks, lane), qop[ks], s[kb]);

    // mask the ragged tail and the causal diagonal
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
    // online softmax with the tile's row maximum
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = halves_max(mx) * c;
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;
    }
    m_run = m_new;
    const float sub = m_use - kPOffset;
    uint32_t pk[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * mm + i], c, -sub));
          l_run += p[i];
        }
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        pk[4 * kb + mm] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
      }
    const i32x8 bp = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc_o[mt] = mfma_f8(vt_op(vl, mt, lane), bp, acc_o[mt]);

    if (j + 1 < n_kv) store_tile8(smem + ((j + 1) & 1) * kStage, tr);
    __syncthreads();
  }

  if (qrow >= Nq) return;
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
