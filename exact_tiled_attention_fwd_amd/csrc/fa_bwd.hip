// fa_bwd.hip - attention backward (dQ, dK, dV) for gfx950.
//
// The forward stores only O and the row LSE; the backward recomputes the
// probabilities tile by tile from Q, K and that LSE instead of reading a
// stored attention matrix ("Enter Flash Attention", point 2, recomputation,
// in "Flash Attention: Revolutionizing Transformer Efficiency", unite.ai).
// With P = exp(scale Q K^T - LSE) (0 where masked) the gradients of the
// forward definition for an upstream gradient dO are
//   dV = P^T dO,  dP = dO V^T,  delta = rowsum(dO * O),
//   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, in stream order:
//   fa_bwd_delta_kernel  delta = rowsum(dO * O) in fp32, one pass over dO, O;
//   fa_bwd_dkdv_kernel   one workgroup per (b, kv-head, 128 keys): each wave
//                        keeps 32 keys' K and V in registers and dK^T, dV^T
//                        accumulators, and walks the query tiles of every
//                        q-head of its group, tile-major (64 rows of Q, dO,
//                        LSE, delta staged in LDS, double-buffered);
//   fa_bwd_dq_kernel     one workgroup per (b, q-head, 128 query rows): each
//                        wave keeps 32 rows' Q^T, dO^T operands and a dQ^T
//                        accumulator, and walks the key tiles (64 rows of K
//                        and V staged in LDS).
// Neither kernel writes another's output, so no atomics are needed and the
// result is deterministic; dQ pays for that by recomputing S and dP.
//
// All products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation;
// P and dS are rounded to the input type only as MFMA operands. Operand
// orientation keeps every accumulator usable as the next B operand without
// shuffles:
//   dK/dV kernel: S = Q K^T and dP = dO V^T (lane = key column), then
//                 dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read
//                 transposed from LDS (ds_read_b64_tr_b16);
//   dQ kernel:    S^T = K Q^T and dP^T = V dO^T (lane = query column), then
//                 dQ^T += K^T dS^T with K^T read transposed from LDS.
#include "fa_bwd_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = 64;  // rows of a staged Q/dO (dK/dV kernel) or K/V (dQ kernel) tile

// LDS tiles are row-major [64][D] 16-bit with 16-byte chunks XOR-swizzled by
// row. The tiles are read both ways: as rows (one chunk column of 32 rows)
// and transposed (ds_read_b64_tr_b16: 8 rows x 4 adjacent chunks). With
// a = (row / 4) % 4 and e = row % 4 the XOR value is 4 (e ^ a) + a at
// d = 128 (256-byte rows) and 4 ((row / 2) % 2 ^ a % 2) + a at d = 64
// (128-byte rows, two to a bank row): a bijection of row % 16, so a chunk
// column of 16 rows covers all 64 banks, and the 8 rows of a transposed read
// fall on 4 different 4-chunk bank quads, each twice. Both reads are then
// free of bank conflicts (the plain row % 16 XOR put a transposed read on 2
// quads, 4 deep).
template <int D>
__device__ inline int chunk_pos(int row, int c) {
  const int a = (row >> 2) & 3;
  if constexpr (D == 128) return c ^ (4 * ((row & 3) ^ a) + a);
  else return c ^ ((4 * (((row >> 1) & 1) ^ (a & 1)) + a) & 7);
}

// Row operand (A of a rows x d product): row `row`, 8 elements from chunk c.
template <int D>
__device__ inline u32x4 row_op(const char* __restrict__ t, int row, int c) {
  return *reinterpret_cast<const u32x4*>(t + row * (D * 2) + chunk_pos<D>(row, c) * 16);
}

// Transposed operand (A of a d x rows product): lane l receives
// T[16 G + 8 p + 4 h + e][32 mt + l % 32] for e = 0..3, p = 0, 1 (h = l / 32),
// the row order in which an accumulator holds its rows (acc_key), so a
// packed accumulator is the matching B operand.
template <int D>
__device__ inline u32x4 tr_op(const char* __restrict__ t, int G, int mt, int lane) {
  const int gi = lane >> 4, e = (lane >> 2) & 3, qq = lane & 3;
  const int h = gi >> 1, dh = gi & 1;
  const int c = 4 * mt + 2 * dh + (qq >> 1);
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = 16 * G + 8 * p + 4 * h + e;
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(t + row * (D * 2) + chunk_pos<D>(row, c) * 16 + 8 * (qq & 1)));
    const u32x2 w = __builtin_bit_cast(u32x2, x);
    out[2 * p] = w[0];
    out[2 * p + 1] = w[1];
  }
  return out;
}

// Global -> registers -> LDS staging of one [64][D] tile by 256 threads:
// NP 16-byte chunks per thread, rows at or beyond nvalid re-read row
// nvalid - 1 (their contributions are masked to zero).
template <int D>
struct Stage {
  static constexpr int CPR = D / 8;
  static constexpr int NP = kTileRows * CPR / kThreads;
  __device__ static inline void load(const uint16_t* __restrict__ base, int nvalid, u32x4 (&r)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int idx = threadIdx.x + kThreads * p;
      const int row = min(idx / CPR, nvalid - 1), c = idx % CPR;
      r[p] = *reinterpret_cast<const u32x4*>(base + (size_t)row * D + c * 8);
    }
  }
  __device__ static inline void store(char* __restrict__ t, const u32x4 (&r)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int idx = threadIdx.x + kThreads * p;
      const int row = idx / CPR, c = idx % CPR;
      *reinterpret_cast<u32x4*>(t + row * (D * 2) + chunk_pos<D>(row, c) * 16) = r[p];
    }
  }
};

typedef __attribute__((address_space(3))) void lds_void_t;

// One 1 KiB direct-to-LDS load: lane l's 16 bytes from sbase + voff land at
// LDS address lds + 16 l. Written as asm so that the compiler's wait
// insertion does not wait for these loads before every LDS read; the tile
// loop waits for them itself before its barrier.
// m0 carries the LDS address; it is listed as clobbered (the compiler warns
// that m0 is reserved), and no other instruction of these kernels reads or
// writes m0 (their assembly has no other m0 reference).
__device__ __attribute__((always_inline)) inline void dma16(const uint16_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Source byte offset, in a [64][D] tile, of the chunk that load instruction
// i of wave w writes to LDS chunk position p = 256 i + 64 w + lane (row
// p / (D/8), position p % (D/8)); the XOR swizzle of chunk_pos is an
// involution, so position -> chunk uses the same map. Rows at or beyond
// nvalid re-read row nvalid - 1.
template <int D>
__device__ inline uint32_t dma_off(int i, int w, int lane, int nvalid) {
  constexpr int CPR = D / 8;
  const int p = 256 * i + 64 * w + lane;
  const int row = p / CPR, pos = p % CPR;
  return (uint32_t)(min(row, nvalid - 1) * (D * 2) + chunk_pos<D>(row, pos) * 16);
}

// LSE in log2 units, +inf where the row does not exist or saw no key, so
// that exp2(s c - lse2) is 0 there.
__device__ inline float lse2_of(const float* __restrict__ lse, int row, int n) {
  if (row >= n) return __builtin_inff();
  const float x = lse[row];
  return x > -__builtin_inff() ? x * kLog2e : __builtin_inff();
}

// The two 16-bit values packed in w (low half first) as fp32, exactly.
template <int DT>
__device__ inline float lo_f32(uint32_t w) {
  if constexpr (DT == DT_BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <int DT>
__device__ inline float hi_f32(uint32_t w) {
  if constexpr (DT == DT_BF16) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// ------------------------------------------------------------------ delta
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void fa_bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                               const uint16_t* __restrict__ dout,
                                                               float* __restrict__ delta, long long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  const long long row = (long long)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + c * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(lo_f32<DT>(a[i]), lo_f32<DT>(b[i]), acc);
      acc = __builtin_fmaf(hi_f32<DT>(a[i]), hi_f32<DT>(b[i]), acc);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < rows && c == 0) delta[row] = acc;
}

// ------------------------------------------------------------------ dK, dV
// 8 waves: wave w owns keys 32 (w % 4) .. +31 of the workgroup's 128 and rows
// 32 (w / 4) .. +31 of every 64-row query tile, so two waves (one per half
// of the rows) accumulate partial dK, dV for the same keys; the halves are
// added through LDS at the end.
constexpr int kDkdvThreads = 512;

template <int D>
__device__ inline uint32_t dma_off8(int i, int w, int lane, int nvalid) {  // 8 loading waves
  constexpr int CPR = D / 8;
  const int p = 512 * i + 64 * w + lane;
  const int row = p / CPR, pos = p % CPR;
  return (uint32_t)(min(row, nvalid - 1) * (D * 2) + chunk_pos<D>(row, pos) * 16);
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kDkdvThreads, 1) void fa_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
    float c2) {
  constexpr int KS = D / 16, MT = D / 32;
  constexpr int TILE = kTileRows * D * 2;
  constexpr int BUF = 2 * TILE + 2 * kTileRows * 4;  // Q, dO, lse2, delta
  constexpr int KL_BYTES = kBwdKeyRows * D * 2;      // K rows of the workgroup's keys
  constexpr int RED = MT * 16 * 256 * 4;             // one accumulator set of 4 waves
  constexpr int SMEM = 2 * BUF + KL_BYTES > RED ? 2 * BUF + KL_BYTES : RED;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  char* const kls = smem + 2 * BUF;

  const int nbg = B * Hkv;
  const int kt = blockIdx.x / nbg, bg = blockIdx.x % nbg;  // key tiles from the first: heaviest first
  const int b = bg / Hkv, g = bg % Hkv, grp = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform for the scalar LDS address
  const int kw = wave & 3, rh = wave >> 2;               // key group, row half of each tile
  const int kt0 = kt * kBwdKeyRows;
  const int wk0 = kt0 + 32 * kw;                         // first key of this wave
  const int key = wk0 + (lane & 31);                     // this lane's key column
  const int off = Nk - Nq;                               // causal: key j visible to query i iff j <= i + off

  // V rows of this wave's 32 keys in registers (B operand of dP = dO V^T);
  // the K rows of all 128 keys in LDS (B operand of S = Q K^T, read per use).
  const size_t kvo = (size_t)bg * Nk * D;
  const int krow = min(key, Nk - 1);
  u32x4 vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    vop[ks] = *reinterpret_cast<const u32x4*>(v + kvo + (size_t)krow * D + 16 * ks + 8 * half);
  {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int p = 0; p < kBwdKeyRows * CPR / kDkdvThreads; ++p) {
      const int idx = threadIdx.x + kDkdvThreads * p;
      const int row = idx / CPR, c = idx % CPR;
      const int src = min(kt0 + row, Nk - 1);
      *reinterpret_cast<u32x4*>(kls + row * (D * 2) + chunk_pos<D>(row, c) * 16) =
          *reinterpret_cast<const u32x4*>(k + kvo + (size_t)src * D + c * 8);
    }
  }
  f32x16 acc_dk[MT], acc_dv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_dk[mt][r] = acc_dv[mt][r] = 0.f;

  // Query tiles that see at least one key of this workgroup, for every
  // q-head of the group.
  const int q_first = CAUSAL ? max(0, kt0 - off) : 0;
  const int t_first = q_first / kTileRows;
  const int n_t = (Nq + kTileRows - 1) / kTileRows;
  const int per_head = max(0, n_t - t_first);
  const int total = grp * per_head;
  // Visit order of the (query tile, q-head) pairs: tile-major with the
  // group's q-heads innermost, so that the workgroups of one kv-head that
  // run side by side (on one XCD: workgroup id L runs on XCD L % 8) read the
  // same Q and dO tile at about the same time and it is fetched into that
  // XCD's L2 once. The first half of the key blocks, dispatched first, walk
  // the tiles down from the last one; the second half start as the first
  // finish, the lightest first, and walk up from their first tile, which
  // keeps them in step with each other as well.
  const int n_kt = (Nk + kBwdKeyRows - 1) / kBwdKeyRows;
  const bool down = kt < (n_kt + 1) / 2;
  auto tile_of = [&](int it) { return down ? n_t - 1 - it / grp : t_first + it / grp; };

  // Q and dO tiles go HBM -> LDS directly (slot it & 1), one tile ahead; the
  // tile's LSE (log2 units) and delta go through one register of threads
  // 0..127. Each wave waits for its own loads before the tile barrier.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)smem;
  float rl = 0.f;
  auto issue = [&](int it) {
    const int h = g * grp + it % grp, t = tile_of(it);
    const size_t qo = ((size_t)b * Hq + h) * Nq;
    const int i0 = t * kTileRows;
    const int nvalid = min(kTileRows, Nq - i0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t* base = (u ? dout : q) + (qo + i0) * D;
      const uint32_t slot = lds0 + (uint32_t)((it & 1) * BUF + u * TILE + 64 * wv * 16);
#pragma unroll
      for (int i = 0; i < TILE / 8192; ++i) dma16(base, dma_off8<D>(i, wv, lane, nvalid), slot + 8192 * i);
    }
    if (threadIdx.x < kTileRows)
      rl = lse2_of(lse + qo + i0, threadIdx.x, Nq - i0);
    else if (threadIdx.x < 2 * kTileRows)
      rl = (i0 + (int)threadIdx.x - kTileRows < Nq) ? delta[qo + i0 + threadIdx.x - kTileRows] : 0.f;
  };
  auto put_rl = [&](int it) {
    if (threadIdx.x < 2 * kTileRows) reinterpret_cast<float*>(smem + (it & 1) * BUF + 2 * TILE)[threadIdx.x] = rl;
  };

  if (total > 0) {
    issue(0);
    put_rl(0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    if (it + 1 < total) issue(it + 1);
    const char* qt = smem + (it & 1) * BUF;
    const char* dot = qt + TILE;
    const float* l2 = reinterpret_cast<const float*>(qt + 2 * TILE);
    const float* dl = l2 + kTileRows;
    const int i0 = tile_of(it) * kTileRows;
    const int r0 = i0 + 32 * rh;  // first query row of this wave in the tile
    // skip a block entirely above the causal diagonal
    if (!CAUSAL || wk0 <= r0 + 31 + off) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32<DT>(row_op<D>(qt, 32 * rh + (lane & 31), 2 * ks + half),
                       row_op<D>(kls, 32 * kw + (lane & 31), 2 * ks + half), s);
        dp = mfma32<DT>(row_op<D>(dot, 32 * rh + (lane & 31), 2 * ks + half), vop[ks], dp);
      }
      // masking only where this wave's keys reach past its first row or Nk
      const bool need_mask = (wk0 + 31 >= Nk) || (CAUSAL && wk0 + 31 > r0 + off);
      // P and dS; register r holds query row 32 rh + acc_key(r, half) of the tile.
      uint32_t pk[8], dsk[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int rl0 = 32 * rh + 8 * m + 4 * half;
        const f32x4 L = *reinterpret_cast<const f32x4*>(l2 + rl0);
        const f32x4 Dv = *reinterpret_cast<const f32x4*>(dl + rl0);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * m + e;
          float x = exp2_fast(__builtin_fmaf(s[r], c2, -L[e]));
          if (need_mask) {
            const bool hide = (key >= Nk) | (CAUSAL & (key > i0 + rl0 + e + off));
            x = hide ? 0.f : x;
          }
          p[e] = x;
          ds[e] = x * (dp[r] - Dv[e]);
        }
        pk[2 * m] = pack2<DT>(p[0], p[1]);
        pk[2 * m + 1] = pack2<DT>(p[2], p[3]);
        dsk[2 * m] = pack2<DT>(ds[0], ds[1]);
        dsk[2 * m + 1] = pack2<DT>(ds[2], ds[3]);
      }
      // dV^T += dO^T P, dK^T += Q^T dS over this wave's 32 rows
#pragma unroll
      for (int G = 0; G < 2; ++G) {
        const u32x4 bp = {pk[4 * G], pk[4 * G + 1], pk[4 * G + 2], pk[4 * G + 3]};
        const u32x4 bs = {dsk[4 * G], dsk[4 * G + 1], dsk[4 * G + 2], dsk[4 * G + 3]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc_dv[mt] = mfma32<DT>(tr_op<D>(dot, 2 * rh + G, mt, lane), bp, acc_dv[mt]);
          acc_dk[mt] = mfma32<DT>(tr_op<D>(qt, 2 * rh + G, mt, lane), bs, acc_dk[mt]);
        }
      }
    }
    if (it + 1 < total) put_rl(it + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile it + 1 has landed
    __syncthreads();
  }

  // Add the two row halves' partial sums (through LDS, register-major so a
  // register of all 256 lanes of a half is one contiguous row), then write.
  // acc register r of block mt holds d = 32 mt + acc_key(r, half) of this key.
  float* red = reinterpret_cast<float*>(smem);
  const int rlane = kw * 64 + lane;
  auto reduce = [&](f32x16 (&acc)[MT]) {
    if (rh == 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(mt * 16 + r) * 256 + rlane] = acc[mt][r];
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] += red[(mt * 16 + r) * 256 + rlane];
    }
    __syncthreads();
  };
  reduce(acc_dk);
  reduce(acc_dv);

  if (rh != 0 || key >= Nk) return;
  uint16_t* dkr = dk + kvo + (size_t)key * D;
  uint16_t* dvr = dv + kvo + (size_t)key * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = 32 * mt + 8 * m + 4 * half;
      const u32x2 wk = {pack2<DT>(acc_dk[mt][4 * m] * scale, acc_dk[mt][4 * m + 1] * scale),
                        pack2<DT>(acc_dk[mt][4 * m + 2] * scale, acc_dk[mt][4 * m + 3] * scale)};
      const u32x2 wvv = {pack2<DT>(acc_dv[mt][4 * m], acc_dv[mt][4 * m + 1]),
                         pack2<DT>(acc_dv[mt][4 * m + 2], acc_dv[mt][4 * m + 3])};
      *reinterpret_cast<u32x2*>(dkr + d0) = wk;
      *reinterpret_cast<u32x2*>(dvr + d0) = wvv;
    }
}

// ------------------------------------------------------------------ dQ
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int B, int Hq, int Hkv, int Nq, int Nk, float scale, float c2, int n_qt) {
  constexpr int KS = D / 16, MT = D / 32;
  constexpr int TILE = kTileRows * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];  // (K, V) x 2 buffers

  // last query tiles first; one kv-head's workgroups on one XCD when the
  // (batch, kv-head) pairs divide over the 8 XCDs, so its K and V are
  // fetched into that XCD's L2 once
  const Work wk = map_work(blockIdx.x, B, Hq, Hkv, n_qt);
  const int qt = wk.qt, b = wk.b, h = wk.h, g = wk.g;
  const int bh = b * Hq + h;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int q0 = qt * kBwdQueryRows;
  const int q0w = q0 + 32 * wave;                  // first query row of this wave
  const int qrow = q0w + (lane & 31);             // this lane's query column
  const int off = Nk - Nq;
  const size_t qo = (size_t)bh * Nq;
  const size_t kvo = ((size_t)b * Hkv + g) * Nk * D;

  // Q^T and dO^T operands (B of S^T = K Q^T, dP^T = V dO^T), LSE and delta of this row.
  const int qr = min(qrow, Nq - 1);
  u32x4 qop[KS], dop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qop[ks] = *reinterpret_cast<const u32x4*>(q + (qo + qr) * D + 16 * ks + 8 * half);
    dop[ks] = *reinterpret_cast<const u32x4*>(dout + (qo + qr) * D + 16 * ks + 8 * half);
  }
  const float l2 = lse2_of(lse + qo, qrow, Nq);
  const float dl = qrow < Nq ? delta[qo + qrow] : 0.f;

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  int n_kv = (Nk + kTileRows - 1) / kTileRows;
  if (CAUSAL) {
    const int last_key = min(q0 + kBwdQueryRows, Nq) - 1 + off;
    n_kv = last_key < 0 ? 0 : min(n_kv, last_key / kTileRows + 1);
  }

  // K_j and V_j go HBM -> LDS directly (slot j & 1), issued one tile ahead;
  // each wave's loads are waited for (vmcnt) before the barrier that ends
  // the tile, so the next tile is complete for every wave after it.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)smem;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform for the scalar LDS address
  auto issue = [&](int j) {
    const int nvalid = min(kTileRows, Nk - j * kTileRows);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* base = (t ? v : k) + kvo + (size_t)j * kTileRows * D;
      const uint32_t slot = lds0 + (uint32_t)((j & 1) * 2 * TILE + t * TILE + 64 * wv * 16);
#pragma unroll
      for (int i = 0; i < TILE / 4096; ++i) dma16(base, dma_off<D>(i, wv, lane, nvalid), slot + 4096 * i);
    }
  };
  if (n_kv > 0) issue(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q, dO operands and tile 0
  __syncthreads();
  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) issue(j + 1);
    const char* kt = smem + (j & 1) * 2 * TILE;
    const char* vt = kt + TILE;
    // S^T = K Q^T and dP^T = V dO^T for both 32-key blocks (four chains)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma32<DT>(row_op<D>(kt, 32 * kb + (lane & 31), 2 * ks + half), qop[ks], s[kb]);
        dp[kb] = mfma32<DT>(row_op<D>(vt, 32 * kb + (lane & 31), 2 * ks + half), dop[ks], dp[kb]);
      }
    // masking only on the causal diagonal or a ragged last tile
    const bool need_mask = (j * kTileRows + kTileRows > Nk) || (CAUSAL && j * kTileRows + kTileRows - 1 > q0w + off);
    uint32_t dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // register r holds key j*64 + 32 kb + acc_key(r, half) of this lane's query
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float x = exp2_fast(__builtin_fmaf(s[kb][r + u], c2, -l2));
          if (need_mask) {
            const int key = j * kTileRows + 32 * kb + acc_key(r + u, half);
            const bool hide = (key >= Nk) | (CAUSAL & (key > qrow + off));
            x = hide ? 0.f : x;
          }
          ds[u] = x * (dp[kb][r + u] - dl);
        }
        dsk[kb][r >> 1] = pack2<DT>(ds[0], ds[1]);
      }
    }
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int kb = G >> 1, o4 = 4 * (G & 1);
      const u32x4 bs = {dsk[kb][o4], dsk[kb][o4 + 1], dsk[kb][o4 + 2], dsk[kb][o4 + 3]};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32<DT>(tr_op<D>(kt, G, mt, lane), bs, acc[mt]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile j + 1 has landed
    __syncthreads();
  }

  if (qrow >= Nq) return;
  uint16_t* row = dq + (qo + qrow) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = 32 * mt + 8 * m + 4 * half;
      const u32x2 w = {pack2<DT>(acc[mt][4 * m] * scale, acc[mt][4 * m + 1] * scale),
                       pack2<DT>(acc[mt][4 * m + 2] * scale, acc[mt][4 * m + 3] * scale)};
      *reinterpret_cast<u32x2*>(row + d0) = w;
    }
}

template <int DT, int D, bool CAUSAL>
hipError_t launch_t(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.Nq;
  constexpr int RPB = kThreads / (D / 8);
  const long long nb_delta = (rows + RPB - 1) / RPB;
  const long long nb_kv = (long long)((a.Nk + kBwdKeyRows - 1) / kBwdKeyRows) * a.B * a.Hkv;
  const int n_qt = (a.Nq + kBwdQueryRows - 1) / kBwdQueryRows;
  const long long nb_q = (long long)n_qt * a.B * a.Hq;
  if (nb_delta > 0x7fffffffLL || nb_kv > 0x7fffffffLL || nb_q > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fa_bwd_delta_kernel<DT, D>), dim3((unsigned)nb_delta), dim3(kThreads), 0, stream,
                     (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows);
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<DT, D, CAUSAL>), dim3((unsigned)nb_kv), dim3(kDkdvThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                     a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale, c2);
  hipLaunchKernelGGL((fa_bwd_dq_kernel<DT, D, CAUSAL>), dim3((unsigned)nb_q), dim3(kThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                     a.delta, (uint16_t*)a.dq, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale, c2, n_qt);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_c(const BwdArgs& a, hipStream_t stream) {
  return a.causal ? launch_t<DT, D, true>(a, stream) : launch_t<DT, D, false>(a, stream);
}

template <int DT>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_c<DT, 128>(a, stream) : launch_c<DT, 64>(a, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  return a.dtype == DT_BF16 ? launch_d<DT_BF16>(a, stream) : launch_d<DT_FP16>(a, stream);
}

}  // namespace fa
