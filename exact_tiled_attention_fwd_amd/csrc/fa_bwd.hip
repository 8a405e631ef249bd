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
// The same for an LSE value already loaded.
__device__ inline float lse2_of_value(float x) { return x > -__builtin_inff() ? x * kLog2e : __builtin_inff(); }

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
// 8 waves over 128 keys: wave w takes keys 32 (w % 4) .. +31 and, for S and
// dP (and so P and dS), rows 32 (w / 4) .. +31 of every 64-row query tile.
// The two waves of a key group split the accumulation: the first (w < 4)
// adds dV^T over all 64 rows, the second dK^T; each hands the other, through
// LDS, the half it lacks (the first its dS, the second its P). So a wave
// keeps a single 32 x d accumulator, and the K and V rows of its keys stay in
// registers as the B operands of S and dP.
constexpr int kDkdvThreads = 512;

template <bool V>
struct BoolC {
  static constexpr bool value = V;
};

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kDkdvThreads, 1) void fa_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
    float c2) {
  constexpr int KS = D / 16, MT = D / 32;
  constexpr int TILE = kTileRows * D * 2;
  constexpr int BUF = 2 * TILE + 2 * kTileRows * 4;  // Q, dO, lse2, delta
  constexpr int NBUF = 3;                            // staged query tiles: previous, this, next
  constexpr int XW = 2 * 64 * 16;                    // a wave's packed P or dS: 2 x 16 bytes per lane
  __shared__ __attribute__((aligned(16))) char smem[NBUF * BUF + 2 * 8 * XW];
  char* const xch = smem + NBUF * BUF;               // [tile parity][wave][2][64 lanes][16 bytes]

  const int nbg = B * Hkv;
  const int kt = blockIdx.x / nbg, bg = blockIdx.x % nbg;  // key tiles from the first: heaviest first
  const int b = bg / Hkv, g = bg % Hkv, grp = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform for the scalar LDS address
  const int kw = wave & 3, rh = wave >> 2;               // key group, row half of each tile
  const bool dv_wave = (wv >> 2) == 0;                   // accumulates dV (else dK)
  const int kt0 = kt * kBwdKeyRows;
  const int wk0 = kt0 + 32 * kw;                         // first key of this wave
  const int key = wk0 + (lane & 31);                     // this lane's key column
  const int off = Nk - Nq;                               // causal: key j visible to query i iff j <= i + off

  // K and V rows of this wave's 32 keys: the B operands of S = Q K^T and dP = dO V^T.
  const size_t kvo = (size_t)bg * Nk * D;
  const int krow = min(key, Nk - 1);
  u32x4 kop[KS], vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kop[ks] = *reinterpret_cast<const u32x4*>(k + kvo + (size_t)krow * D + 16 * ks + 8 * half);
    vop[ks] = *reinterpret_cast<const u32x4*>(v + kvo + (size_t)krow * D + 16 * ks + 8 * half);
  }
  f32x16 acc[MT];  // dV^T or dK^T of this wave's keys
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

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
  auto tile_at = [&](int ti) { return down ? n_t - 1 - ti : t_first + ti; };  // ti-th tile visited

  // Q and dO tiles go HBM -> LDS directly (slot it % 3), one tile ahead; the
  // tile's LSE (log2 units) and delta go through one register of threads
  // 0..127. Each wave waits for its own loads before the tile barrier.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)smem;
  float rl = 0.f;
  auto issue = [&](int t, int hg, int slot) {  // query tile t of q-head hg of the group
    const int h = g * grp + hg;
    const size_t qo = ((size_t)b * Hq + h) * Nq;
    const int i0 = t * kTileRows;
    const int nvalid = min(kTileRows, Nq - i0);
    // the Q and dO loads come from the dV waves only (a quarter of each
    // tile per wave): the dK waves' path through a tile is the longer one
    if (dv_wave) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint16_t* base = (u ? dout : q) + (qo + i0) * D;
        const uint32_t dst = lds0 + (uint32_t)(slot * BUF + u * TILE + 64 * wv * 16);
#pragma unroll
        for (int i = 0; i < TILE / 4096; ++i) dma16(base, dma_off<D>(i, wv, lane, nvalid), dst + 4096 * i);
      }
    }
    // One plain load per thread of 0..127 (LSE, then delta), of a row that
    // exists; nothing is computed from it until put_rl, so no wait for it
    // (or for the tile loads before it) is placed here.
    if (threadIdx.x < 2 * kTileRows) {
      const int r = (int)threadIdx.x % kTileRows;
      rl = (threadIdx.x < kTileRows ? lse : delta)[qo + i0 + min(r, Nq - i0 - 1)];
    }
  };
  auto put_rl = [&](int slot, int i0) {  // i0: first row of the tile in that slot
    if (threadIdx.x < 2 * kTileRows) {
      const bool row_ok = (int)threadIdx.x % kTileRows < Nq - i0;
      const float x = threadIdx.x < kTileRows ? (row_ok ? lse2_of_value(rl) : __builtin_inff()) : (row_ok ? rl : 0.f);
      reinterpret_cast<float*>(smem + slot * BUF + 2 * TILE)[threadIdx.x] = x;
    }
  };

  // Lane offsets (bytes in a [64][D] tile) of the operand reads: the row
  // operand (row 32 RH + lane % 32, chunk 2 ks + half) and the transposed
  // one (two ds_read_b64_tr_b16: lane l receives T[16 G + 8 p + 4 h + e]
  // [32 mt + l % 32] for e = 0..3, p = 0, 1, h = l / 32, the row order of an
  // accumulator, so a packed accumulator is the matching B operand) for
  // 16-row group G = 0; group G adds 16 G rows, since the swizzle depends on
  // the row only through row % 16.
  auto row_off = [&](int rh_, int ks) {
    const int row = 32 * rh_ + (lane & 31);
    return (uint32_t)(row * (D * 2) + chunk_pos<D>(row, 2 * ks + half) * 16);
  };
  uint32_t tro[MT][2];
  {
    const int gi = lane >> 4, e = (lane >> 2) & 3, qq = lane & 3;
    const int hh = gi >> 1, dh = gi & 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const int row = 8 * p2 + 4 * hh + e, c = 4 * mt + 2 * dh + (qq >> 1);
        tro[mt][p2] = (uint32_t)(row * (D * 2) + chunk_pos<D>(row, c) * 16 + 8 * (qq & 1));
      }
  }

  constexpr int NU = 4 * MT, NM = 2 * KS, PF = 4;
  uint32_t own[8], oth[8];  // packed B operands of U: this wave's half, the partner's half
  uint32_t fresh[8];        // this wave's half of the tile just softmaxed
  f32x16 s, dp;

  // The loop for the waves of row half RH (0: accumulate dV, 1: dK).
  auto run = [&](auto rhc) {
    constexpr int RH = decltype(rhc)::value ? 1 : 0;
    uint32_t rwo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rwo[ks] = row_off(RH, ks);

    // Matrix-core phases: M = S and dP of this wave's rows of the tile (2 KS
    // ops, A = Q and dO rows, alternating), U = the dV^T (or dK^T) update over
    // both row halves (2 x 2 x MT ops, A = dO^T (or Q^T) read transposed). A
    // operands come through a ring of 4 registers, fetched 4 ops ahead.
    auto phase = [&](auto do_u, const char* tile) {
      constexpr bool DU = decltype(do_u)::value;
      constexpr int N = DU ? NU : NM;
      const char* tsrc = tile + (RH == 0 ? TILE : 0);  // dO^T for dV, Q^T for dK
      auto read = [&](int t) -> u32x4 {
        if constexpr (DU) {
          const int h = t / (2 * MT), G = (t / MT) % 2, mt = t % MT;
          const char* tg = tsrc + (2 * h + G) * 16 * (D * 2);
          u32x4 out;
#pragma unroll
          for (int p2 = 0; p2 < 2; ++p2) {
            const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tg + tro[mt][p2]));
            const u32x2 w = __builtin_bit_cast(u32x2, x);
            out[2 * p2] = w[0];
            out[2 * p2 + 1] = w[1];
          }
          return out;
        } else {
          return *reinterpret_cast<const u32x4*>(tile + ((t & 1) ? TILE : 0) + rwo[t >> 1]);
        }
      };
      u32x4 buf[PF];
#pragma unroll
      for (int t = 0; t < PF; ++t) buf[t] = read(t);
      if constexpr (!DU) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < N; ++t) {
        const u32x4 a = buf[t % PF];
        if (t + PF < N) buf[t % PF] = read(t + PF);
        if constexpr (DU) {
          const int h = t / (2 * MT), G = (t / MT) % 2, mt = t % MT;
          const uint32_t* bsrc = (h == RH) ? own : oth;
          const u32x4 bb = {bsrc[4 * G], bsrc[4 * G + 1], bsrc[4 * G + 2], bsrc[4 * G + 3]};
          acc[mt] = mfma32<DT>(a, bb, acc[mt]);
        } else {
          if (t & 1)
            dp = mfma32<DT>(a, vop[t >> 1], dp);
          else
            s = mfma32<DT>(a, kop[t >> 1], s);
        }
      }
      // keep the order: the first PF operands' reads, then each MFMA
      // followed by the reads of the operand PF ahead
      __builtin_amdgcn_sched_group_barrier(0x100, DU ? 2 * PF : PF, 0);
#pragma unroll
      for (int t = 0; t < N; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (t + PF < N) __builtin_amdgcn_sched_group_barrier(0x100, DU ? 2 : 1, 0);
      }
    };

    // P and dS of this wave's rows (register r holds query row 32 RH +
    // acc_key(r, half) of the tile); keeps one, hands the other to the partner.
    auto softmax = [&](const char* tile, int i0, int it) {
      const float* l2 = reinterpret_cast<const float*>(tile + 2 * TILE);
      const float* dl = l2 + kTileRows;
      const int r0 = i0 + 32 * RH;
      // the same in every lane; read as wave-uniform so that tiles off the
      // diagonal skip the masking by a scalar branch
      const bool need_mask =
          __builtin_amdgcn_readfirstlane((int)((wk0 + 31 >= Nk) || (CAUSAL && wk0 + 31 > r0 + off))) != 0;
      uint32_t pk[8], dsk[8];
      // masked scores to -inf first (their P and dS are then exactly 0), so
      // the exponentials below carry no per-element select
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + 32 * RH + 8 * (r >> 2) + 4 * half + (r & 3);
          if ((key >= Nk) | (CAUSAL & (key > row + off))) s[r] = -__builtin_inff();
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int rl0 = 32 * RH + 8 * m + 4 * half;
        const f32x4 L = *reinterpret_cast<const f32x4*>(l2 + rl0);
        const f32x4 Dv = *reinterpret_cast<const f32x4*>(dl + rl0);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * m + e;
          const float x = exp2_fast(__builtin_fmaf(s[r], c2, -L[e]));
          p[e] = x;
          ds[e] = x * (dp[r] - Dv[e]);
        }
        pk[2 * m] = pack2<DT>(p[0], p[1]);
        pk[2 * m + 1] = pack2<DT>(p[2], p[3]);
        dsk[2 * m] = pack2<DT>(ds[0], ds[1]);
        dsk[2 * m + 1] = pack2<DT>(ds[2], ds[3]);
      }
      const uint32_t* give = RH == 0 ? dsk : pk;
      char* xw = xch + ((it & 1) * 8 + wv) * XW + lane * 16;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<u32x4*>(xw + 1024 * u) = u32x4{give[4 * u], give[4 * u + 1], give[4 * u + 2], give[4 * u + 3]};
#pragma unroll
      for (int j = 0; j < 8; ++j) fresh[j] = RH == 0 ? pk[j] : dsk[j];
    };

    // U of tile j: both row halves' P (or dS), this wave's from registers,
    // the partner's from the exchange buffer of parity j & 1 (zero for a row
    // half that sees none of these keys).
    auto update = [&](int j, bool j_own, bool j_oth, const char* tile) {
      if (j_oth) {
        const char* xr = xch + ((j & 1) * 8 + (wv ^ 4)) * XW + lane * 16;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(xr + 1024 * u);
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) oth[4 * u + q2] = w[q2];
        }
      } else {
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) oth[q2] = 0u;
      }
      if (!j_own) {
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) own[q2] = 0u;
      }
      phase(BoolC<true>{}, tile);
    };

    // One barrier per tile. In the interval of tile it a wave runs S, dP and
    // the softmax of tile it (its half for the partner to the exchange
    // buffer of parity it & 1) and U of tile it - 1; the two waves of a key
    // group, which share a SIMD, take these in opposite orders (row half 0:
    // S first), so that one's vector work meets the other's matrix-core
    // work. Tiles it - 1, it and it + 1 (in flight) are in use at once: three
    // slots; the loads of tile it + 1 go to the slot of tile it - 2, last
    // read by U in the previous interval. The exchange buffer of a parity is
    // written in one interval, read in the next and rewritten in the one
    // after, each across a barrier.
    int cur = 0, prv = 0;
    int ti = 0, hg = 0;                 // visit position of tile it: tile index, q-head in the group
    bool p_own = false, p_oth = false;  // the previous tile's row halves see these keys
    for (int it = 0; it < total; ++it) {
      const int nxt = cur == NBUF - 1 ? 0 : cur + 1;
      int ti_n = ti, hg_n = hg + 1;
      if (hg_n == grp) {
        hg_n = 0;
        ++ti_n;
      }
      if (it + 1 < total) issue(tile_at(ti_n), hg_n, nxt);
      const int i0 = tile_at(ti) * kTileRows;
      // a row half sees these keys unless it lies entirely above the causal diagonal
      const bool a_lo = !CAUSAL || wk0 <= i0 + 31 + off, a_hi = !CAUSAL || wk0 <= i0 + 63 + off;
      const bool a_own = RH ? a_hi : a_lo, a_oth = RH ? a_lo : a_hi;
      const char* tile = smem + cur * BUF;
      const bool do_u = it > 0 && (p_own || p_oth);
      if (RH == 1 && do_u) update(it - 1, p_own, p_oth, smem + prv * BUF);
      if (a_own) {
        phase(BoolC<false>{}, tile);
        softmax(tile, i0, it);
      }
      if (RH == 0 && do_u) update(it - 1, p_own, p_oth, smem + prv * BUF);
#pragma unroll
      for (int q2 = 0; q2 < 8; ++q2) own[q2] = fresh[q2];
      p_own = a_own;
      p_oth = a_oth;
      if (it + 1 < total) put_rl(nxt, tile_at(ti_n) * kTileRows);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile it + 1 has landed
      __syncthreads();
      prv = cur;
      cur = nxt;
      ti = ti_n;
      hg = hg_n;
    }
    if (total > 0 && (p_own || p_oth)) update(total - 1, p_own, p_oth, smem + prv * BUF);
  };

  if (total > 0) {
    issue(tile_at(0), 0, 0);
    put_rl(0, tile_at(0) * kTileRows);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (dv_wave)
    run(BoolC<false>{});
  else
    run(BoolC<true>{});

  // acc register r of block mt holds d = 32 mt + acc_key(r, half) of this key.
  if (key >= Nk) return;
  uint16_t* row = (dv_wave ? dv : dk) + kvo + (size_t)key * D;
  const float f = dv_wave ? 1.f : scale;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = 32 * mt + 8 * m + 4 * half;
      const u32x2 w = {pack2<DT>(acc[mt][4 * m] * f, acc[mt][4 * m + 1] * f),
                       pack2<DT>(acc[mt][4 * m + 2] * f, acc[mt][4 * m + 3] * f)};
      *reinterpret_cast<u32x2*>(row + d0) = w;
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
  // wave index read as wave-uniform, so that the per-tile mask test below is
  // a scalar branch (tiles off the diagonal skip the masking entirely)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, half = lane >> 5;
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

  // Lane offsets (bytes in a [64][D] tile) of the operand reads: K or V rows
  // lane % 32 (+ 32 kb, a constant), chunk 2 ks + half; K^T transposed (the
  // pattern of the dK/dV kernel) for 16-row group 0, group G adding 16 G
  // rows, since the swizzle depends on the row only through row % 16.
  uint32_t rwo[KS], tro[MT][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    rwo[ks] = (uint32_t)((lane & 31) * (D * 2) + chunk_pos<D>(lane & 31, 2 * ks + half) * 16);
  {
    const int gi = lane >> 4, e = (lane >> 2) & 3, qq = lane & 3;
    const int hh = gi >> 1, dh = gi & 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const int row = 8 * p2 + 4 * hh + e, c = 4 * mt + 2 * dh + (qq >> 1);
        tro[mt][p2] = (uint32_t)(row * (D * 2) + chunk_pos<D>(row, c) * 16 + 8 * (qq & 1));
      }
  }

  // Matrix-core phases, A operands through a ring of PF registers fetched PF
  // ops ahead (the first PF reads pinned ahead of the first MFMA):
  //   SD(kb): S^T and dP^T of 32-key block kb (2 KS ops, A = K and V rows,
  //           alternating; B = Q^T, dO^T in registers);
  //   DQ:     dQ^T += K^T dS^T (4 x MT ops, A = K^T transposed).
  constexpr int PF = 4;
  f32x16 s, dp;
  uint32_t dsk[2][8];
  auto phase = [&](auto is_dq, const char* kt, const char* vt, int kb) {
    constexpr bool DQ = decltype(is_dq)::value;
    constexpr int N = DQ ? 4 * MT : 2 * KS;
    auto read = [&](int t) -> u32x4 {
      if constexpr (DQ) {
        const int G = t / MT, mt = t % MT;
        const char* tg = kt + G * 16 * (D * 2);
        u32x4 out;
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tg + tro[mt][p2]));
          const u32x2 w = __builtin_bit_cast(u32x2, x);
          out[2 * p2] = w[0];
          out[2 * p2 + 1] = w[1];
        }
        return out;
      } else {
        return *reinterpret_cast<const u32x4*>(((t & 1) ? vt : kt) + kb * 32 * (D * 2) + rwo[t >> 1]);
      }
    };
    u32x4 buf[PF];
#pragma unroll
    for (int t = 0; t < PF; ++t) buf[t] = read(t);
    if constexpr (!DQ) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < N; ++t) {
      const u32x4 a = buf[t % PF];
      if (t + PF < N) buf[t % PF] = read(t + PF);
      if constexpr (DQ) {
        const int G = t / MT, mt = t % MT;
        const int kb2 = G >> 1, o4 = 4 * (G & 1);
        const u32x4 bs = {dsk[kb2][o4], dsk[kb2][o4 + 1], dsk[kb2][o4 + 2], dsk[kb2][o4 + 3]};
        acc[mt] = mfma32<DT>(a, bs, acc[mt]);
      } else {
        if (t & 1)
          dp = mfma32<DT>(a, dop[t >> 1], dp);
        else
          s = mfma32<DT>(a, qop[t >> 1], s);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, DQ ? 2 * PF : PF, 0);
#pragma unroll
    for (int t = 0; t < N; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + PF < N) __builtin_amdgcn_sched_group_barrier(0x100, DQ ? 2 : 1, 0);
    }
  };

  if (n_kv > 0) issue(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q, dO operands and tile 0
  __syncthreads();
  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) issue(j + 1);
    const char* kt = smem + (j & 1) * 2 * TILE;
    const char* vt = kt + TILE;
    // masking only on the causal diagonal or a ragged last tile
    const bool need_mask = (j * kTileRows + kTileRows > Nk) || (CAUSAL && j * kTileRows + kTileRows - 1 > q0w + off);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      phase(BoolC<false>{}, kt, vt, kb);
      // register r holds key j*64 + 32 kb + acc_key(r, half) of this lane's query
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float x = exp2_fast(__builtin_fmaf(s[r + u], c2, -l2));
          if (need_mask) {
            const int key = j * kTileRows + 32 * kb + acc_key(r + u, half);
            const bool hide = (key >= Nk) | (CAUSAL & (key > qrow + off));
            x = hide ? 0.f : x;
          }
          ds[u] = x * (dp[r + u] - dl);
        }
        dsk[kb][r >> 1] = pack2<DT>(ds[0], ds[1]);
      }
    }
    phase(BoolC<true>{}, kt, vt, 0);
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
