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
// head-width-128 kernel, two groups of 4 waves alternate on the same SIMDs,
// one issuing matrix-core work while the other runs its softmax, and the
// waves of group 0 move every K and V tile HBM -> LDS directly
// (global_load_lds_dwordx4) into 4-slot rings, K two tiles and V one tile
// ahead, with one barrier per step:
//   S^T = K Q^T             A = K rows from LDS, B = Q^T held in registers
//   online softmax          p = 2^(s c - m + 4) against the running
//                           reference m; the row maximum is taken only on a
//                           row's first tile or when some lane's sum exceeds
//                           448 (E4M3's largest value, which then bounds
//                           every p); the 2^4 keeps small values normal and
//                           cancels against the running sum
//   O^T += V^T P^T          A = V^T gathered from the row-major V tile with
//                           transposed 8-bit LDS reads (ds_read_b64_tr_b8),
//                           in the key order of the P operand; B = P rounded
//                           to E4M3 (RNE)
#include <type_traits>

#include "fa_fp8_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 512;           // 8 waves = 2 groups of 4
constexpr int kBM = kFp8BlockRows;      // 256 query rows
constexpr int kD = 128;                 // head width = bytes per row in fp8
constexpr int kRows = 64;               // keys per tile
constexpr int kSlots = 4;               // ring depth for K and for V
constexpr int kTile = kRows * kD;       // 8 KiB
constexpr float kPOffset = 4.f;         // P is scaled by 2^4 before rounding
constexpr float kSumLimit8 = 448.f;     // largest finite E4M3 value

__device__ inline f32x16 mfma_f8(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ inline i32x8 cat(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// LDS tiles are row-major [64 keys][128 bytes], 8 chunks of 16 bytes a row.
//   K: chunk c of row r at position c ^ ((r / 2) % 8). An A-operand read
//      takes one chunk column of 32 rows; each 16 rows of it fill all banks.
//   V: chunk c of row r at position c ^ 2 ((r / 2) % 2 + 2 ((r / 8) % 2)).
//      A transposed read takes 8 key rows x 2 chunks per 16 lanes (32 bytes
//      a row, two 8-byte halves); the 16 rows of a half-wave (keys k and
//      k + 4) then fill all banks.
// Both maps are involutions in c, so position -> chunk is the same map.
__device__ inline int k_phys(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ inline int v_phys(int r, int c) { return c ^ (2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1))); }

// Byte offset in the global tile of the 16-byte chunk that load instruction
// i (0, 1) of wave w (0..3 of group 0) writes to LDS position
// p = 256 i + 64 w + lane (row p / 8, position p % 8). Rows at or beyond
// nvalid re-read row nvalid - 1; their scores are masked to -inf. The
// swizzles depend on the row only through row % 16, so for a full tile the
// offset of instruction 1 is that of instruction 0 plus 32 rows.
template <bool IS_V>
__device__ inline uint32_t dma_src(int i, int w, int lane, int nvalid) {
  const int p = 256 * i + 64 * w + lane;
  const int row = p >> 3, pos = p & 7;
  const int c = IS_V ? v_phys(row, pos) : k_phys(row, pos);
  return (uint32_t)(min(row, nvalid - 1) * kD + c * 16);
}

// One 1 KiB direct-to-LDS load: lane l's 16 bytes from sbase + voff land at
// LDS address lds + 16 l. Asm, so that the compiler's wait insertion, which
// cannot tell ring slots apart, does not wait for every load in flight before
// each LDS read; the step barriers do the waiting.
// m0 carries the LDS address; it is listed as clobbered (the compiler warns
// that m0 is reserved), and no other instruction of these kernels reads or
// writes m0 (their assembly has no other m0 reference).
__device__ __attribute__((always_inline)) inline void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Barrier after waiting until this thread has at most `pending` (0, 2 or 4,
// wave-uniform) direct-to-LDS loads outstanding.
__device__ __attribute__((always_inline)) inline void dma_barrier(int pending) {
  pending = __builtin_amdgcn_readfirstlane(pending);  // wave-uniform: scalar branches
  if (pending >= 4)
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
  else if (pending >= 2)
    __builtin_amdgcn_s_waitcnt(0x0F72);  // vmcnt(2)
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// A operand of S^T = K Q^T: key 32 kb + lane % 32, head-dim bytes
// 64 ks + 32 h .. +31 (chunks 4 ks + 2 h and the next).
__device__ inline i32x8 k_op(const char* __restrict__ kl, int kb, int ks, int lane) {
  const int r = 32 * kb + (lane & 31), c = 4 * ks + 2 * (lane >> 5);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(kl + r * kD + k_phys(r, c) * 16);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(kl + r * kD + k_phys(r, c + 1) * 16);
  return cat(lo, hi);
}

// A operand of O^T += V^T P^T for head-dim rows 32 mt ..: byte b of lane l
// is V[key(b)][32 mt + l % 32] with key(b) = 32 (b / 16) + 8 ((b % 16) / 4)
// + 4 h + b % 4 (h = l / 32), the key order in which a lane packs its P
// values. ds_read_b64_tr_b8 gives lane i of each 16-lane group byte i % 8 of
// the 8 bytes addressed by lane 2 e + i / 8, as its byte e (e = 0..7); so in
// read t lane 2 e + s of a group addresses key row key(8 t + e), head-dim
// bytes 32 mt + 16 g + 8 s (g = (l / 16) % 2), and every lane ends up with
// bytes 8 t .. 8 t + 7 of its operand.
__device__ inline i32x8 vt_op(const char* __restrict__ vl, int mt, int lane) {
  const int j = lane & 15, e = j >> 1, s = j & 1, g = (lane >> 4) & 1, h = lane >> 5;
  const int c = 2 * mt + g;
  i32x8 out;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int key = 32 * (t >> 1) + 16 * (t & 1) + 8 * (e >> 2) + 4 * h + (e & 3);
    const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2_t*)(vl + key * kD + v_phys(key, c) * 16 + 8 * s));
    out[2 * t] = w[0];
    out[2 * t + 1] = w[1];
  }
  return out;
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
// every lane's sum is at most kSumLimit8 the values fit E4M3 and are kept.
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

// The 4 tile loads of one step (K_{i+2}: 2, V_{i+1}: 2 instructions per
// wave), slotted in after MFMAs 1, 3, 5, 7 of a full 8-op matrix-core phase.
// Full tiles only. With ALWAYS the loads carry no branch (which would split
// the phase into several scheduling regions): the caller points a tile that
// does not exist at tile 0 and at the ring slot it would have had, which no
// wave reads.
template <bool ALWAYS = false>
struct DmaSpread {
  const uint8_t* kbase;
  const uint8_t* vbase;
  uint32_t kslot, vslot;
  bool has_k, has_v;
  uint32_t dk, dv;
  __device__ __attribute__((always_inline)) void operator()(int t) const {
    if ((t & 1) == 0) return;
    const int j = t >> 1;
    if (j < 2) {
      if (ALWAYS || has_k) dma16(kbase + 32 * kD * j, dk, kslot + 4096 * j);
    } else {
      if (ALWAYS || has_v) dma16(vbase + 32 * kD * (j - 2), dv, vslot + 4096 * (j - 2));
    }
  }
};
struct NoDma {
  __device__ void operator()(int) const {}
};

// ALIGNED: every key tile is full (Nk a multiple of the tile rows).
template <bool CAUSAL, bool ALIGNED>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, const float* __restrict__ q_ds,
    const float* __restrict__ k_ds, const float* __restrict__ v_ds, int B, int Hq, int Hkv, int Nq, int Nk,
    float scale_log2, int n_qt) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kSlots * kTile];
  char* const kring = smem;                   // K tile t in slot t % 4
  char* const vring = smem + kSlots * kTile;  // V tile t in slot t % 4
  const Work wk = map_work(blockIdx.x, B, Hq, Hkv, n_qt);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int grp = wave >> 2;  // 0: matrix cores first, issues the tile loads; 1: softmax first
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
  // Wait for Q (and the descales) here, once: the tile loads are asm the
  // compiler does not count, so a wait it placed inside the loop would also
  // wait for them.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

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
  // interleaved. All A operands of the phase are read from LDS first; ex(n)
  // runs after the n-th MFMA.
  auto mma_t = [&](auto do_o_t, auto do_s_t, int jo, int js, const auto& ex) {
    constexpr bool DO_O = decltype(do_o_t)::value, DO_S = decltype(do_s_t)::value;
    const char* vl = vring + (jo % kSlots) * kTile;
    const char* kl = kring + (js % kSlots) * kTile;
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
    int n = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (DO_O) {
        acc_o[t] = mfma_f8(ao[t], bp, acc_o[t]);
        ex(n++);
      }
      if constexpr (DO_S) {
        s[t & 1] = mfma_f8(as[t], qop[t >> 1], s[t & 1]);
        ex(n++);
      }
    }
  };
  auto mma = [&](bool do_o, int jo, bool do_s, int js) {
    if (do_o && do_s)
      mma_t(std::true_type{}, std::true_type{}, jo, js, NoDma{});
    else if (do_o)
      mma_t(std::true_type{}, std::false_type{}, jo, js, NoDma{});
    else if (do_s)
      mma_t(std::false_type{}, std::true_type{}, jo, js, NoDma{});
  };

  // ---- direct-to-LDS tile loads, issued by the waves of group 0 only (they
  // wait at the step barrier anyway): 2 instructions per wave per tile.
  const uint32_t lds_k = (uint32_t)(uintptr_t)(lds_void_t*)kring;
  const uint32_t lds_v = (uint32_t)(uintptr_t)(lds_void_t*)vring;
  const int wg = wv & 3;  // wave index within its group
  const uint32_t dk = dma_src<false>(0, wg, lane, kRows);  // source offsets of a full tile
  const uint32_t dv = dma_src<true>(0, wg, lane, kRows);
  auto issue = [&](bool is_v, int t) {
    const int nvalid = min(kRows, Nk - t * kRows);
    const uint8_t* base = (is_v ? vp : kp) + (size_t)t * kRows * kD;
    const uint32_t slot = (is_v ? lds_v : lds_k) + (uint32_t)((t % kSlots) * kTile) + (uint32_t)(64 * wg * 16);
    if (nvalid == kRows) {
      dma16(base, is_v ? dv : dk, slot);
      dma16(base + 32 * kD, is_v ? dv : dk, slot + 4096);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(base, is_v ? dma_src<true>(i, wg, lane, nvalid) : dma_src<false>(i, wg, lane, nvalid), slot + 4096 * i);
    }
  };
  // Loads issued at the start of step i: K_{i+2} and V_{i+1}; returns the
  // number of load instructions this thread issued (wave-uniform).
  auto issue_step = [&](int i) -> int {
    int n = 0;
    if (grp == 0) {
      if (i + 2 < n_kv) {
        issue(false, i + 2);
        n += 2;
      }
      if (i + 1 < n_kv) {
        issue(true, i + 1);
        n += 2;
      }
    }
    return n;
  };

  // Prologue: K_0 (read first), then K_1 and V_0 (the loads of "step -1").
  if (grp == 0 && 0 < n_kv) issue(false, 0);
  dma_barrier(issue_step(-1));  // K_0 has landed

  // Step i = phase A, barrier Y_i, phase B (the schedule of the 16-bit
  // kernel):
  //   group 0: A = O(i-1), S(i), loads K_{i+2}, V_{i+1}   B = softmax(i)
  //   group 1: A = softmax(i-1)                           B = O(i-1), S(i)
  // Y_i waits for the loads issued in step i - 1 (K_{i+1}, V_i). Between Y_i
  // and Y_{i+1} the waves read K_i, K_{i+1}, V_{i-1} and V_i, while the loads
  // in flight write K_{i+2}, K_{i+3}, V_{i+1} and V_{i+2}: distinct slots.
  if (grp == 0) {
    for (int i = 0; i <= n_kv; ++i) {
      const bool do_o = i >= 1 && i - 1 < wt, do_s = i < wt;
      const bool has_k = i + 2 < n_kv, has_v = i + 1 < n_kv;
      int n_new = 2 * has_k + 2 * has_v;
      if (ALIGNED && do_o && do_s) {
        // all 4 loads; a missing K_{i+2} / V_{i+1} re-reads tile 0
        const DmaSpread<true> ex{has_k ? kp + (size_t)(i + 2) * kRows * kD : kp,
                                 has_v ? vp + (size_t)(i + 1) * kRows * kD : vp,
                                 lds_k + (uint32_t)(((i + 2) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
                                 lds_v + (uint32_t)(((i + 1) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
                                 true, true, dk, dv};
        mma_t(std::true_type{}, std::true_type{}, i - 1, i, ex);
        n_new = 4;
      } else if (do_o && do_s) {
        // full phase: with full tiles the loads are spread over its MFMAs
        const bool spread = (!has_k || Nk - (i + 2) * kRows >= kRows) && (!has_v || Nk - (i + 1) * kRows >= kRows);
        if (!spread) issue_step(i);
        const DmaSpread<> ex{kp + (size_t)(i + 2) * kRows * kD, vp + (size_t)(i + 1) * kRows * kD,
                           lds_k + (uint32_t)(((i + 2) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
                           lds_v + (uint32_t)(((i + 1) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
                           has_k && spread, has_v && spread, dk, dv};
        mma_t(std::true_type{}, std::true_type{}, i - 1, i, ex);
      } else {
        issue_step(i);
        mma(do_o, i - 1, do_s, i);
      }
      dma_barrier(n_new);  // Y_i
      if (i < wt) softmax(i);
    }
  } else {
    for (int i = 0; i <= n_kv; ++i) {
      const int n_new = issue_step(i);
      if (i >= 1 && i - 1 < wt) softmax(i - 1);
      dma_barrier(n_new);  // Y_i
      mma(i >= 1 && i - 1 < wt, i - 1, i < wt, i);
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
  if (a.Nk % kRows == 0)
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<CAUSAL, true>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream, a.q, a.k,
                       a.v, (uint16_t*)a.o, a.lse, a.q_descale, a.k_descale, a.v_descale, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.scale * kLog2e, n_qt);
  else
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<CAUSAL, false>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream, a.q, a.k,
                       a.v, (uint16_t*)a.o, a.lse, a.q_descale, a.k_descale, a.v_descale, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.scale * kLog2e, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
  return a.causal ? launch_t<true>(a, stream) : launch_t<false>(a, stream);
}

}  // namespace fa
