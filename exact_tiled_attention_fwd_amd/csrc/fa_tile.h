// fa_tile.h - gfx950 device building blocks shared by the prefill and decode
// kernels: the matrix-core (MFMA) phase of a tile pair, the online-softmax
// step, the per-lane reductions and the prefill work order.
//
// The arithmetic follows "Flash Attention: Revolutionizing Transformer
// Efficiency" (unite.ai), sections "The math of Flash Attention" (subtract the
// running maximum; merge partial softmaxes by rescaling with exp(m_old-m_new))
// and "Implementation details" (running max M and running sum L per query
// row). The output accumulator is kept unnormalised and divided by the row
// sum once at the end (FlashAttention-2's deferred normalisation).
//
// Orientation. Both products run on the 32x32x16 MFMA with the contraction
// index contiguous in each lane:
//   S^T[key][query] = K[key][:] . Q[query][:]          (A = K tile, B = Q^T)
//   O^T[d][query]  += V^T[d][key] . P^T[key][query]    (A = V^T tile, B = P^T)
// The S^T accumulator holds, in lane l, query column l%32 and 16 keys, so the
// per-query max and sum are lane-local up to one exchange with lane l^32, and
// the accumulator registers are already the B operand of the second product
// once rounded to 16 bits; the V^T operand is gathered from row-major V with
// transposed LDS reads in the key order of that accumulator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "fa_launch.h"  // Layout

namespace fa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum { DT_BF16 = 0, DT_FP16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// MFMA counts of one tile pair of ROWS keys at head width D.
template <int D, int ROWS>
struct Tile {
  static_assert(D == 64 || D == 128, "head width");
  static_assert(ROWS % 32 == 0, "tile rows");
  static constexpr int KB = ROWS / 32;  // 32-key blocks
  static constexpr int KS = D / 16;     // MFMA k-steps over d
  static constexpr int MT = D / 32;     // 32-row blocks of O^T
};

// ------------------------------------------------------------------ MFMA
template <int DT>
__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round two fp32 to the 16-bit type (nearest-even), packed low/high.
template <int DT>
__device__ inline uint32_t pack2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  if constexpr (DT == DT_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Matrix-core phase of one wave on one tile pair: optionally O^T += V^T P^T
// for the previous tile (DO_O) and S^T = K Q^T for the current one (DO_S),
// the O operations first. The A operands come from LDS through a ring of
// kPF registers, fetched kPF MFMAs ahead; mma_prefetch issues the first kPF
// reads (it may run before the barrier that opens the phase when those tiles
// are already complete), mma_run does the rest.
constexpr int kPF = 4;

// RD (the operand reader) supplies k(kl, kb, ks, lane) and vt(vl, mt, G, lane),
// VT_READS (LDS reads per V^T operand) and INTERLEAVE.
template <int D, int ROWS, bool DO_O, bool DO_S, class RD>
struct MmaPlan {
  using T = Tile<D, ROWS>;
  static constexpr int NO = DO_O ? T::KB * 2 * T::MT : 0;
  static constexpr int NS = DO_S ? T::KS * T::KB : 0;
  static constexpr int N = NO + NS;
  static_assert(N >= kPF, "pipeline depth");
  // With both products in the phase and a reader that asks for it, O and S
  // ops alternate (spreading the reads of the slower operand); otherwise the
  // O ops come first.
  static constexpr bool ALT = RD::INTERLEAVE && DO_O && DO_S && NO == NS;
  __device__ static constexpr bool is_o(int t) { return ALT ? (t & 1) == 0 : t < NO; }
  __device__ static constexpr int idx(int t) { return ALT ? t >> 1 : (t < NO ? t : t - NO); }
  // O op i: P block kb, 16-key half u, O^T row block mt (mt fastest).
  __device__ static inline void o_op(int i, int& kb, int& u, int& mt) {
    kb = i / (2 * T::MT);
    u = (i / T::MT) % 2;
    mt = i % T::MT;
  }
  // S op i: d step ks, key block kb (kb fastest).
  __device__ static inline void s_op(int i, int& ks, int& kb) {
    ks = i / T::KB;
    kb = i % T::KB;
  }
  __device__ static inline u32x4 read(const char* __restrict__ vl, const char* __restrict__ kl, int t, int lane) {
    if (is_o(t)) {
      int kb, u, mt;
      o_op(idx(t), kb, u, mt);
      return RD::vt(vl, mt, 2 * kb + u, lane);
    }
    int ks, kb;
    s_op(idx(t), ks, kb);
    return RD::k(kl, kb, ks, lane);
  }
};

template <int D, int ROWS, bool DO_O, bool DO_S, class RD>
__device__ __attribute__((always_inline)) inline void mma_prefetch(u32x4 (&buf)[kPF], const char* __restrict__ vl, const char* __restrict__ kl,
                                    int lane) {
#pragma unroll
  for (int t = 0; t < kPF; ++t) buf[t] = MmaPlan<D, ROWS, DO_O, DO_S, RD>::read(vl, kl, t, lane);
}

// Work slotted in after each MFMA of a phase (called with the op index), or
// between the exponentials of a softmax step; all() does all of it at once.
struct NoExtra {
  __device__ void operator()(int) const {}
  __device__ void all() const {}
};

template <int DT, int D, int ROWS, bool DO_O, bool DO_S, class RD, class EX = NoExtra>
__device__ __attribute__((always_inline)) inline void mma_run(u32x4 (&buf)[kPF], const char* __restrict__ vl, const char* __restrict__ kl,
                               const uint32_t (&pk)[ROWS / 32][8], const u32x4 (&qop)[D / 16],
                               f32x16 (&acc_o)[D / 32], f32x16 (&s)[ROWS / 32], int lane, const EX& ex = EX{}) {
  using P = MmaPlan<D, ROWS, DO_O, DO_S, RD>;
  using T = Tile<D, ROWS>;
  if constexpr (DO_S) {
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < P::N; ++t) {
    const u32x4 a = buf[t % kPF];
    if (t + kPF < P::N) buf[t % kPF] = P::read(vl, kl, t + kPF, lane);
    if (P::is_o(t)) {
      int kb, u, mt;
      P::o_op(P::idx(t), kb, u, mt);
      const u32x4 b = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
      acc_o[mt] = mfma32<DT>(a, b, acc_o[mt]);
    } else {
      int ks, kb;
      P::s_op(P::idx(t), ks, kb);
      s[kb] = mfma32<DT>(a, qop[ks], s[kb]);
    }
    ex(t);
  }
  // Keep the issue order: (MFMA, next operand's reads) pairs, then the tail
  // MFMAs.
#pragma unroll
  for (int t = 0; t < P::N; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (t + kPF < P::N) {
      if (P::is_o(t + kPF))
        __builtin_amdgcn_sched_group_barrier(0x100, RD::VT_READS, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
}

// max / sum of x over lanes l and l^32. v_permlane32_swap(x, x) returns, in
// every lane, the pair {x[l & 31], x[(l & 31) + 32]}.
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key offset (within a 32-key block) of accumulator register r in lane half h.
__device__ inline int acc_key(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Reference-point rule of the online softmax. Any common shift m gives the
// same exact result (the merge identity of "The math of Flash Attention",
// unite.ai, holds for any shift), so m only has to keep the exponentials in
// range. A tile is first exponentiated against the current m with no
// maximum taken; only when some lane's sum of those exponentials leaves
// (0, limit] (or m is still -inf: the row's first tile) is the tile's row
// maximum taken, m moved to it, the running sum and the output accumulator
// rescaled by exp(m_old - m_new), and the tile exponentiated again. Every p
// is then at most the limit, so nothing overflows and a 16-bit P keeps its
// relative precision at any magnitude. The limit is 2^16 for bf16 and 2^15
// for fp16, whose largest finite value (65504) is below 2^16: a P just under
// 2^16 would round to infinity.
template <int DT>
constexpr float sum_limit() {
  return DT == DT_FP16 ? 32768.f : 65536.f;
}

// Exponentiates NS 32-key blocks of S^T (raw scores, masked entries -inf)
// against the reference m_use (log2 units): P = exp2(c s - m_use) with
// c = scale*log2(e), rounded to the input type and packed two per register
// in accumulator order into pk. Returns this lane's sum of the unrounded P.
// ex(i) is called once per pair of exponentials (i = 0 .. 8 NS - 1).
template <int DT, int NS, class EX = NoExtra>
__device__ __attribute__((always_inline)) inline float exp_tile(const f32x16 (&s)[NS], float c, float m_use,
                                                                 uint32_t (&pk)[NS][8], const EX& ex = EX{}) {
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NS; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2_fast(__builtin_fmaf(s[kb][r], c, -m_use));
      const float p1 = exp2_fast(__builtin_fmaf(s[kb][r + 1], c, -m_use));
      psum += p0 + p1;
      pk[kb][r >> 1] = pack2<DT>(p0, p1);
      ex(8 * kb + (r >> 1));
    }
  return psum;
}

// The slow branch of the rule: take the tile's row maximum, move the
// reference to it, rescale the running sum and the accumulator by
// exp2(m_old - m_new), and exponentiate the tile again. Returns the new sum.
template <int DT, int NS, int MT>
__device__ __attribute__((always_inline)) inline float move_reference(const f32x16 (&s)[NS], float c, float& m_run,
                                                                      float& l_run, f32x16 (&acc_o)[MT],
                                                                      uint32_t (&pk)[NS][8]) {
  float mx = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < NS; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = halves_max(mx) * c;
  const float m_new = fmaxf(m_run, mx);
  const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2_fast(m_run - m_new);
  l_run *= alpha;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;
  m_run = m_new;
  return exp_tile<DT, NS>(s, c, (m_new == -__builtin_inff()) ? 0.f : m_new, pk);
}

// One online-softmax step over NS 32-key blocks of S^T. Updates the row
// reference m_run (per lane = per query column), this lane's share of the
// running sum l_run, rescales acc_o when m_run moves, and leaves P in pk.
// ex(i) is called once per pair of exponentials of the pass against the
// current reference point; a row's first tile, which has no such pass,
// calls ex.all() instead.
template <int DT, int NS, int MT, class EX = NoExtra>
__device__ __attribute__((always_inline)) inline void softmax_step(f32x16 (&s)[NS], float c, float& m_run,
                                                                   float& l_run, f32x16 (&acc_o)[MT],
                                                                   uint32_t (&pk)[NS][8], const EX& ex = EX{}) {
  float psum = 0.f;
  bool slow = __builtin_amdgcn_ballot_w64(m_run == -__builtin_inff()) != 0;
  if (slow) {
    ex.all();
  } else {
    psum = exp_tile<DT, NS>(s, c, m_run, pk, ex);
    slow = __builtin_amdgcn_ballot_w64(!(psum <= sum_limit<DT>())) != 0;
  }
  if (slow) psum = move_reference<DT, NS, MT>(s, c, m_run, l_run, acc_o, pk);
  l_run += psum;
}

// ------------------------------------------------------------------ work order
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

// Work order for packed batches, where a later query tile is not in general
// a heavier one: sequence-major, so that one (sequence, kv-head) pair's K/V
// is read by all its query tiles and q-heads while it sits in L2; query
// tiles of a sequence heaviest first. When Hkv is a multiple of 8, XCD x
// (workgroup ids L with L % 8 == x) serves the kv-heads g with g % 8 == x.
__device__ inline Work map_work_packed(int L, int B, int Hq, int Hkv, int n_qt) {
  const int grp = Hq / Hkv;
  const int per_pair = n_qt * grp;
  int s = L, x = 0, gstride = 1, goff = 0, gper = Hkv;
  if ((Hkv & 7) == 0) {
    x = L & 7;
    s = L >> 3;
    gstride = 8;
    goff = x;
    gper = Hkv >> 3;
  }
  const int p = s / per_pair, rem = s % per_pair;
  Work w;
  w.b = p / gper;
  w.g = (p % gper) * gstride + goff;
  w.qt = n_qt - 1 - rem / grp;
  w.h = w.g * grp + rem % grp;
  return w;
}

// ------------------------------------------------------------------ slabs
// Packed variable-length batches: sequence b's query rows are rows
// [cu_q[b], cu_q[b+1]) of each head's [total_q, d] slab, its keys rows
// [cu_k[b], cu_k[b+1]) of each kv-head's [total_k, d] slab.
struct Varlen {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
};

// The slabs one workgroup reads and writes, with their row counts and row
// strides (elements).
struct Slabs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;  // null: not written
  int Nq, Nk;
  int qs, ks, vs, os;
};

// Fixed layout: row i of (b, h) of q at q + b ly.q[0] + h ly.q[1] + i ly.q[2]
// (likewise k, v with the kv-head, and o); lse [B, Hq, Nq].
// Packed layout: token t of head h at q + h ly.q[1] + t ly.q[2]; lse
// [Hq, total_q]. Offsets are clamped into [0, total] and made non-decreasing,
// so no offset array, however wrong, leads outside the tensors.
template <bool VARLEN>
__device__ inline Slabs slabs_of(const Work& w, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                 float* lse, int Hq, int Nq, int Nk, const Varlen& vl, const Layout& ly) {
  Slabs s;
  if constexpr (VARLEN) {
    const int q_lo = min(max(vl.cu_q[w.b], 0), vl.total_q);
    const int q_hi = min(max(vl.cu_q[w.b + 1], q_lo), vl.total_q);
    const int k_lo = min(max(vl.cu_k[w.b], 0), vl.total_k);
    const int k_hi = min(max(vl.cu_k[w.b + 1], k_lo), vl.total_k);
    s.q = q + w.h * ly.q[1] + q_lo * ly.q[2];
    s.o = o + w.h * ly.o[1] + q_lo * ly.o[2];
    s.lse = lse ? lse + (size_t)w.h * vl.total_q + q_lo : nullptr;
    s.k = k + w.g * ly.k[1] + k_lo * ly.k[2];
    s.v = v + w.g * ly.v[1] + k_lo * ly.v[2];
    s.Nq = q_hi - q_lo;
    s.Nk = k_hi - k_lo;
  } else {
    s.q = q + w.b * ly.q[0] + w.h * ly.q[1];
    s.o = o + w.b * ly.o[0] + w.h * ly.o[1];
    s.lse = lse ? lse + ((size_t)w.b * Hq + w.h) * Nq : nullptr;
    s.k = k + w.b * ly.k[0] + w.g * ly.k[1];
    s.v = v + w.b * ly.v[0] + w.g * ly.v[1];
    s.Nq = Nq;
    s.Nk = Nk;
  }
  s.qs = (int)ly.q[2];
  s.ks = (int)ly.k[2];
  s.vs = (int)ly.v[2];
  s.os = (int)ly.o[2];
  return s;
}

}  // namespace fa
