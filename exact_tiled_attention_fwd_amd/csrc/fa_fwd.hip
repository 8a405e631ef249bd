// fa_fwd.hip - prefill attention forward for gfx950, head width 128 or 64.
//
// One workgroup owns 256 query rows of one (batch, q-head): 8 waves of 32
// rows in two groups of 4 that alternate between matrix-core phases and
// online-softmax phases, Q-outer and K/V-inner ("Implementation details",
// "Flash Attention: Revolutionizing Transformer Efficiency", unite.ai; the
// merge identity of "The math of Flash Attention" on the same page). Key
// tiles are 16 KiB: 64 keys at d = 128, 128 keys at d = 64.
//
// The waves of one group move each K and V tile HBM -> LDS directly
// (global_load_lds_dwordx4: no staging registers, no LDS store instructions,
// no vector-ALU work), into 4-slot rings issued two tiles (K) and one tile
// (V) ahead of the step that reads them; the fourth slot lets one barrier per
// step order both the loads and the reuse of slots. V stays row-major in LDS
// and is read transposed (ds_read_b64_tr_b16) as the A operand of
// O^T += V^T P^T, so no lane shuffles are needed anywhere. The vector ALUs are
// left to the softmax.
#include <atomic>

#include "fa.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = kFwdBlockRows;  // 256 query rows per workgroup
constexpr int kBMs = 128;           // query rows per item in split mode
constexpr int kThreads = 512;       // 8 waves = 2 groups of 4
constexpr int kSlots = 4;           // ring depth for K and for V

// Tile geometry for head width D: 16 KiB K or V tiles (64 keys at D = 128,
// 128 keys at D = 64), D / 8 chunks of 16 bytes per row, 256 / (D / 8) rows
// per block of 256 chunk positions (one load instruction of each of the 4
// loading waves).
template <int D>
struct Geo {
  static constexpr int ROWS = 8192 / D;
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 256 / CPR;
  static constexpr int TILE = ROWS * D * 2;
};

// LDS layouts, row-major [ROWS][D] 16-bit:
//   D = 128 (256-byte rows, 16 chunks): K chunk c of row r at c ^ (r % 16),
//     so the 16 rows of a quarter-wave A-operand fetch of one chunk column
//     land on distinct banks; V chunk c at c ^ 4 (r % 4), conflict-free
//     transposed reads (a half-wave reads 4 rows x 4 chunks).
//   D = 64 (128-byte rows, 8 chunks; rows r and r + 2 share banks): K chunk
//     c at c ^ ((r / 2) % 8); V chunk c at c ^ 4 ((r / 2) % 2), which puts the
//     4 rows x 4 chunks of a half-wave transposed read on distinct banks.
template <int D>
__device__ inline int k_phys(int row, int c) {
  return D == 128 ? c ^ (row & 15) : c ^ ((row >> 1) & 7);
}
template <int D>
__device__ inline int v_phys(int row, int c) {
  return D == 128 ? c ^ (4 * (row & 3)) : c ^ (4 * ((row >> 1) & 1));
}

// Byte offset in the global tile (rows rsb bytes apart) of the 16-byte chunk
// that load instruction i (0..3) of wave w (0..3 of the loading group)
// writes to LDS position p = 256 i + 64 w + lane (row p / CPR, position
// p % CPR). The swizzles are involutions, so position -> chunk uses the same
// map. Rows at or beyond nvalid re-read row nvalid - 1: their scores are
// masked to -inf and contribute exactly 0. For a full tile the offset of
// instruction i is that of instruction 0 plus RPI i rows (the swizzles depend
// on the row only through row % 16), so one offset register serves all four.
template <int D, bool IS_V>
__device__ inline uint32_t dma_src(int i, int w, int lane, int nvalid, uint32_t rsb) {
  constexpr int CPR = Geo<D>::CPR;
  const int p = 256 * i + 64 * w + lane;
  const int row = p / CPR, pos = p % CPR;
  const int c = IS_V ? v_phys<D>(row, pos) : k_phys<D>(row, pos);
  return (uint32_t)min(row, nvalid - 1) * rsb + (uint32_t)(c * 16);
}

// One 1 KiB direct-to-LDS load: lane l's 16 bytes from sbase + voff land at
// LDS address lds + 16 l. Written as asm so that the compiler's wait
// insertion, which cannot tell the ring slots apart, does not wait for every
// load in flight before each LDS read; the phase barriers do the waiting.
// m0 carries the LDS address; it is listed as clobbered (the compiler warns
// that m0 is reserved), and no other instruction of these kernels reads or
// writes m0 (their assembly has no other m0 reference).
__device__ __attribute__((always_inline)) inline void dma16(const uint16_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Barrier that first waits until this thread has at most `pending` (0, 4 or
// 8, wave-uniform) direct-to-LDS loads outstanding. No release fence: it
// would also wait for the loads that are meant to stay in flight.
__device__ __attribute__((always_inline)) inline void dma_barrier(int pending) {
  pending = __builtin_amdgcn_readfirstlane(pending);  // wave-uniform: scalar branches
  if (pending >= 8)
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
  else if (pending >= 4)
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Operand reader of the layouts above. K: one 16-byte read per lane (row
// 32 kb + lane % 32, chunk 2 ks + lane / 32). V^T: two transposed reads; lane
// l gets V[16 G + 8 p + 4 h + e][32 mt + l % 32] for e = 0..3, p = 0, 1
// (h = l / 32), which is the key order of the P accumulator.
template <int D>
struct DmaReader {
  static constexpr int VT_READS = 2;
  static constexpr bool INTERLEAVE = true;  // transposed reads are slower per wave: spread them
  __device__ static inline u32x4 k(const char* __restrict__ kl, int kb, int ks, int lane) {
    const int row = 32 * kb + (lane & 31);
    return *reinterpret_cast<const u32x4*>(kl + row * (2 * D) + k_phys<D>(row, 2 * ks + (lane >> 5)) * 16);
  }
  __device__ static inline u32x4 vt(const char* __restrict__ vl, int mt, int G, int lane) {
    const int gi = lane >> 4, e = (lane >> 2) & 3, qq = lane & 3;
    const int h = gi >> 1, dh = gi & 1;
    const int c = 4 * mt + 2 * dh + (qq >> 1);
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int row = 16 * G + 8 * p + 4 * h + e;
      const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(vl + row * (2 * D) + v_phys<D>(row, c) * 16 + 8 * (qq & 1)));
      const u32x2 w = __builtin_bit_cast(u32x2, t);
      out[2 * p] = w[0];
      out[2 * p + 1] = w[1];
    }
    return out;
  }
};

// The 8 tile loads of one step, slotted in after every (N / 8)-th MFMA of an
// N-op matrix-core phase (MFMAs 2, 6, ..., 30 of 32; 1, 3, ..., 15 of 16), so
// that the loads of the four loading waves reach the address unit a few at a
// time instead of in one burst. Full tiles only. With ALWAYS the loads are
// issued unconditionally (no branch splits the phase): the caller points a
// tile that does not exist at tile 0 and its ring slot, which no wave reads.
template <int N, bool ALWAYS = false>
struct DmaSpread {
  const uint16_t* kbase;
  const uint16_t* vbase;
  uint32_t kslot, vslot;
  bool has_k, has_v;
  uint32_t dk, dv;
  long long kstep, vstep;  // RPI rows, in elements
  __device__ __attribute__((always_inline)) void operator()(int t) const {
    constexpr int ST = N / 8;
    static_assert(ST * 8 == N, "phase length");
    if (t % ST != ST / 2) return;
    const int j = t / ST;
    if (j < 4) {
      if (ALWAYS || has_k) dma16(kbase + kstep * j, dk, kslot + 4096 * j);
    } else {
      if (ALWAYS || has_v) dma16(vbase + vstep * (j - 4), dv, vslot + 4096 * (j - 4));
    }
  }
};

// Split mode (causal grids too small to fill the GPU): a workgroup takes the
// 128-row blocks nb - 1 - qt and qt of one head in turn, so every workgroup
// has the same number of visible keys. Waves w and w + 4 hold the same 32
// query rows and the two groups take the two halves of every key tile; at
// the end of a block the halves are joined by the merge identity of "The
// math of Flash Attention" through LDS. Tiles, ring and loads are those of
// the 256-row mode; the second block's Q and first K and V tiles are loaded
// while the first is joined and written.
// ALIGNED: every key tile is full (Nk a multiple of the tile rows), so the
// loads of a full matrix-core phase need no branch.
template <int DT, int D, bool CAUSAL, bool VARLEN, bool SPLIT, bool ALIGNED>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int Nq_all, int Nk_all,
    float scale_log2, int n_qt, Varlen vlen, Layout ly) {
  constexpr int ROWS = Geo<D>::ROWS, kTile = Geo<D>::TILE, RPI = Geo<D>::RPI;
  static_assert(!SPLIT || (CAUSAL && !VARLEN), "split mode serves causal, unpacked grids");
  constexpr int WR = SPLIT ? ROWS / 2 : ROWS;  // keys of a tile one wave multiplies
  constexpr int KS = D / 16, KB = WR / 32, MT = D / 32;
  using Rd = DmaReader<D>;
  // Split mode joins the key halves through LDS from V slot 1 on (16 MT + 2
  // floats per lane), so that K slots 0, 1 and V slot 0 can take the next
  // block's first tiles meanwhile.
  constexpr int XW = 16 * MT + 2;
  constexpr int kXOff = (kSlots + 1) * kTile;
  constexpr int kSmem = SPLIT && kXOff + 4 * XW * 64 * 4 > 2 * kSlots * kTile ? kXOff + 4 * XW * 64 * 4
                                                                             : 2 * kSlots * kTile;
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  char* const kring = smem;                   // K tile t in slot t % 4
  char* const vring = smem + kSlots * kTile;  // V tile t in slot t % 4

  const Work wk = VARLEN ? map_work_packed(blockIdx.x, B, Hq, Hkv, n_qt) : map_work(blockIdx.x, B, Hq, Hkv, n_qt);
  const Slabs sl = slabs_of<VARLEN>(wk, q, k, v, o, lse, Hq, Nq_all, Nk_all, vlen, ly);
  const int Nq = sl.Nq, Nk = sl.Nk;
  const int nb = (Nq + kBMs - 1) / kBMs;
  const int n_items = SPLIT && nb - 1 - wk.qt > wk.qt ? 2 : 1;
  u32x4 qop[KS];  // Q^T operand (B operand of S^T = K Q^T), held for a whole block
  for (int item = 0; item < n_items; ++item) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int grp = wave >> 2;  // 0: matrix cores first; 1: softmax first
    // Q^T of the rows from q0x on
    auto load_q = [&](int q0x) {
      const int qr = q0x + 32 * (SPLIT ? (wave & 3) : wave) + (lane & 31);
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (qr < Nq)
          qop[ks] = *reinterpret_cast<const u32x4*>(sl.q + (size_t)qr * sl.qs + 16 * ks + 8 * half);
        else
          qop[ks] = u32x4{0u, 0u, 0u, 0u};
      }
    };
    const int q0 = SPLIT ? kBMs * (item == 0 ? nb - 1 - wk.qt : wk.qt) : wk.qt * kBM;
    if (VARLEN && q0 >= Nq) return;  // past this sequence's rows (the whole workgroup)
    // The second block of split mode has its Q and first tiles in flight
    // since the end of the first.
    const bool prefetched = SPLIT && item > 0;
    const int q0w = q0 + 32 * (SPLIT ? (wave & 3) : wave);  // first query row of this wave
    const int off = Nk - Nq;         // causal: key j visible to query i iff j <= i + off
    const int key0 = SPLIT ? grp * WR : 0;            // first key of a tile this wave multiplies
    const uint32_t koff = (uint32_t)(key0 * 2 * D);  // its byte offset in a ring slot

    const uint16_t* kp = sl.k;
    const uint16_t* vp = sl.v;

    // Key tiles this workgroup visits (none for rows that see no key).
    int n_kv = (Nk + ROWS - 1) / ROWS;
    if (CAUSAL) {
      const int last_key = min(q0 + (SPLIT ? kBMs : kBM), Nq) - 1 + off;
      n_kv = last_key < 0 ? 0 : min(n_kv, last_key / ROWS + 1);
    }
    // Key tiles this wave computes on (0 if the wave has no valid query row).
    const bool wave_active = q0w < Nq;
    int wave_tiles = wave_active ? n_kv : 0;
    if (CAUSAL && wave_active) {
      const int last = min(q0w + 31, Nq - 1) + off;
      wave_tiles = last < key0 ? 0 : min(n_kv, (last - key0) / ROWS + 1);
    }

    const int qrow = q0w + (lane & 31);
    if (!prefetched) load_q(q0);
    // Wait for Q here, once: the tile loads are asm the compiler does not count,
    // so a Q wait it placed inside the loop would also wait for them.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    f32x16 acc_o[MT];
  #pragma unroll
    for (int mt = 0; mt < MT; ++mt)
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;
    float m_run = -__builtin_inff();  // row reference point, log2 units
    float l_run = 0.f;                // this lane's share of the running sum
    f32x16 s[KB];                     // S^T of the tile last multiplied
    uint32_t pk[KB][8];               // P of the tile last softmaxed

    // SM(j): mask the ragged key tail / causal diagonal, online softmax -> pk.
    auto softmax = [&](int j) {
      const int j0 = j * ROWS + key0;
      const bool need_mask = (j0 + WR > Nk) || (CAUSAL && j0 + WR - 1 > q0w + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(Nk, qrow + off + 1) : Nk;  // keys < lim are visible
  #pragma unroll
        for (int kb = 0; kb < KB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r)
            if (j0 + 32 * kb + acc_key(r, half) >= lim) s[kb][r] = -__builtin_inff();
      }
      softmax_step<DT, KB, MT>(s, scale_log2, m_run, l_run, acc_o, pk);
    };
    // Matrix-core phase: MB(jo) = O^T += V^T_jo P^T (if do_o), MA(js) = S^T = K_js Q^T (if do_s).
    // mma_pre issues the first operand reads; mma finishes the phase.
    u32x4 obuf[kPF];
    auto mma_pre = [&](bool do_o, int jo, bool do_s, int js) {
      const char* vl = vring + (jo % kSlots) * kTile + koff;
      const char* kl = kring + (js % kSlots) * kTile + koff;
      if (do_o && do_s)
        mma_prefetch<D, WR, true, true, Rd>(obuf, vl, kl, lane);
      else if (do_o)
        mma_prefetch<D, WR, true, false, Rd>(obuf, vl, kl, lane);
      else if (do_s)
        mma_prefetch<D, WR, false, true, Rd>(obuf, vl, kl, lane);
    };
    auto mma = [&](bool do_o, int jo, bool do_s, int js) {
      const char* vl = vring + (jo % kSlots) * kTile + koff;
      const char* kl = kring + (js % kSlots) * kTile + koff;
      if (do_o && do_s)
        mma_run<DT, D, WR, true, true, Rd>(obuf, vl, kl, pk, qop, acc_o, s, lane);
      else if (do_o)
        mma_run<DT, D, WR, true, false, Rd>(obuf, vl, kl, pk, qop, acc_o, s, lane);
      else if (do_s)
        mma_run<DT, D, WR, false, true, Rd>(obuf, vl, kl, pk, qop, acc_o, s, lane);
    };

    // ---- direct-to-LDS tile loads, issued by the waves of group 0 only (they
    // wait at the Y barrier anyway): 4 instructions per wave per tile.
    const uint32_t lds_k = (uint32_t)(uintptr_t)(lds_void_t*)kring;
    const uint32_t lds_v = (uint32_t)(uintptr_t)(lds_void_t*)vring;
    const int wg = wv & 3;  // wave index within its group
    const uint32_t ksb = 2u * (uint32_t)sl.ks, vsb = 2u * (uint32_t)sl.vs;  // row strides in bytes
    const uint32_t dk = dma_src<D, false>(0, wg, lane, ROWS, ksb);  // source offsets of a full tile
    const uint32_t dv = dma_src<D, true>(0, wg, lane, ROWS, vsb);
    const long long kstep = (long long)RPI * sl.ks, vstep = (long long)RPI * sl.vs;
    auto issue = [&](bool is_v, int t) {
      const int nvalid = min(ROWS, Nk - t * ROWS);
      const uint16_t* base = is_v ? vp + (long long)t * ROWS * sl.vs : kp + (long long)t * ROWS * sl.ks;
      const uint32_t slot = (is_v ? lds_v : lds_k) + (uint32_t)((t % kSlots) * kTile) + (uint32_t)(64 * wg * 16);
      if (nvalid == ROWS) {
  #pragma unroll
        for (int i = 0; i < 4; ++i) dma16(base + (is_v ? vstep : kstep) * i, is_v ? dv : dk, slot + 4096 * i);
      } else {
  #pragma unroll
        for (int i = 0; i < 4; ++i)
          dma16(base, is_v ? dma_src<D, true>(i, wg, lane, nvalid, vsb) : dma_src<D, false>(i, wg, lane, nvalid, ksb),
                slot + 4096 * i);
      }
    };
    // Loads issued at the start of step i: K_{i+2} and V_{i+1}; returns the
    // number of load instructions this thread issued (wave-uniform).
    auto issue_step = [&](int i) -> int {
      int n = 0;
      if (grp == 0) {
        if (i + 2 < n_kv) {
          issue(false, i + 2);
          n += 4;
        }
        if (i + 1 < n_kv) {
          issue(true, i + 1);
          n += 4;
        }
      }
      return n;
    };

    // Prologue: K_0 (read first), then K_1 and V_0 (the loads of "step -1").
    if (prefetched) {
      dma_barrier(0);  // K_0, K_1, V_0 (waited for with Q above)
    } else {
      if (grp == 0 && 0 < n_kv) issue(false, 0);
      dma_barrier(issue_step(-1));  // K_0 has landed
    }

    // Step i = phase A, barrier Y_i, phase B; Y_i is the step's only barrier:
    //   group 0: A = MB(i-1), MA(i), loads K_{i+2}, V_{i+1}   B = SM(i), first reads of MB(i), MA(i+1)
    //   group 1: A = SM(i-1), first reads of MB(i-1), MA(i)  B = MB(i-1), MA(i)
    // Y_i waits for the loads issued in step i - 1 (K_{i+1}, V_i). Between Y_i
    // and Y_{i+1} the waves read K_i, K_{i+1}, V_{i-1} and V_i, while the loads
    // in flight write K_{i+2}, K_{i+3}, V_{i+1} and V_{i+2}: distinct slots of
    // the 4-slot rings. A slot is rewritten only after the barrier that follows
    // the MFMAs consuming its last reads.
    if (grp == 0) {
      mma_pre(false, 0, 0 < wave_tiles, 0);
      for (int i = 0; i <= n_kv; ++i) {
        const bool do_o = i >= 1 && i - 1 < wave_tiles, do_s = i < wave_tiles;
        const bool has_k = i + 2 < n_kv, has_v = i + 1 < n_kv;
        int n_new = 4 * has_k + 4 * has_v;
        if (ALIGNED && do_o && do_s) {
          // all 8 loads, a missing K_{i+2} / V_{i+1} re-reading tile 0 into
          // the slot that tile would have had (read by no wave)
          const DmaSpread<MmaPlan<D, WR, true, true, Rd>::N, true> ex{
              has_k ? kp + (long long)(i + 2) * ROWS * sl.ks : kp, has_v ? vp + (long long)(i + 1) * ROWS * sl.vs : vp,
              lds_k + (uint32_t)(((i + 2) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
              lds_v + (uint32_t)(((i + 1) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
              true, true, dk, dv, kstep, vstep};
          mma_run<DT, D, WR, true, true, Rd>(obuf, vring + ((i - 1) % kSlots) * kTile + koff,
                                             kring + (i % kSlots) * kTile + koff, pk, qop, acc_o, s, lane, ex);
          n_new = 8;
        } else if (do_o && do_s) {
          // full phase: with full tiles the loads are spread over its MFMAs
          const bool spread = (!has_k || Nk - (i + 2) * ROWS >= ROWS) && (!has_v || Nk - (i + 1) * ROWS >= ROWS);
          if (!spread) issue_step(i);
          const DmaSpread<MmaPlan<D, WR, true, true, Rd>::N> ex{kp + (long long)(i + 2) * ROWS * sl.ks,
                                                              vp + (long long)(i + 1) * ROWS * sl.vs,
                             lds_k + (uint32_t)(((i + 2) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
                             lds_v + (uint32_t)(((i + 1) % kSlots) * kTile) + (uint32_t)(64 * wg * 16),
                             has_k && spread, has_v && spread, dk, dv, kstep, vstep};
          mma_run<DT, D, WR, true, true, Rd>(obuf, vring + ((i - 1) % kSlots) * kTile + koff,
                                                    kring + (i % kSlots) * kTile + koff, pk, qop, acc_o, s, lane, ex);
        } else {
          issue_step(i);
          if (do_o)
            mma_run<DT, D, WR, true, false, Rd>(obuf, vring + ((i - 1) % kSlots) * kTile + koff,
                                                       kring + (i % kSlots) * kTile + koff, pk, qop, acc_o, s, lane);
          else if (do_s)
            mma_run<DT, D, WR, false, true, Rd>(obuf, vring + koff, kring + (i % kSlots) * kTile + koff, pk, qop,
                                                       acc_o, s, lane);
        }
        dma_barrier(n_new);  // Y_i
        if (i < wave_tiles) softmax(i);
        mma_pre(i < wave_tiles, i, i + 1 < wave_tiles, i + 1);
      }
    } else {
      for (int i = 0; i <= n_kv; ++i) {
        const int n_new = issue_step(i);
        if (i >= 1 && i - 1 < wave_tiles) softmax(i - 1);
        mma_pre(i >= 1 && i - 1 < wave_tiles, i - 1, i < wave_tiles, i);
        dma_barrier(n_new);  // Y_i
        mma(i >= 1 && i - 1 < wave_tiles, i - 1, i < wave_tiles, i);
      }
    }

    // Split mode, first block: every wave is past the last barrier, so no K
    // slot is read any more, and group 1 has finished its last V reads (group
    // 0 finished them before that barrier). Load the next block's K_0, K_1
    // (group 0) and V_0 (group 1) now, and its Q (group 1 here, group 0 once
    // its join is done); the buffer of the join starts at V slot 1.
    const bool next = SPLIT && item + 1 < n_items;
    const int q0n = kBMs * wk.qt;
    if (next) {
      const int last_key = min(q0n + kBMs, Nq) - 1 + off;
      const int n_kvn = last_key < 0 ? 0 : min((Nk + ROWS - 1) / ROWS, last_key / ROWS + 1);
      if (grp == 0) {
        if (0 < n_kvn) issue(false, 0);
        if (1 < n_kvn) issue(false, 1);
      } else {
        if (0 < n_kvn) issue(true, 0);
        load_q(q0n);
      }
    }

    // ---- epilogue: normalise once, write O and LSE
    auto epilogue = [&]() {
      const float l_tot = halves_sum(l_run);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (qrow < Nq) {
        uint16_t* orow = sl.o + (size_t)qrow * sl.os;
  #pragma unroll
        for (int mt = 0; mt < MT; ++mt)
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
    };
    if constexpr (!SPLIT) {
      if (!wave_active) return;
      epilogue();
    } else {
      // Join the two key halves of each row. Group 1 leaves its (m, l, O^T
      // accumulator) in LDS from V slot 1 on, past the first barrier (its own
      // last V reads); group 0 merges them into its own and writes the block.
      // The third barrier keeps the next block's loads (V_1 at its first
      // step) off the buffer until then.
      float* const xb = reinterpret_cast<float*>(smem + kXOff) + (wave & 3) * (XW * 64) + lane;
      __syncthreads();
      if (grp == 1) {
  #pragma unroll
        for (int mt = 0; mt < MT; ++mt)
  #pragma unroll
          for (int r = 0; r < 16; ++r) xb[(16 * mt + r) * 64] = acc_o[mt][r];
        xb[16 * MT * 64] = m_run;
        xb[(16 * MT + 1) * 64] = l_run;
      }
      __syncthreads();
      if (grp == 0) {
        const float m1 = xb[16 * MT * 64], l1 = xb[(16 * MT + 1) * 64];
        const float m = fmaxf(m_run, m1);
        const float a0 = m_run == -__builtin_inff() ? 0.f : exp2_fast(m_run - m);
        const float a1 = m1 == -__builtin_inff() ? 0.f : exp2_fast(m1 - m);
  #pragma unroll
        for (int mt = 0; mt < MT; ++mt)
  #pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[mt][r] = a0 * acc_o[mt][r] + a1 * xb[(16 * mt + r) * 64];
        l_run = a0 * l_run + a1 * l1;
        m_run = m;
        if (next) load_q(q0n);
        if (wave_active) epilogue();
      }
      __syncthreads();
    }
  }  // item
}

// Compute units of the current device (0 if the query fails), asked once per device.
int device_cus() {
  static std::atomic<int> cache[256];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

std::atomic<int> g_schedule{FA_SCHEDULE_AUTO};

// Split mode when a causal grid of 256-row workgroups fits on the GPU at
// once: the workgroup of the last query tile then sets the time, while in
// split mode every workgroup has the same work. A grid of several rounds is
// balanced already by the heaviest-first order.
bool use_split(long long nblocks, int rows) {
  const int mode = g_schedule.load(std::memory_order_relaxed);
  if (mode != FA_SCHEDULE_AUTO) return mode == FA_SCHEDULE_SPLIT;
  const int cus = device_cus();
  return rows > kBMs && cus > 0 && nblocks <= cus;
}

template <int DT, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int rows = VARLEN ? a.max_seqlen_q : a.Nq;
  const int n_qt = (rows + kBM - 1) / kBM;
  const long long nblocks = (long long)n_qt * a.B * a.Hq;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (nblocks == 0) return hipSuccess;
  const Varlen vl{a.cu_q, a.cu_k, a.total_q, a.total_k};
  if constexpr (CAUSAL && !VARLEN) {
    if (use_split(nblocks, rows)) {
      const int n_pairs = ((rows + kBMs - 1) / kBMs + 1) / 2;
      const long long nsplit = (long long)n_pairs * a.B * a.Hq;
      if (a.Nk % (8192 / D) == 0)
        hipLaunchKernelGGL((fa_fwd_kernel<DT, D, true, false, true, true>), dim3((unsigned)nsplit), dim3(kThreads), 0,
                           stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                           a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_pairs, vl, a.layout);
      else
        hipLaunchKernelGGL((fa_fwd_kernel<DT, D, true, false, true, false>), dim3((unsigned)nsplit), dim3(kThreads), 0,
                           stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                           a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_pairs, vl, a.layout);
      return hipGetLastError();
    }
  }
  if (!VARLEN && a.Nk % (8192 / D) == 0)
    hipLaunchKernelGGL((fa_fwd_kernel<DT, D, CAUSAL, VARLEN, false, !VARLEN>), dim3((unsigned)nblocks), dim3(kThreads),
                       0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                       a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_qt, vl, a.layout);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<DT, D, CAUSAL, VARLEN, false, false>), dim3((unsigned)nblocks), dim3(kThreads),
                       0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                       a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_qt, vl, a.layout);
  return hipGetLastError();
}

template <int DT, int D, bool CAUSAL>
hipError_t launch_v(const FwdArgs& a, hipStream_t stream) {
  return a.cu_q != nullptr ? launch_t<DT, D, CAUSAL, true>(a, stream) : launch_t<DT, D, CAUSAL, false>(a, stream);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const bool c = a.causal != 0;
  if (a.dtype == DT_BF16) return c ? launch_v<DT_BF16, D, true>(a, stream) : launch_v<DT_BF16, D, false>(a, stream);
  return c ? launch_v<DT_FP16, D, true>(a, stream) : launch_v<DT_FP16, D, false>(a, stream);
}

}  // namespace

int set_fwd_schedule(int mode) {
  if (mode != FA_SCHEDULE_AUTO && mode != FA_SCHEDULE_TILES && mode != FA_SCHEDULE_SPLIT) return -1;
  return g_schedule.exchange(mode);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace fa
