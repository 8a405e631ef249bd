// fa_decode.hip - one query token per sequence against its KV cache (gfx950).
//
// Decode reads every cached K/V row once and does little arithmetic per byte,
// so its time is set by memory traffic ("Advanced techniques for enhancing LLM
// throughput", cabseo.com, "Autoregressive and memory-bound operations"). The
// keys of each (sequence, kv-head) are cut into chunks; one wave streams one
// chunk and serves all q-heads of the group from that single read
// (grouped-query attention, SDPA page, devhandbook.co.kr, Example 5).
//
// Split kernel: a grid of as many single-wave workgroups as the GPU holds at
// once. The cached rows of all (sequence, kv-head) pairs, in that order and
// in blocks of 32, form one stream; each wave takes an equal contiguous share
// of it (cut at block boundaries, never less than one chunk), so every wave
// has the same amount of work whatever the mix of sequence lengths, and no
// wave slot is spent on the empty rows past a short sequence's end. A share
// that spans several pairs gives one partial result per pair. No workgroup
// barriers. K goes from HBM straight into the A-operand registers of
// S^T = K Q^T (lane l holds key l%32); V goes through a per-wave LDS tile
// in row-major order and is read back transposed with ds_read_b64_tr_b16 as
// the A operand of O^T += V^T P^T. The q-heads of group g are the columns of
// the B operand (up to 32; unused columns are zero). The next block's loads
// are issued as soon as the current block's registers are consumed, so each
// wave keeps a block in flight while it computes. Each partial's normalised
// output and LSE go to the workspace. The cache is either one contiguous
// slab per (sequence, kv-head) or a set of fixed-size pages reached through a
// per-sequence page table.
// Combine kernel: per (b, h), merge the partials of sequence b with the LSE form
// of the softmax-merge identity ("The math of Flash Attention", unite.ai).
#include <mutex>

#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBlk = 32;  // keys per block

// V block in LDS: row-major [32][D], 16-byte chunks XOR-swizzled by row so
// that the 8 rows one transposed read touches fall in distinct banks.
template <int D>
struct VBlock {
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int RPB = 256 / (2 * D);   // rows per 256 bytes of banks
  static constexpr int BYTES = kBlk * D * 2;
  static constexpr int PER_LANE = kBlk * CPR / 64;  // chunks per lane
  __device__ static inline int sw(int row) { return 4 * ((row / RPB) % (CPR / 4)); }
  __device__ static inline int off(int row, int chunk) { return row * (2 * D) + ((chunk ^ sw(row)) * 16); }
};

// Transposed read of the A operand of O^T += V^T P^T for O^T rows 32*mt.. and
// the 16-key group G of the block. ds_read_b64_tr_b16 gives lane i of each
// 16-lane group element i%4 of lanes 4e + i/4 (e = 0..3); lane 4e+q therefore
// points at key row 16G + 8p + 4h + e, columns 32mt + 16*dh + 4q .. +3, so lane
// l ends up with V[16G + 8p + 4h + e][32mt + l%32] for e = 0..3, which is the
// key order of the P accumulator (p = 0, 1 are the two halves).
template <int D>
__device__ inline u32x4 vt_tr_operand(const char* __restrict__ vl, int mt, int G, int lane) {
  using V = VBlock<D>;
  const int gi = lane >> 4, s = lane & 15, e = s >> 2, q = s & 3;
  const int h = gi >> 1, dh = gi & 1;
  const int chunk = 4 * mt + 2 * dh + (q >> 1);
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = 16 * G + 8 * p + 4 * h + e;
    const char* addr = vl + V::off(row, chunk) + 8 * (q & 1);
    const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(addr));
    const u32x2 w = __builtin_bit_cast(u32x2, t);
    out[2 * p] = w[0];
    out[2 * p + 1] = w[1];
  }
  return out;
}

// Where the cache rows live. Contiguous: [B, Hkv, Lcap, D]. Paged: pages of
// `page` rows, [num_pages, Hkv, page, D], logical row j of sequence b in page
// table[b * max_pages + j / page] ("Paged attention", cabseo.com).
struct PageMap {
  const int32_t* table;
  int page, max_pages, num_pages;
  int shift;  // log2(page) when page is a power of two, else -1
};

// The block stream: pair (b, g) holds nblk_b = ceil(L_b / 32) blocks and
// starts at block pre_b + g nblk_b, pre_b = Hkv (nblk_0 + ... + nblk_{b-1}).
// A wave walks the sequences 64 at a time: lane j holds nblk of sequence
// blk + j and the inclusive block count up to it, so finding the pair of a
// stream position is one ballot. Positions are visited in increasing order,
// so the walk only moves forward.
struct BlockWalk {
  const int32_t* seqlens;
  int B, Hkv, Lcap;
  int blk = 0;        // first sequence of the lane block
  int blk_start = 0;  // stream blocks before sequence blk
  int nblk = 0;       // this lane's blocks per pair
  int incl = 0;       // stream blocks of sequences blk .. blk + lane
  int blk_total = 0;  // stream blocks of the whole lane block
  __device__ void load(int lane) {
    const int b = blk + lane;
    const int L = b < B ? min(max(seqlens[b], 0), Lcap) : 0;
    nblk = (L + 31) / 32;
    int x = nblk * Hkv;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    incl = x;
    blk_total = __shfl(x, 63, 64);
  }
  // Stream position p (< the stream length) -> pair (b, g), block lb within
  // it, the pair's first stream block seg0, its rows L and blocks nb.
  __device__ void find(int p, int lane, int& b, int& g, int& lb, int& seg0, int& L, int& nb) {
    while (p - blk_start >= blk_total) {
      blk_start += blk_total;
      blk += 64;
      load(lane);
    }
    const int r = p - blk_start;
    const int j = __builtin_popcountll(__builtin_amdgcn_ballot_w64(incl <= r));
    nb = __builtin_amdgcn_readlane(nblk, j);
    const int ex = __builtin_amdgcn_readlane(incl, j) - nb * Hkv;
    const int rr = r - ex;
    b = blk + j;
    g = rr / nb;
    lb = rr - g * nb;
    seg0 = blk_start + ex + g * nb;
    L = min(max(seqlens[b], 0), Lcap);
  }
};

// One wave per workgroup. At d = 128 a wave holds about 340 registers (Q,
// the O accumulator and one block of K and V in flight), so one wave runs
// per SIMD; capping it at 256 for two waves per SIMD measured slower.
//
// Wave w of W takes stream blocks [w S, (w + 1) S), S = max(ceil(T / W),
// chunk / 32) for a stream of T blocks. Its partial of pair (b, g) goes to
// slot w - floor(seg0 / S) of the pair (seg0: the pair's first block), at
// most ceil(Lcap / chunk) + 1 slots. Wave 0 also writes S and every pre_b to
// the header (hdr[0] = S, hdr[1 + b] = pre_b) for the combine kernel.
template <int DT, int D, bool PAGED>
__global__ __launch_bounds__(64) void fa_decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int32_t* __restrict__ hdr, int B, int Hq, int Hkv, int Lcap, int chunk, int slots, float scale_log2,
    PageMap pm) {
  constexpr int KS = D / 16, MT = D / 32, CPR = D / 8;
  using V = VBlock<D>;
  __shared__ __attribute__((aligned(16))) char vl[V::BYTES];

  const int lane = threadIdx.x, half = lane >> 5;
  const int grp = Hq / Hkv;
  const int wave_id = blockIdx.x;
  BlockWalk walk{seqlens, B, Hkv, Lcap};
  walk.load(lane);
  int T;  // stream length in blocks
  while (true) {
    if (wave_id == 0 && walk.blk + lane < B)
      hdr[1 + walk.blk + lane] = walk.blk_start + walk.incl - walk.nblk * Hkv;
    T = walk.blk_start + walk.blk_total;
    if (walk.blk + 64 >= B) break;
    walk.blk_start = T;
    walk.blk += 64;
    walk.load(lane);
  }
  const int S = max((T + (int)gridDim.x - 1) / (int)gridDim.x, chunk / 32);
  if (wave_id == 0 && lane == 0) hdr[0] = S;
  if ((long long)wave_id * S >= T) return;  // nothing left for this wave
  int p = wave_id * S;
  const int end = (int)min((long long)T, (long long)p + S);
  walk.blk = 0;
  walk.blk_start = 0;
  walk.load(lane);
  while (p < end) {
    int b, g, lb, seg0, L, nbk;
    walk.find(p, lane, b, g, lb, seg0, L, nbk);
    const int le = min(nbk, lb + (end - p));
    const int k0 = lb * kBlk;
    const int n = min(le * kBlk, L) - k0;  // >= 1: block lb holds cached rows
    const int slot = wave_id - seg0 / S;
    p += le - lb;

    const int col = lane & 31;  // q-head within the group (B-operand column)
    const size_t bg = (size_t)b * Hkv + g;

    // Page entries of this chunk, 64 at a time, one per lane; a block of 32
    // rows never straddles two pages (page is a multiple of 32). An entry
    // outside [0, num_pages) is not followed (page 0 is read instead) and
    // poisons this chunk's result.
    int pg_lane = 0, pg_base = -(1 << 30);
    bool bad = false;
    auto page_of = [&](int row) -> int {  // row: logical cache row, wave-uniform
      const int idx = pm.shift >= 0 ? row >> pm.shift : row / pm.page;
      if (idx - pg_base >= 64 || idx < pg_base) {
        pg_base = idx;
        const int e = idx + lane;
        pg_lane = (e < pm.max_pages) ? pm.table[(size_t)b * pm.max_pages + e] : 0;
      }
      int pg = __builtin_amdgcn_readlane(pg_lane, idx - pg_base);
      if (pg < 0 || pg >= pm.num_pages) {
        bad = true;
        pg = 0;
      }
      return pg;
    };
    // Element offset of the first cache row of the 32-row block at chunk
    // offset j0 (the same for K and V).
    auto block_off = [&](int j0) -> size_t {
      if constexpr (PAGED) {
        const int row = k0 + j0;
        const int within = pm.shift >= 0 ? row & (pm.page - 1) : row % pm.page;
        return (((size_t)page_of(row) * Hkv + g) * pm.page + within) * D;
      } else {
        return (bg * Lcap + k0 + j0) * D;
      }
    };

    u32x4 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (col < grp)
        qop[ks] = *reinterpret_cast<const u32x4*>(q + ((size_t)b * Hq + g * grp + col) * D + 16 * ks + 8 * half);
      else
        qop[ks] = u32x4{0u, 0u, 0u, 0u};
    }

    f32x16 acc_o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;
    float m_run = -__builtin_inff();
    float l_run = 0.f;

    // Block loads. Rows at or beyond n re-read row n-1 (their scores are
    // masked to -inf, so they contribute 0); no row past L is touched.
    u32x4 ka[KS];         // K: lane holds key l%32, d chunk 2ks + l/32
    u32x4 vr[V::PER_LANE];  // V: chunk lane + 64i of the row-major block
    size_t boff = block_off(0);  // offset of the block being loaded
    auto load_k = [&](int j0) {
      const uint16_t* kp = kc + boff;
      const int row = min(col, n - 1 - j0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[ks] = *reinterpret_cast<const u32x4*>(kp + (size_t)row * D + 16 * ks + 8 * half);
    };
    auto load_v = [&](int j0) {
      const uint16_t* vp = vc + boff;
#pragma unroll
      for (int i = 0; i < V::PER_LANE; ++i) {
        const int ci = lane + 64 * i;
        const int row = min(ci / CPR, n - 1 - j0);
        vr[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)row * D + (ci % CPR) * 8);
      }
    };
    load_k(0);
    load_v(0);

    const int nb = (n + kBlk - 1) / kBlk;
    for (int bi = 0; bi < nb; ++bi) {
      const int j0 = bi * kBlk;
      const bool more = bi + 1 < nb;
      // ---- S^T = K Q^T for this block; then K registers are free for the next block
      f32x16 sacc[1];
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[0][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[0] = mfma32<DT>(ka[ks], qop[ks], sacc[0]);
      if (more) {
        boff = block_off(j0 + kBlk);
        load_k(j0 + kBlk);
      }
      // ---- V block to LDS (previous block's transposed reads are complete:
      // every LDS read of this wave returned before its MFMA issued)
#pragma unroll
      for (int i = 0; i < V::PER_LANE; ++i) {
        const int ci = lane + 64 * i;
        *reinterpret_cast<u32x4*>(vl + V::off(ci / CPR, ci % CPR)) = vr[i];
      }
      if (more) load_v(j0 + kBlk);
      // ---- mask the ragged end of the chunk, online softmax
      if (j0 + kBlk > n) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j0 + acc_key(r, half) >= n) sacc[0][r] = -__builtin_inff();
      }
      uint32_t pk[1][8];
      softmax_step<DT, 1, MT>(sacc, scale_log2, m_run, l_run, acc_o, pk);
      // ---- O^T += V^T P^T (LDS writes of this wave complete before its reads)
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the V block is in LDS
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 bop = {pk[0][4 * u], pk[0][4 * u + 1], pk[0][4 * u + 2], pk[0][4 * u + 3]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc_o[mt] = mfma32<DT>(vt_tr_operand<D>(vl, mt, u, lane), bop, acc_o[mt]);
      }
    }

    // ---- chunk result: normalised O (fp32) and LSE to the workspace
    const float l_tot = bad ? __builtin_nanf("") : halves_sum(l_run);
    if (col < grp) {
      const size_t row = ((size_t)b * Hq + g * grp + col) * slots + slot;
      const float inv = 1.f / l_tot;  // l_tot > 0: the chunk holds at least one key
      float* orow = ws_o + row * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * mt + 8 * i + 4 * half;
          float4 w = {acc_o[mt][4 * i] * inv, acc_o[mt][4 * i + 1] * inv, acc_o[mt][4 * i + 2] * inv,
                      acc_o[mt][4 * i + 3] * inv};
          *reinterpret_cast<float4*>(orow + d0) = w;
        }
      if (half == 0) ws_lse[row] = (m_run + __builtin_log2f(l_tot)) * kLn2;
    }
  }
}

// Merge the partial results of (b, h): LSE = log sum_s exp(LSE_s),
// O = sum_s exp(LSE_s - LSE) O_s. One wave per (b, h): the lanes reduce the
// partial LSEs together, then each lane accumulates D/64 output elements
// over the partials, eight row loads in flight at a time. The partials of
// pair (b, g) are the slots 0 .. floor((seg0 + nblk - 1) / S) - floor(seg0 / S),
// with S and pre_b (seg0 = pre_b + g nblk) from the split kernel's header.
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int DT, int D>
__global__ __launch_bounds__(64) void fa_decode_combine_kernel(const float* __restrict__ ws_o,
                                                               const float* __restrict__ ws_lse,
                                                               const int32_t* __restrict__ hdr,
                                                               const int32_t* __restrict__ seqlens,
                                                               uint16_t* __restrict__ o, float* __restrict__ lse,
                                                               int Hq, int Hkv, int Lcap, int slots) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / Hq, g = (bh % Hq) / (Hq / Hkv);
  const int lane = threadIdx.x;
  const int L = min(max(seqlens[b], 0), Lcap);
  const int nblk = (L + 31) / 32;
  int ns = 0;
  if (nblk > 0) {
    const int S = hdr[0];
    const int seg0 = hdr[1 + b] + g * nblk;
    ns = (seg0 + nblk - 1) / S - seg0 / S + 1;
  }
  const float* lp = ws_lse + (size_t)bh * slots;
  const float* op = ws_o + (size_t)bh * slots * D + lane * PER;
  float m = -__builtin_inff();
  for (int s = lane; s < ns; s += 64) m = fmaxf(m, lp[s]);
  m = wave_max(m);
  float sum = 0.f;
  for (int s = lane; s < ns; s += 64) sum += __expf(lp[s] - m);
  sum = wave_sum(sum);
  const float lse_all = (ns > 0) ? m + __logf(sum) : -__builtin_inff();
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const float w = (s0 + lane < ns) ? __expf(lp[s0 + lane] - lse_all) : 0.f;
    const int cnt = min(64, ns - s0);
    for (int j = 0; j < cnt; j += 8) {
      float rows[8][PER];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < PER; ++i) rows[u][i] = (j + u < cnt) ? op[(size_t)(s0 + j + u) * D + i] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u));
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += wj * rows[u][i];
      }
    }
  }
  uint16_t* orow = o + (size_t)bh * D;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow + lane * 2) = pack2<DT>(acc[0], acc[1]);
  } else {
    const uint32_t w = pack2<DT>(acc[0], 0.f);
    orow[lane] = (uint16_t)(w & 0xFFFFu);
  }
  if (lse != nullptr && lane == 0) lse[bh] = lse_all;
}

// Single-wave workgroups of `kernel` that the current device holds at once
// (workgroups per CU from the occupancy calculator x CUs), computed once per
// (device, kernel) and kept for the life of the process.
hipError_t resident_waves(const void* kernel, int* waves) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  struct Entry {
    const void* kernel;
    int dev, waves;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].kernel == kernel && cache[i].dev == dev) {
      *waves = cache[i].waves;
      return hipSuccess;
    }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0);
  if (e != hipSuccess) return e;
  *waves = max(1, cus * max(1, per_cu));
  if (used < 64) cache[used++] = Entry{kernel, dev, *waves};
  return hipSuccess;
}

template <int DT, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(a.workspace);
  float* ws_o = reinterpret_cast<float*>(ws);
  float* ws_lse = reinterpret_cast<float*>(ws + a.ws_lse_offset);
  int32_t* hdr = reinterpret_cast<int32_t*>(ws + a.ws_hdr_offset);
  int shift = -1;
  if (a.page_size > 0 && (a.page_size & (a.page_size - 1)) == 0) shift = __builtin_ctz((unsigned)a.page_size);
  const PageMap pm{a.block_table, a.page_size, a.max_pages, a.num_pages, shift};
  // As many waves as fit on the GPU at once; the stream has at most
  // B * Hkv * ceil(Lcap / 32) blocks, which must fit an int.
  if ((long long)a.B * a.Hkv * ((a.Lcap + 31) / 32) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const void* kernel = a.block_table != nullptr ? (const void*)fa_decode_split_kernel<DT, D, true>
                                                : (const void*)fa_decode_split_kernel<DT, D, false>;
  int waves = 0;
  hipError_t e = resident_waves(kernel, &waves);
  if (e != hipSuccess) return e;
  if (a.block_table != nullptr)
    hipLaunchKernelGGL((fa_decode_split_kernel<DT, D, true>), dim3((unsigned)waves), dim3(64), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.seqlens, ws_o,
                       ws_lse, hdr, a.B, a.Hq, a.Hkv, a.Lcap, a.chunk, a.slots, a.scale * kLog2e, pm);
  else
    hipLaunchKernelGGL((fa_decode_split_kernel<DT, D, false>), dim3((unsigned)waves), dim3(64), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.seqlens, ws_o,
                       ws_lse, hdr, a.B, a.Hq, a.Hkv, a.Lcap, a.chunk, a.slots, a.scale * kLog2e, pm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_decode_combine_kernel<DT, D>), dim3(a.B * a.Hq), dim3(64), 0, stream, ws_o, ws_lse, hdr,
                     a.seqlens, (uint16_t*)a.o, a.lse, a.Hq, a.Hkv, a.Lcap, a.slots);
  return hipGetLastError();
}

}  // namespace

// Workspace of fa_decode_noalloc: a file-scope device array, one copy per
// GPU, held for the life of the process. Host code never passes the array's
// name to a kernel (on the host it only stands for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and cached.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 256;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == DT_BF16) return a.d == 128 ? launch_decode_t<DT_BF16, 128>(a, stream) : launch_decode_t<DT_BF16, 64>(a, stream);
  return a.d == 128 ? launch_decode_t<DT_FP16, 128>(a, stream) : launch_decode_t<DT_FP16, 64>(a, stream);
}

}  // namespace fa
