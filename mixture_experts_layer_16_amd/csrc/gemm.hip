// Expert FFNs as grouped GEMMs: one launch for gate/up (+ activation), one for
// down, over every routed expert and every shared expert at once.
//
// Expert structure: SwiGLU with three matrices (V4.1 page "Mixture-of-Experts",
// "Le compte des paramètres"; activation clip from its table "Les chiffres de
// DeepSeek-V4.1-Flash"), or the two-layer ReLU expert of the "Mixture of
// Experts" fiche (dataistudio.com, code section).  The shared expert is one more
// group whose rows are all N tokens ("Mixture-of-Experts : routage et
// capacité", "L'idée — Top-k et mélange").
//
// Groups and tiles are planned on the device from the dispatch offsets, so the
// host never waits for the per-expert row counts: the grid is sized for an upper
// bound and surplus blocks exit at once.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

enum { MODE_GATEUP = 0, MODE_RELU_UP = 1, MODE_DOWN = 2 };



// ---------------------------------------------------------------------------
// tile plan: groups [0, n_gather) from offsets, then n_ident dense groups.

__global__ __launch_bounds__(1024) void ffn_plan_kernel(
    const int32_t* __restrict__ offsets, int n_gather, int n_ident, int64_t N,
    int64_t rows_cap, int64_t ident_row0, int BM, int BMS, int32_t* __restrict__ plan,
    int32_t* __restrict__ plan_s, int32_t* __restrict__ sat) {
  __shared__ int32_t mt[2 * 1024];
  // the range count of this call's fp16 intermediates starts at zero (the
  // GEMMs that add to it run after this kernel on the same stream)
  if (sat && threadIdx.x == 0) *sat = 0;
  __shared__ int32_t mts[2 * 1024];
  __shared__ int32_t tmp[1024];
  const int G = n_gather + n_ident;
  int32_t* tile_start = plan;
  int32_t* row_begin = plan + G + 1;
  int32_t* rows = row_begin + G;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    int64_t rb, r;
    if (g < n_gather) {
      // clamp to [0, rows_cap] so a malformed offsets array cannot send the
      // GEMMs outside the row buffers
      int64_t lo = offsets[g], hi = offsets[g + 1];
      lo = lo < 0 ? 0 : (lo > rows_cap ? rows_cap : lo);
      hi = hi < lo ? lo : (hi > rows_cap ? rows_cap : hi);
      rb = lo;
      r = hi - lo;
    } else {
      rb = ident_row0 + (int64_t)(g - n_gather) * N;
      r = N;
    }
    // with a second plan, a remainder of at most BMS rows past the last full
    // BM-row tile goes to it (one BMS-row tile) instead of a mostly empty
    // BM-row tile
    int64_t small = 0;
    if (plan_s) {
      const int64_t rem = r % BM;
      small = (rem > 0 && rem <= BMS) ? rem : 0;
      plan_s[G + 1 + g] = (int32_t)(rb + r - small);
      plan_s[G + 1 + G + g] = (int32_t)small;
      mts[g] = small > 0 ? 1 : 0;
    }
    row_begin[g] = (int32_t)rb;
    rows[g] = (int32_t)(r - small);
    mt[g] = (int32_t)((r - small + BM - 1) / BM);
  }
  __syncthreads();
  const int total = block_exclusive_scan_1024(mt, G, tmp);
  for (int g = threadIdx.x; g < G; g += blockDim.x) tile_start[g] = mt[g];
  if (threadIdx.x == 0) tile_start[G] = total;
  if (plan_s) {
    __syncthreads();
    const int total_s = block_exclusive_scan_1024(mts, G, tmp);
    for (int g = threadIdx.x; g < G; g += blockDim.x) plan_s[g] = mts[g];
    if (threadIdx.x == 0) plan_s[G] = total_s;
  }
}

struct Tile {
  int g, m0, n0, M;
  int64_t rb;
  bool ok;
};

// Block -> tile.  Consecutive tile indices go to the same XCD (blocks are dealt
// to the 8 XCDs round-robin, so block b maps to index (b % 8) * per + b / 8);
// within a group, tiles are ordered by super-rows of a few m-tiles, n-tile
// major inside each, so the tiles one XCD runs together share weight rows and
// token rows in that XCD's L2.
__device__ __forceinline__ Tile decode_tile(const int32_t* __restrict__ plan, int G, int ntn,
                                            int BM, int CT) {
  Tile t;
  t.ok = false;
  const int32_t* tile_start = plan;
  const int total = tile_start[G] * ntn;
  const int per = (total + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per) return t;
  const int L = (blockIdx.x % kXcds) * per + slot;
  if (L >= total) return t;
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] * ntn <= L) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int mtg = tile_start[g + 1] - tile_start[g];
  const int local = L - tile_start[g] * ntn;
  // within a group: super-rows of GM m-tiles; inside one, n-tile major, m-tile
  // minor, so the tiles in flight on one XCD share both x rows and weight rows
  constexpr int GM = 8;
  const int sr = local / (GM * ntn);
  const int rem = local - sr * GM * ntn;
  const int gm = min(GM, mtg - sr * GM);
  const int nt = rem / gm;
  const int mtile = sr * GM + (rem - nt * gm);
  t.g = g;
  t.m0 = mtile * BM;
  t.n0 = nt * CT;
  t.M = plan[G + 1 + G + g];
  t.rb = plan[G + 1 + g];
  t.ok = true;
  return t;
}

// LDS line swizzle: XOR applied to the 16-byte chunk position inside a
// 128-byte line.  Chosen so that any 8 consecutive rows, and the rows of each
// parity among any 16 consecutive rows, use distinct positions: conflict-free
// whether the LDS serves a 128-bit read 8 lanes (32 banks) or 16 lanes (64
// banks) at a time.  RPL = rows per line (1 for 64-wide k-slices, 2 for 32).
template <int RPL>
__device__ __forceinline__ int lds_swizzle(int line) {
  if (RPL == 1) return (line & 7) ^ ((line >> 3) & 1);
  return ((line >> 1) & 3) ^ ((line & 1) << 1);
}

// silu(a) * u, clipped to [-clip, clip] when clip > 0.  The reciprocal is the
// hardware approximation (about 1 ulp in fp32), far below the fp16 rounding of
// the stored h.
__device__ __forceinline__ float swiglu(float a, float u, float clip) {
  float h = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * u;
  if (clip > 0.f) h = fminf(fmaxf(h, -clip), clip);
  return h;
}

// The saved up pre-activation (fp16 bits) of a SwiGLU element: u itself, or,
// where this forward clamped silu(a) u (same formula as swiglu above), an
// infinity whose sign times the sign of a is the sign of the clamped h -- so
// the backward follows this pass's clamp decision exactly instead of
// re-deciding it from fp16-rounded values.
__device__ __forceinline__ uint16_t saved_up_bits(float a, float u, float clip) {
  if (clip > 0.f) {
    const float h = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * u;
    if (fabsf(h) > clip) return ((h < 0.f) != (a < 0.f)) ? 0xFC00u : 0x7C00u;
  }
  return f32_to_f16_sat(u);
}

struct GemmParams {
  const void* A;                 // x (gate/up) or h (down)
  const int32_t* token_of_row;   // routed groups of the gate/up pass
  const void* Br0;               // routed: gate (SwiGLU) | W1^T (ReLU) | down
  const void* Br1;               // routed: up (SwiGLU)
  const void* Bs0;               // dense groups
  const void* Bs1;
  void* C;                       // h or y_rows
  const int32_t* plan;
  int G, n_gather;
  int K, Ncols;                  // reduction length; output columns
  int64_t ldA, ldC;              // row strides in elements
  int64_t wstride;               // elements per expert matrix
  int64_t n_tokens;              // clamp for token ids
  int64_t ident_row0;            // first row of the dense groups (token t of dense
                                 // group i is row ident_row0 + i*n_tokens + t)
  float clip;
  // gate/up pass, optional (both or neither): the pre-activations written next
  // to h in the same row layout, fp16 -- Sa = x W_gate^T (SwiGLU), Su = x W_up^T
  // (SwiGLU) or x W1 before the ReLU
  void* Sa;
  void* Su;
  int32_t* sat;                  // optional: count of stored h / y_rows values of
                                 // magnitude 65504 (saturated, or rounded there)
};

// ---------------------------------------------------------------------------
// bf16 grouped GEMM on the matrix cores.
//
// C[m][n] = sum_k A[m][k] * B[n][k]  (both operands contiguous along k).
// A block computes BM rows x BN weight rows; k-slices of BK are staged in LDS
// (double buffered); WM x WN waves, each (BM/WM) rows x (BN/WN) weight rows of
// v_mfma_f32_32x32x16 accumulators.  In the gate/up pass the BN weight rows are
// BN/2 gate rows and the matching BN/2 up rows, so one lane holds the gate and
// up value of the same output element and the SwiGLU (and clip) is applied in
// registers before h is written once.
//
// LDS layout: 128-byte lines holding 128/(2*BK) rows (one row for BK = 64, two
// for BK = 32); the 16-byte chunk at position q of line l is stored at position
// q ^ lds_swizzle(l), so the rows one MFMA operand fetch reads spread over all
// banks, and each thread's chunk of a staged row keeps one swizzled position.
//
// Number formats.  The gate/up pass multiplies bf16 x and bf16 weights; its
// result h is stored in fp16, whose 11-bit significand rounds 8x finer than
// bf16 (for inputs of the usual scale |h| is far inside fp16's range; a value
// beyond +-65504 is saturated, and every stored +-65504 is counted in the call's
// range status).
// The down pass therefore runs on the fp16 matrix cores: the bf16 W_down tile is
// converted to fp16 while it is staged into LDS -- exact for every bf16 value in
// fp16's normal range, and within 2^-24 absolute below it.  Expert output rows
// are written in fp16 as well.  With bf16 h and rows the rounding alone would
// use most of the 2e-2 * RMS(y) error budget; with fp16 it uses about a tenth.
template <int MODE, int BM, int BN, int BK, int WM_, int WN_, int MINB, int NSETS, int FRAGDB>
__global__ __launch_bounds__(64 * WM_ * WN_, MINB) void ffn_gemm_bf16(GemmParams p) {
  constexpr int NT = 64 * WM_ * WN_;          // threads
  constexpr int KCH = BK / 8;                // 16-byte chunks per staged row
  constexpr int RPL = 8 / KCH;               // rows per 128-byte LDS line
  constexpr int STAGE = (BM + BN) * BK;      // elements per LDS stage
  constexpr int RSTEP = NT / KCH;            // rows covered by one pass of the loaders
  constexpr int NA = BM / RSTEP;             // A chunks per thread per stage
  constexpr int NB = BN / RSTEP;             // B chunks per thread per stage
  constexpr int WROWS = BM / WM_;            // rows per wave
  constexpr int FM = WROWS / 32;             // A fragments (32 rows) per wave
  constexpr int FN = BN / WN_ / 32;          // B fragments (32 weight rows) per wave
  constexpr int CT = (MODE == MODE_GATEUP) ? BN / 2 : BN;   // output columns per tile
  constexpr int WCOLS = CT / WN_;            // output columns per wave
  static_assert(NA * RSTEP == BM && NB * RSTEP == BN, "loader shape");
  static_assert((RSTEP / RPL) % 8 == 0, "swizzle period");
  static_assert(MODE != MODE_GATEUP || FN % 2 == 0, "gate/up fragments come in pairs");
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * STAGE];

  const int ntn = (p.Ncols + CT - 1) / CT;
  const Tile tl = decode_tile(p.plan, p.G, ntn, BM, CT);
  if (!tl.ok) return;

  const int tid = threadIdx.x;
  const bool routed = tl.g < p.n_gather;
  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const uint16_t* B0 = static_cast<const uint16_t*>(routed ? p.Br0 : p.Bs0) +
                       (int64_t)(routed ? tl.g : tl.g - p.n_gather) * p.wstride;
  const uint16_t* B1 = nullptr;
  if (MODE == MODE_GATEUP)
    B1 = static_cast<const uint16_t*>(routed ? p.Br1 : p.Bs1) +
         (int64_t)(routed ? tl.g : tl.g - p.n_gather) * p.wstride;

  // ---- global -> register loaders: thread owns chunk kc of rows r0 + RSTEP*i
  const int kc = tid % KCH;
  const int r0 = tid / KCH;
  // the swizzled position of (row, chunk) depends only on r0 for a thread's rows
  const int sw_off = (((r0 % RPL) * KCH + kc) ^ lds_swizzle<RPL>(r0 / RPL)) << 3;
  const uint16_t* ag[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    int m = tl.m0 + r0 + RSTEP * i;
    if (m >= tl.M) m = tl.M - 1;
    int64_t arow;
    if (MODE == MODE_DOWN) {
      arow = tl.rb + m;
    } else if (routed) {
      arow = p.token_of_row[tl.rb + m];
      arow = arow < 0 ? 0 : (arow >= p.n_tokens ? p.n_tokens - 1 : arow);
    } else {
      arow = tl.rb + m - (p.ident_row0 + (int64_t)(tl.g - p.n_gather) * p.n_tokens);
    }
    ag[i] = A + arow * p.ldA + kc * 8;
  }
  const uint16_t* bg[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = r0 + RSTEP * i;
    if (MODE == MODE_GATEUP) {
      int col = tl.n0 + (n & (CT - 1));
      if (col >= p.Ncols) col = p.Ncols - 1;
      bg[i] = ((n < CT) ? B0 : B1) + (int64_t)col * p.K + kc * 8;
    } else {
      int col = tl.n0 + n;
      if (col >= p.Ncols) col = p.Ncols - 1;
      bg[i] = B0 + (int64_t)col * p.K + kc * 8;
    }
  }

  // two register sets: a slice is loaded two compute phases before it is
  // staged into LDS, so a global load has two slices of MFMA work to land
  u32x4_t ra[NSETS][NA], rbv[NSETS][NB];
  // Weight rows: with decode tiles (BM = 32) every weight byte is read once,
  // so they are loaded non-temporally (measured: the weight stream of the
  // decode passes runs ~8% faster than with cached loads); token rows are
  // reused by every weight tile and stay cached.
  auto load_w = [&](const uint16_t* q) -> u32x4_t {
    if constexpr (BM <= 32) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q));
    else return *reinterpret_cast<const u32x4_t*>(q);
  };
  // full k-slices: unconditional loads (no branch, so the compiler's waits only
  // cover the slice actually consumed); a ragged last slice zero-fills
  // Decode tiles walk their full k-slices from a rotated start (a hash of the
  // weight matrix and the n-tile; the ragged last slice stays last).  With
  // power-of-two row strides (d = 4096: 8 KB rows) the tiles that run at once
  // otherwise all read the same column offsets of their weight rows and crowd
  // a subset of the memory channels: measured over six placements of the same
  // weights, mix-D took 0.459-0.494 ms per layer without the rotation and
  // 0.452-0.456 ms with it.  The rotation depends on the tile's weights only,
  // so a row's result does not depend on the launch it is computed in.
  const int nfull_r = p.K / BK;
  int rot = 0;
  if constexpr (BM <= 32) {
    const uint32_t mat = (uint32_t)(routed ? tl.g : tl.g - p.n_gather);
    if (nfull_r > 1)
      rot = (int)(((uint32_t)(tl.n0 / CT) * 2654435761u + mat * 40503u) % (uint32_t)nfull_r);
  }
  auto load_full = [&](int kt, int set) {
    int kr = kt + rot;
    if (kr >= nfull_r) kr -= nfull_r;
    const int k0 = kr * BK;
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[set][i] = *reinterpret_cast<const u32x4_t*>(ag[i] + k0);
#pragma unroll
    for (int i = 0; i < NB; ++i) rbv[set][i] = load_w(bg[i] + k0);
  };
  auto load_tail = [&](int kt, int set) {
    const int k0 = kt * BK;
    const bool ok = (k0 + kc * 8) < p.K;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NA; ++i)
      ra[set][i] = ok ? *reinterpret_cast<const u32x4_t*>(ag[i] + k0) : z;
#pragma unroll
    for (int i = 0; i < NB; ++i) rbv[set][i] = ok ? load_w(bg[i] + k0) : z;
  };
  // row r of the stage starts at line r / RPL
  auto sstore = [&](uint16_t* s, int set) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      *reinterpret_cast<u32x4_t*>(s + ((r0 + RSTEP * i) / RPL) * 64 + sw_off) = ra[set][i];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      u32x4_t v = rbv[set][i];
      if (MODE == MODE_DOWN) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = bf16x2_to_f16x2(v[q]);
      }
      *reinterpret_cast<u32x4_t*>(s + BM * BK + ((r0 + RSTEP * i) / RPL) * 64 + sw_off) = v;
    }
  };

  // ---- MFMA fragment addressing: lane supplies row (lane & 31) of a 32-row
  // fragment and k-chunk kk*2 + (lane >> 5) of the slice
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM_, wn = wave / WM_;
  const int lr = lane & 31, lh = lane >> 5;
  const int lrow_part = lr % RPL;               // fragment bases are multiples of 32
  const int lline = lr / RPL;
  const int lswz = lds_swizzle<RPL>(lline);      // same for every fragment of this lane
  int a_off[FM], b_off[FN], ksw[BK / 16];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_off[i] = ((wm * WROWS + 32 * i) / RPL + lline) * 64;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int base;
    if constexpr (MODE == MODE_GATEUP)   // first half gate rows, then the matching up rows
      base = (j / (FN / 2)) * CT + wn * WCOLS + 32 * (j % (FN / 2));
    else
      base = wn * WCOLS + 32 * j;
    b_off[j] = BM * BK + (base / RPL + lline) * 64;
  }
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) ksw[kk] = ((lrow_part * KCH + kk * 2 + lh) ^ lswz) << 3;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto mfmas = [&](const u32x4_t (&af)[FM], const u32x4_t (&bf)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (MODE == MODE_DOWN)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8_t, af[i]), __builtin_bit_cast(f16x8_t, bf[j]), acc[i][j],
              0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bf[j]),
              acc[i][j], 0, 0, 0);
      }
  };
  auto read_frags = [&](const uint16_t* s, int kk, u32x4_t (&af)[FM], u32x4_t (&bf)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(s + a_off[i] + ksw[kk]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = *reinterpret_cast<const u32x4_t*>(s + b_off[j] + ksw[kk]);
  };
  auto compute = [&](const uint16_t* s) {
    if (FRAGDB) {
      // fragments of step kk+1 are read while the MFMAs of step kk run
      u32x4_t af[2][FM], bf[2][FN];
      read_frags(s, 0, af[0], bf[0]);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        if (kk + 1 < BK / 16) read_frags(s, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
        mfmas(af[kk & 1], bf[kk & 1]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        u32x4_t af[FM], bf[FN];
        read_frags(s, kk, af, bf);
        mfmas(af, bf);
      }
    }
  };

  // Main loop over the full k-slices, unrolled over the two LDS stages and
  // register sets so their offsets are constants.  Iteration kt: load slice
  // kt+2 into register set kt%2 (staged in the previous iteration), compute
  // slice kt from stage kt%2, stage slice kt+1 (set (kt+1)%2) into stage
  // (kt+1)%2.  A ragged last slice is staged and computed after the loop.
  const int nfull = p.K / BK;
  const bool ragged = (p.K % BK) != 0;
  uint16_t* const s0 = sm;
  uint16_t* const s1 = sm + STAGE;
  if (nfull > 0) {
    // Loads and stores below are unconditional (a slice index past the end is
    // clamped to the last full slice and its copy is never read): straight-line
    // code lets the compiler wait only for the loads of the slice being staged
    // instead of for every load in flight.
    const int last = nfull - 1;
    if (NSETS == 2) {
      load_full(0, 0);
      load_full(min(1, last), NSETS - 1);
      sstore(s0, 0);
      __syncthreads();
      int kt = 0;
      for (; kt + 2 <= nfull; kt += 2) {
        load_full(min(kt + 2, last), 0);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
        compute(s0);
        sstore(s1, NSETS - 1);
        __syncthreads();
        load_full(min(kt + 3, last), NSETS - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(s1);
        sstore(s0, 0);
        __syncthreads();
      }
      if (kt < nfull) {          // odd count: the last full slice sits in stage 0
        compute(s0);
        __syncthreads();
      }
    } else {
      // one register set: slice kt+1 is loaded while slice kt is computed
      load_full(0, 0);
      sstore(s0, 0);
      __syncthreads();
      int kt = 0;
      for (; kt + 2 <= nfull; kt += 2) {
        load_full(kt + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        compute(s0);
        sstore(s1, 0);
        __syncthreads();
        load_full(min(kt + 2, last), 0);
        __builtin_amdgcn_sched_barrier(0);
        compute(s1);
        sstore(s0, 0);
        __syncthreads();
      }
      if (kt < nfull) {
        compute(s0);
        __syncthreads();
      }
    }
  }
  if (ragged) {
    load_tail(nfull, 0);
    sstore(s0, 0);
    __syncthreads();
    compute(s0);
  }

  // ---- epilogue.  32x32 accumulator layout: element v of a lane is row
  // 8*(v/4) + 4*(lane/32) + v%4, column lane%32.
  uint16_t* C = static_cast<uint16_t*>(p.C);
  int nsat = 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lrow = wm * WROWS + 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
      const int m = tl.m0 + lrow;
      if (m >= tl.M) continue;
      uint16_t* crow = C + (tl.rb + m) * p.ldC;
      if (MODE == MODE_GATEUP) {
#pragma unroll
        for (int jn = 0; jn < FN / 2; ++jn) {
          const int col = tl.n0 + wn * WCOLS + 32 * jn + lr;
          if (col < p.Ncols) {
            const float a = acc[i][jn][v];
            const float u = acc[i][jn + FN / 2][v];
            crow[col] = f32_to_f16_sat_n(swiglu(a, u, p.clip), nsat);
            if (p.Su) {
              static_cast<uint16_t*>(p.Sa)[(tl.rb + m) * p.ldC + col] = f32_to_f16_sat(a);
              static_cast<uint16_t*>(p.Su)[(tl.rb + m) * p.ldC + col] = saved_up_bits(a, u, p.clip);
            }
          }
        }
      } else {
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) {
          const int col = tl.n0 + wn * WCOLS + 32 * jn + lr;
          if (col < p.Ncols) {
            float vv = acc[i][jn][v];
            if (MODE == MODE_RELU_UP && p.Su)
              static_cast<uint16_t*>(p.Su)[(tl.rb + m) * p.ldC + col] = f32_to_f16_sat(vv);
            if (MODE == MODE_RELU_UP) vv = fmaxf(vv, 0.f);
            crow[col] = f32_to_f16_sat_n(vv, nsat);
          }
        }
      }
    }
  }
  if (p.sat && nsat) atomicAdd(p.sat, nsat);
}

// ---------------------------------------------------------------------------
// bf16 grouped GEMM, direct-to-LDS variant for large groups.
//
// Same tile semantics as ffn_gemm_bf16 (C = A B^T over a BM x 256 tile, gate/up
// pairs, fp16 h and rows):
//  * NW = 4 waves (one per SIMD) in a 2 x 2 layout, each (BM/2) x 128 with up
//    to 256 fp32 accumulator values per lane, or NW = 8 waves (two per SIMD),
//    so one wave's copies and reads issue while the other's MFMAs run: a 4 x 2
//    layout of (BM/4) x 128 in the gate/up pass, a 2 x 4 layout of (BM/2) x 64
//    in the down pass (the W_down fragments a wave converts per MFMA stay as
//    few as with 4 waves);
//  * k-slices of BK (64: 128-byte rows) go from global memory straight into
//    LDS with global_load_lds_dwordx4: one wave instruction fills 8
//    consecutive 128-byte lines (1 KiB); each lane picks the global 16-byte
//    chunk whose swizzled position is its own, so the LDS image equals the
//    swizzled layout without passing through registers;
//  * the k-slices' token rows have two LDS stages and their weight rows three.
//    The weight rows of slice kt+2 are copied during the first two 16-wide
//    steps of slice kt and its token rows right after the barrier that ends
//    slice kt, while the last step of slice kt is still multiplying; the first
//    fragments of slice kt+1 are read in the same shadow, so the matrix cores
//    keep running across the barrier, and no step issues more than half a
//    slice's copies.
// In the down pass the bf16 W_down fragments are converted to fp16 after
// they are read from LDS (the data never passes through registers before),
// in the shadow of the preceding step's matrix instructions.
//
// One wave instruction: each lane copies 16 bytes from its global address to
// LDS at lds_base + 16 * lane.  Written as inline assembly so the compiler does
// not add its conservative wait for every such copy before each LDS read; the
// kernel waits for them itself (s_waitcnt vmcnt) before the barrier that
// publishes a stage.  The instruction has no register result.
__device__ __forceinline__ void g2lds16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

// 16 zero bytes in global memory: the source of the copies for k-chunks past
// the end of a ragged last slice.
__device__ const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

template <int MODE, int BM, int NW>
__global__ __launch_bounds__(64 * NW, 1) void ffn_gemm_dl(GemmParams p) {
  constexpr int BN = 256;
  constexpr int BK = 64;                     // k-slice: one 128-byte LDS line per staged row
  constexpr int KCH = BK / 8;                // 16-byte chunks per staged row
  constexpr int KS = BK / 16;                // 16-wide steps per slice
  constexpr int ROWS = BM + BN;              // staged rows per slice
  constexpr int NLD = ROWS / (8 * NW);       // copy instructions per thread per slice
  constexpr int JA = NLD * BM / ROWS;        // of which into token rows (then weight rows)
  // waves along the columns: 2, or 4 in the 8-wave down pass (each wave 128 rows
  // x 64 columns, so its W_down conversions per MFMA stay those of 4 waves)
  constexpr int WN = (MODE == MODE_DOWN && NW == 8) ? 4 : 2;
  constexpr int WM = NW / WN;                // waves along the rows
  constexpr int WROWS = BM / WM;
  constexpr int FM = WROWS / 32;
  constexpr int CT = (MODE == MODE_GATEUP) ? BN / 2 : BN;
  constexpr int WCOLS = CT / WN;
  // weight fragments of 32 rows: gate/up pairs (two of gate, the matching two of up)
  constexpr int FN = (MODE == MODE_GATEUP) ? 2 * WCOLS / 32 : WCOLS / 32;
  // LDS: two stages of token rows and three of weight rows (a slice's token
  // rows are copied one slice ahead, its weight rows two slices ahead)
  constexpr int SA = BM * 128;               // bytes of one stage of token rows
  constexpr int SW = BN * 128;               // bytes of one stage of weight rows
  constexpr int LDSB = 2 * SA + 3 * SW;
  constexpr int kWhole = 4;                  // copy-mode flag of step(): whole slices
  static_assert(BM % 64 == 0 && BM <= 256 && (NW == 4 || NW == 8) && WROWS >= 32, "tile rows");
  static_assert(JA * 8 * NW == BM && 2 * NLD <= 63, "copies per thread");
  static_assert(KS == 4, "slice steps");
  static_assert(LDSB <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[LDSB];

  const int ntn = (p.Ncols + CT - 1) / CT;
  const Tile tl = decode_tile(p.plan, p.G, ntn, BM, CT);
  if (!tl.ok) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool routed = tl.g < p.n_gather;
  const char* A = static_cast<const char*>(p.A);
  const int64_t eoff = (int64_t)(routed ? tl.g : tl.g - p.n_gather) * p.wstride * 2;
  const char* B0 = static_cast<const char*>(routed ? p.Br0 : p.Bs0) + eoff;
  const char* B1 = B0;
  if (MODE == MODE_GATEUP) B1 = static_cast<const char*>(routed ? p.Br1 : p.Bs1) + eoff;
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(lds) + wave * 1024;

  // ---- loaders: staged row r of a slice (token rows 0 .. BM-1, then weight
  // rows) is the 128-byte LDS line r of its part.  Copy instruction j of wave w
  // fills rows (NW*j + w) * 8 .. + 7; lane i writes row L = (NW*j + w) * 8 + i/8
  // at position i%8, which holds k-chunk (i%8) ^ swizzle(L); swizzle(L) depends
  // on i/8 and on w.
  const int lline = lane >> 3;
  const int gchunk = (lane & 7) ^ lline ^ (wave & 1);
  const char* src[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int r = (NW * j + wave) * 8 + lline;
    if (r < BM) {
      int m = tl.m0 + r;
      if (m >= tl.M) m = tl.M - 1;
      int64_t arow;
      if (MODE == MODE_DOWN) {
        arow = tl.rb + m;
      } else if (routed) {
        arow = p.token_of_row[tl.rb + m];
        arow = arow < 0 ? 0 : (arow >= p.n_tokens ? p.n_tokens - 1 : arow);
      } else {
        arow = tl.rb + m - (p.ident_row0 + (int64_t)(tl.g - p.n_gather) * p.n_tokens);
      }
      src[j] = A + arow * p.ldA * 2 + gchunk * 16;
    } else {
      const int n = r - BM;
      if (MODE == MODE_GATEUP) {
        int col = tl.n0 + (n & (CT - 1));
        if (col >= p.Ncols) col = p.Ncols - 1;
        src[j] = ((n < CT) ? B0 : B1) + (int64_t)col * p.K * 2 + gchunk * 16;
      } else {
        int col = tl.n0 + n;
        if (col >= p.Ncols) col = p.Ncols - 1;
        src[j] = B0 + (int64_t)col * p.K * 2 + gchunk * 16;
      }
    }
  }
  const int nfull = p.K / BK;
  const int nsl = nfull + ((p.K % BK) ? 1 : 0);   // slices; the last may be ragged
  // source of copy j of slice kt: in a ragged last slice the chunks at or past
  // K come from a zero chunk, so the products there vanish
  auto src_of = [&](int j, int kt) -> const char* {
    const bool ok = kt < nfull || kt * BK + gchunk * 8 < p.K;
    return ok ? src[j] + (int64_t)kt * BK * 2 : reinterpret_cast<const char*>(kZeroChunk);
  };
  // copy j of a slice: token-row copies (j < JA) of slice ka go to the stage
  // at LDS address ca, weight-row copies of slice kb to the stage at cb
  auto copy_one = [&](int j, uint32_t ca, uint32_t cb, int ka, int kb) {
    if (j < JA) g2lds16(src_of(j, ka), ca + NW * 1024 * j);
    else g2lds16(src_of(j, kb), cb + NW * 1024 * (j - JA));
  };
  // the same for slices known to be whole (no zero-chunk selection: fewer
  // instructions between the MFMAs)
  auto copy_whole = [&](int j, uint32_t ca, uint32_t cb, int ka, int kb) {
    if (j < JA) g2lds16(src[j] + (int64_t)ka * BK * 2, ca + NW * 1024 * j);
    else g2lds16(src[j] + (int64_t)kb * BK * 2, cb + NW * 1024 * (j - JA));
  };

  // ---- fragment reads: lane supplies row lr of a 32-row fragment and k-chunk
  // 2*kk + lh of the slice; fragment bases are multiples of 32 rows, so the
  // swizzle of the lane's line depends on lr alone
  // Waves w and w+4 share a SIMD.  With 8 waves the row bands are dealt so
  // that every SIMD holds one wave of rows 0-127 and one of rows 128-255: a
  // tile with at most 128 valid rows then keeps each SIMD busy with one wave,
  // while the waves without rows only copy and wait.
  const int wm = (NW == 8) ? (WN == 4 ? (wave >> 2) : 2 * (wave >> 2) + ((wave & 3) >> 1))
                            : wave % WM;
  const int wn = (NW == 8) ? (WN == 4 ? (wave & 3) : (wave & 1)) : wave / WM;
  const bool act = __builtin_amdgcn_readfirstlane(tl.m0 + wm * WROWS < tl.M ? 1 : 0) != 0;
  const int lr = lane & 31, lh = lane >> 5;
  const int lsw = lds_swizzle<1>(lr);
  int a_off[FM], b_off[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_off[i] = (wm * WROWS + 32 * i + lr) * 128;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int base;
    if constexpr (MODE == MODE_GATEUP)   // gate rows, then the matching up rows
      base = (j >> 1) * CT + wn * WCOLS + 32 * (j & 1);
    else
      base = wn * WCOLS + 32 * j;
    b_off[j] = (base + lr) * 128;              // within a stage of weight rows
  }
  int kq[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) kq[kk] = ((2 * kk + lh) ^ lsw) * 16;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // LDS offsets of the token rows and of the weight rows of slice kt
  auto ra_of = [&](int kt) { return (kt & 1) * SA; };
  auto rb_of = [&](int kt) { return 2 * SA + (kt % 3) * SW; };
  auto read_frags = [&](int ra, int rb, int kk, u32x4_t (&af)[FM], u32x4_t (&bf)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(lds + ra + a_off[i] + kq[kk]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = *reinterpret_cast<const u32x4_t*>(lds + rb + b_off[j] + kq[kk]);
  };
  // One 16-wide step on fragments (af, bf) with a fixed instruction order:
  // after MFMA m come the reads 2m and 2m+1 of the next step's fragments (into
  // na/nb, when RD; token rows at LDS offset ra, weight rows at rb) and this
  // MFMA's share of the copies (when DMA: token rows of slice dka to LDS
  // address ca, weight rows of slice dkb to cb), so loads and copies issue
  // while the matrix cores are busy and every fragment read has most of a step
  // to land.  ACT false: a wave without valid rows issues the copies only.
  auto step = [&](auto ACT, auto RD, auto DMA, const u32x4_t (&af)[FM], const u32x4_t (&bf)[FN],
                  int ra, int rb, int rkk, u32x4_t (&na)[FM], u32x4_t (&nb)[FN], uint32_t ca,
                  uint32_t cb, int dka, int dkb) {
    constexpr bool kAct = decltype(ACT)::value;
    constexpr bool kRd = decltype(RD)::value && kAct;
    // DMA: 0 none; 1 the token-row copies; 2 / 3 the first / second half of
    // the weight-row copies; plus kWhole when the slices copied are whole
    constexpr bool kCopyWhole = decltype(DMA)::value >= kWhole;
    constexpr int kDma = decltype(DMA)::value % kWhole;
    constexpr int JB = JA + (NLD - JA) / 2;
    constexpr int D0 = (kDma == 2) ? JA : (kDma == 3 ? JB : 0);
    constexpr int D1 = (kDma == 1) ? JA : (kDma == 2 ? JB : NLD);
    constexpr int ND = kDma ? D1 - D0 : 0;
    constexpr int NM = FM * FN, NR = FM + FN;
    const u32x4_t (&b)[FN] = bf;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int i = m / FN, j = m % FN;
      // weight fragment first: the block of C^T, so each lane ends up with
      // runs of 4 consecutive output columns of one row
      if constexpr (kAct) {
        if (MODE == MODE_DOWN)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8_t, b[j]), __builtin_bit_cast(f16x8_t, af[i]), acc[i][j],
              0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, b[j]), __builtin_bit_cast(bf16x8_t, af[i]), acc[i][j],
              0, 0, 0);
      }
      if constexpr (kRd) {
#pragma unroll
        for (int r = 2 * m; r < 2 * m + 2; ++r) {
          if (r < FM)
            na[r] = *reinterpret_cast<const u32x4_t*>(lds + ra + a_off[r] + kq[rkk]);
          else if (r < NR)
            nb[r - FM] = *reinterpret_cast<const u32x4_t*>(lds + rb + b_off[r - FM] + kq[rkk]);
        }
      }
      if constexpr (ND > 0) {
#pragma unroll
        for (int d = D0 + m * ND / NM; d < D0 + (m + 1) * ND / NM; ++d)
          if constexpr (kCopyWhole) copy_whole(d, ca, cb, dka, dkb);
          else copy_one(d, ca, cb, dka, dkb);
      }
      // down pass: the next step's W_down fragments become fp16 in the second
      // half of the step, once their reads have landed
      if constexpr (kRd && MODE == MODE_DOWN) {
        constexpr int H = NM / 2;
        if (m >= H) {
#pragma unroll
          for (int q = (m - H) * 4 * FN / (NM - H); q < (m - H + 1) * 4 * FN / (NM - H); ++q)
            nb[q / 4][q % 4] = bf16x2_to_f16x2(nb[q / 4][q % 4]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto convert_b = [&](u32x4_t (&bf)[FN]) {
    if (MODE == MODE_DOWN) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) bf[j][q] = bf16x2_to_f16x2(bf[j][q]);
    }
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  using D_NONE = std::integral_constant<int, 0>;

  // the slice loop, once with the matrix work (waves with rows) and once
  // without it (copies, waits and barriers only, in the same order)
  auto slice_loop = [&](auto ACT) {
    u32x4_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    // prologue: slices 0 and 1 (clamped to the last slice: copies into a
    // stage no slice uses are never read); wait for slice 0
    const uint32_t wb = lds_base + 2 * SA;
#pragma unroll
    for (int j = 0; j < NLD; ++j) copy_one(j, lds_base, wb, 0, 0);
#pragma unroll
    for (int j = 0; j < NLD; ++j)
      copy_one(j, lds_base + SA, wb + SW, min(1, nsl - 1), min(1, nsl - 1));
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");
    __syncthreads();
    if constexpr (decltype(ACT)::value) read_frags(ra_of(0), rb_of(0), 0, fa0, fb0);
    if constexpr (decltype(ACT)::value) convert_b(fb0);
    // Steady state over slices 0 .. nsl-2, slice kt's token rows in token stage
    // kt % 2 and its weight rows in weight stage kt % 3, its step-0 fragments
    // already in fa0/fb0.  Steps 0 and 1 each issue half of the weight-row
    // copies of slice kt+2 (into the weight stage that slice kt-1 freed);
    // step 2; then the wait for slice kt+1 and the barrier that publishes it and
    // frees token stage kt % 2 and weight stage kt % 3; then the last step of
    // slice kt, with the token-row copies of slice kt+2 and the first fragment
    // reads of slice kt+1 in its shadow.  Copies complete in issue order, so
    // the wait lets exactly the weight rows of slice kt+2 stay in flight.
    // Spreading the copies over three steps instead of issuing them together
    // after the barrier keeps the address queue from stalling the waves'
    // matrix instructions behind it.
    // The slices kt+2 < nfull copy whole slices (copy_whole); the last ones
    // may copy a ragged slice or clamped repeats (copy_one).
    auto slice = [&](auto WHOLE, int kt) {
      constexpr int w = decltype(WHOLE)::value ? kWhole : 0;
      using D_A = std::integral_constant<int, 1 + w>;
      using D_B1 = std::integral_constant<int, 2 + w>;
      using D_B2 = std::integral_constant<int, 3 + w>;
      const int ra = ra_of(kt), rb = rb_of(kt);
      const uint32_t cbw = lds_base + rb_of(kt + 2);
      const int kbw = min(kt + 2, nsl - 1);
      step(ACT, T_{}, D_B1{}, fa0, fb0, ra, rb, 1, fa1, fb1, 0u, cbw, 0, kbw);
      step(ACT, T_{}, D_B2{}, fa1, fb1, ra, rb, 2, fa0, fb0, 0u, cbw, 0, kbw);
      step(ACT, T_{}, D_NONE{}, fa0, fb0, ra, rb, 3, fa1, fb1, 0u, 0u, 0, 0);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD - JA) : "memory");
      __syncthreads();
      step(ACT, T_{}, D_A{}, fa1, fb1, ra_of(kt + 1), rb_of(kt + 1), 0, fa0, fb0,
           lds_base + ra, 0u, min(kt + 2, nsl - 1), 0);
    };
    int kt = 0;
    for (; kt + 1 < nsl && kt + 2 < nfull; ++kt) slice(T_{}, kt);
    for (; kt + 1 < nsl; ++kt) slice(F_{}, kt);
    // last slice
    const int ra = ra_of(nsl - 1), rb = rb_of(nsl - 1);
    step(ACT, T_{}, D_NONE{}, fa0, fb0, ra, rb, 1, fa1, fb1, 0u, 0u, 0, 0);
    step(ACT, T_{}, D_NONE{}, fa1, fb1, ra, rb, 2, fa0, fb0, 0u, 0u, 0, 0);
    step(ACT, T_{}, D_NONE{}, fa0, fb0, ra, rb, 3, fa1, fb1, 0u, 0u, 0, 0);
    step(ACT, F_{}, D_NONE{}, fa1, fb1, 0, 0, 0, fa0, fb0, 0u, 0u, 0, 0);
  };
  if (act) slice_loop(T_{});
  else slice_loop(F_{});
  // no copy may still be writing LDS when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue.  acc[i][j] holds the 32 x 32 block of C^T: element v of
  // lane (lr, lh) is row 32i + lr of the wave's block and column
  // 8*(v/4) + 4*lh + v%4 of fragment j.  Each lane packs its runs of 4 columns
  // (fp16) into LDS rows, 64 columns per pass, and the rows leave as 16-byte
  // stores.
  __syncthreads();   // every wave is done with the stages (copies were waited for)
  {
    constexpr int HC = 64;                       // columns per pass
    constexpr int PS = HC * 2 + 16;              // LDS row stride in bytes (padded)
    constexpr int NPASS = (MODE == MODE_GATEUP) ? 1 : FN / 2;
    constexpr int RDS = WROWS * HC * 2 / 1024;   // 16-byte reads per lane per pass
    static_assert(NW * WROWS * PS <= LDSB, "epilogue staging fits the stages");
    char* eb = lds + wave * (WROWS * PS);
    int nsat = 0;
    // WHAT: 0 = the pass's output (h or the expert row); 1 = the gate
    // pre-activation a (SwiGLU) or the up pre-activation before the ReLU;
    // 2 = the up pre-activation u (SwiGLU)
    auto emit = [&](auto WHAT, uint16_t* C) {
    constexpr int kWhat = decltype(WHAT)::value;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int vq = 0; vq < 4; ++vq) {
            uint32_t hb[4];   // fp16 bits
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              float h;
              if (MODE == MODE_GATEUP) {
                const float a = acc[i][jj][4 * vq + c], u = acc[i][jj + 2][4 * vq + c];
                h = swiglu(a, u, p.clip);
                hb[c] = kWhat == 0 ? f32_to_f16_sat(h)
                                   : (kWhat == 1 ? f32_to_f16_sat(a) : saved_up_bits(a, u, p.clip));
              } else {
                h = acc[i][2 * pass + jj][4 * vq + c];
                if (MODE == MODE_RELU_UP && kWhat == 0) h = fmaxf(h, 0.f);
                hb[c] = f32_to_f16_sat(h);
              }
            }
            uint2 pk;
            pk.x = hb[0] | (hb[1] << 16);
            pk.y = hb[2] | (hb[3] << 16);
            *reinterpret_cast<uint2*>(eb + (32 * i + lr) * PS + (32 * jj + 8 * vq + 4 * lh) * 2) =
                pk;
          }
      // LDS operations of one wave complete in order: the reads below see the
      // writes above
#pragma unroll
      for (int q = 0; q < RDS; ++q) {
        const int idx = q * 64 + lane;
        const int row = idx / (HC / 8), c8 = idx % (HC / 8);
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(eb + row * PS + c8 * 16);
        const int m = tl.m0 + wm * WROWS + row;
        const int col = tl.n0 + wn * WCOLS + pass * HC + c8 * 8;
        if (m < tl.M && col < p.Ncols) {
          *reinterpret_cast<u32x4_t*>(C + (tl.rb + m) * p.ldC + col) = val;
          // the range count reads the stored bits (padding rows and columns,
          // which repeat the last valid ones, are not stored)
          if constexpr (kWhat == 0)
            nsat += f16x2_at_limit(val[0]) + f16x2_at_limit(val[1]) + f16x2_at_limit(val[2]) +
                    f16x2_at_limit(val[3]);
        }
      }
    }
    };
    emit(std::integral_constant<int, 0>{}, static_cast<uint16_t*>(p.C));
    if (MODE != MODE_DOWN && p.Su) {
      // the pre-activations, for a backward pass (same staging, one more pass
      // each; the LDS operations of one wave complete in order)
      if constexpr (MODE == MODE_GATEUP) {
        emit(std::integral_constant<int, 1>{}, static_cast<uint16_t*>(p.Sa));
        emit(std::integral_constant<int, 2>{}, static_cast<uint16_t*>(p.Su));
      } else {
        emit(std::integral_constant<int, 1>{}, static_cast<uint16_t*>(p.Su));
      }
    }
    if (p.sat && nsat) atomicAdd(p.sat, nsat);
  }
}

// ---------------------------------------------------------------------------
// fp32 grouped GEMM on the vector ALUs (fp32 FMA, fp32 accumulation): the fp32
// workloads are small and latency-bound.  Tile 64 x 64 outputs, 256 threads with
// 4 x 4 outputs each (x2 for gate and up), k-slices of 16 through LDS.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_gemm_f32(GemmParams p) {
  constexpr int FBM = kF32BM, FBN = kF32BN, FBK = 16;
  constexpr int NB = (MODE == MODE_GATEUP) ? 2 : 1;
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[NB][FBK][FBN + 4];
  const int ntn = (p.Ncols + FBN - 1) / FBN;
  const Tile tl = decode_tile(p.plan, p.G, ntn, FBM, FBN);
  if (!tl.ok) return;
  const int tid = threadIdx.x;
  const bool routed = tl.g < p.n_gather;
  const float* A = static_cast<const float*>(p.A);
  const float* Bm[2];
  Bm[0] = static_cast<const float*>(routed ? p.Br0 : p.Bs0) +
          (int64_t)(routed ? tl.g : tl.g - p.n_gather) * p.wstride;
  Bm[1] = (MODE == MODE_GATEUP)
              ? static_cast<const float*>(routed ? p.Br1 : p.Bs1) +
                    (int64_t)(routed ? tl.g : tl.g - p.n_gather) * p.wstride
              : nullptr;

  // loader: 64 rows x 16 k = 1024 elements, 4 per thread: row = tid/4 + 64*0.., k = ...
  const int lk = tid & 15;
  const int lrow0 = tid >> 4;   // 0..15, rows lrow0 + 16*i
  const float* arow[4];
  const float* brow[NB][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = tl.m0 + lrow0 + 16 * i;
    if (m >= tl.M) m = tl.M - 1;
    int64_t r;
    if (MODE == MODE_DOWN) {
      r = tl.rb + m;
    } else if (routed) {
      r = p.token_of_row[tl.rb + m];
      r = r < 0 ? 0 : (r >= p.n_tokens ? p.n_tokens - 1 : r);
    } else {
      r = tl.rb + m - (p.ident_row0 + (int64_t)(tl.g - p.n_gather) * p.n_tokens);
    }
    arow[i] = A + r * p.ldA;
    int col = tl.n0 + lrow0 + 16 * i;
    if (col >= p.Ncols) col = p.Ncols - 1;
#pragma unroll
    for (int b = 0; b < NB; ++b) brow[b][i] = Bm[b] + (int64_t)col * p.K;
  }

  const int ty = tid >> 4, tx = tid & 15;
  float acc[NB][4][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.f;

  for (int k0 = 0; k0 < p.K; k0 += FBK) {
    const bool ok = k0 + lk < p.K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk][lrow0 + 16 * i] = ok ? arow[i][k0 + lk] : 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) Bs[b][lk][lrow0 + 16 * i] = ok ? brow[b][i][k0 + lk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float av[4], bv[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[b][j] = Bs[b][kk][tx * 4 + j];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(av[i], bv[b][j], acc[b][i][j]);
    }
    __syncthreads();
  }

  float* C = static_cast<float*>(p.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tl.m0 + ty * 4 + i;
    if (m >= tl.M) continue;
    float* crow = C + (tl.rb + m) * p.ldC;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tl.n0 + tx * 4 + j;
      if (col >= p.Ncols) continue;
      float v;
      if (MODE == MODE_GATEUP) {
        const float a = acc[0][i][j], u = acc[NB - 1][i][j];
        v = a / (1.0f + expf(-a)) * u;
        if (p.clip > 0.f) v = fminf(fmaxf(v, -p.clip), p.clip);
      } else if (MODE == MODE_RELU_UP) {
        v = fmaxf(acc[0][i][j], 0.f);
      } else {
        v = acc[0][i][j];
      }
      crow[col] = v;
    }
  }
}

struct GemmCfg {
  int bm, bn, bk, wm, wn, minb, nsets, fragdb;
  int dl;   // 1: ffn_gemm_dl (bm rows x 256, 2*wm waves; its own k-slices and stages)
};

// Tile configuration of the bf16 grouped GEMMs for one call (both passes use
// the same row tiling BM, since they share one tile plan).
//  * batches of at most 64 tokens (decode): 32-row tiles, so the matrix cores
//    do not multiply padding rows; the weights stream through LDS with two
//    slices in flight; the down pass uses 128-wide weight tiles (64-wide when
//    that gives fewer than two tiles per CU) so enough blocks run when d is
//    small relative to the CU count;
//  * groups averaging at least 128 rows: the direct-to-LDS 256 x 256 kernel
//    (8 waves for gate/up, 4 for down);
//  * otherwise 128-row tiles, 4 waves, two blocks per CU.
GemmCfg choose_cfg(const FfnCall& c, int mode) {
  const int64_t groups = c.n_gather + c.n_ident;
  const int64_t rows = c.routed_rows + c.n_ident * c.N;
  const int64_t avg = groups > 0 ? rows / groups : 0;
  if (c.N <= 64) {
    if (mode == MODE_DOWN) {
      // fewer than two 128-wide down tiles per CU (few experts of a wide
      // model, e.g. 8 x 4096): 64-wide tiles of 2 waves, four blocks per CU,
      // so every CU keeps loads in flight (measured -3% on mix-D's down pass)
      if ((int64_t)groups * ((c.d + 127) / 128) < 2 * kCus)
        return GemmCfg{32, 64, 64, 1, 2, 4, 2, 0, 0};
      return GemmCfg{32, 128, 64, 1, 4, 2, 2, 0, 0};
    }
    return GemmCfg{32, 256, 64, 1, 4, 2, 2, 0, 0};
  }
  // 8 waves, 2 per SIMD (one wave's copies hide behind the other's MFMAs):
  // gate/up 64 x 128 each, down 128 x 64 each (each wave's fp16 conversion of
  // W_down fragments is amortised over as many MFMAs as with 4 waves of 128 x
  // 128; measured 2-4% faster for the stage)
  if (avg >= 128) return GemmCfg{256, 256, 64, 4, 2, 1, 2, 0, 1};
  return GemmCfg{128, 256, 32, 2, 2, 2, 2, 0, 0};
}

// a configuration is usable by a pass if the gate/up fragments pair up
template <int MODE, int BNv, int WNv>
constexpr bool cfg_valid() {
  return MODE != MODE_GATEUP || ((BNv / WNv / 32) % 2 == 0 && BNv / WNv / 32 >= 2);
}

template <int MODE, int BMv, int BNv, int BKv, int WMv, int WNv, int MINBv, int NS, int FD>
void launch_bf16(const GemmParams& gp, int64_t blocks, hipStream_t s) {
  if constexpr (cfg_valid<MODE, BNv, WNv>())
    ffn_gemm_bf16<MODE, BMv, BNv, BKv, WMv, WNv, MINBv, NS, FD>
        <<<(unsigned)blocks, 64 * WMv * WNv, 0, s>>>(gp);
}

template <int MODE>
hipError_t launch_gemm(const GemmParams& gp, int dtype, const GemmCfg& cfg, int64_t max_mtiles,
                       hipStream_t s) {
  int CT;
  if (dtype == MOE_BF16) CT = (MODE == MODE_GATEUP) ? cfg.bn / 2 : cfg.bn;
  else CT = kF32BN;
  const int64_t ntn = (gp.Ncols + CT - 1) / CT;
  int64_t blocks = max_mtiles * ntn;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks <= 0) return hipSuccess;
  if (dtype == MOE_BF16 && cfg.dl) {
    // the instances launch_ffn plans: 256-row tiles on 8 waves, and the 128-row
    // remainder tiles of both passes on 4 waves
#define MOE_DL(a, w, used)                                                        \
  if (cfg.bm == a && 2 * cfg.wm == w) {                                           \
    if constexpr (used)                                                           \
      ffn_gemm_dl<MODE, a, w><<<(unsigned)blocks, 64 * w, 0, s>>>(gp);           \
    else                                                                          \
      return hipErrorInvalidValue;                                                \
  } else
    MOE_DL(256, 8, true)
    MOE_DL(128, 4, true)
    return hipErrorInvalidValue;
#undef MOE_DL
  } else if (dtype == MOE_BF16) {
#define MOE_TRY(a, n, b, c, d, e, f, g)                                                 \
  if (cfg.bm == a && cfg.bn == n && cfg.bk == b && cfg.wm == c && cfg.wn == d &&        \
      cfg.minb == e && cfg.nsets == f && cfg.fragdb == g)                               \
    launch_bf16<MODE, a, n, b, c, d, e, f, g>(gp, blocks, s);                           \
  else
    MOE_TRY(128, 256, 32, 2, 2, 2, 2, 0)
    MOE_TRY(32, 256, 64, 1, 4, 2, 2, 0)
    MOE_TRY(32, 128, 64, 1, 4, 2, 2, 0)
    MOE_TRY(32, 64, 64, 1, 2, 4, 2, 0)
    return hipErrorInvalidValue;
#undef MOE_TRY
  } else {
    ffn_gemm_f32<MODE><<<(unsigned)blocks, 256, 0, s>>>(gp);
  }
  return hipGetLastError();
}

}  // namespace

// Upper bound on the m-tiles of a call: each routed group adds at most one
// partial tile beyond routed_rows / bm.
static int64_t max_mtiles(const FfnCall& c, int bm) {
  int64_t t = 0;
  if (c.n_gather > 0) t += (c.routed_rows + bm - 1) / bm + c.n_gather;
  t += (int64_t)c.n_ident * ((c.N + bm - 1) / bm);
  return t;
}

hipError_t launch_ffn(const FfnCall& c, hipStream_t s) {
  const int G = c.n_gather + c.n_ident;
  if (G <= 0 || c.N <= 0) return hipSuccess;
  const GemmCfg cfg_up =
      c.dtype == MOE_BF16 ? choose_cfg(c, MODE_GATEUP) : GemmCfg{kF32BM, kF32BN, 16, 1, 1, 1, 1, 0, 0};
  const GemmCfg cfg_dn =
      c.dtype == MOE_BF16 ? choose_cfg(c, MODE_DOWN) : GemmCfg{kF32BM, kF32BN, 16, 1, 1, 1, 1, 0, 0};
  const int bm = cfg_up.bm;
  // 256-row direct-to-LDS tiles: remainders of at most 128 rows run as
  // 128-row tiles from a second plan, so a group of 300 rows costs one full
  // and one half tile rather than two full ones.  Only with many groups: the
  // second launch needs enough remainder tiles to fill the chip (measured:
  // -3% time with 257 or 385 groups, +8% with 65).
  const bool split =
      !c.plan_ready && cfg_up.dl && bm == 256 && cfg_dn.dl && cfg_dn.bm == 256 && G >= 128;
  // remainder tiles: 128 rows on 4 waves in both passes.  (Leaving the gate/up
  // remainders in the main launch as tiles of at most 128 valid rows, which the
  // 8-wave kernel runs on one wave per SIMD, measured 1-2% slower for the stage.)
  const GemmCfg cfg_s{128, 256, 64, 2, 2, 1, 2, 0, 1};
  int32_t* plan_s = split ? c.plan + plan_stride(G) : nullptr;
  const int64_t mt = max_mtiles(c, bm);
  const int64_t mt_s = split ? (int64_t)G : 0;
  const int64_t rows_cap = c.routed_rows;
  auto mark = [&](int i) {
    if (c.marks[i]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(c.marks[i]), s);
  };
  mark(0);
  hipError_t err = hipSuccess;
  if (!c.plan_ready) {
    ffn_plan_kernel<<<1, 1024, 0, s>>>(c.offsets, c.n_gather, c.n_ident, c.N, rows_cap,
                                       c.identity_row0, bm, 128, c.plan, plan_s, c.sat);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  mark(1);

  GemmParams up{};
  up.A = c.x;
  up.token_of_row = c.token_of_row;
  up.plan = c.plan;
  up.G = G;
  up.n_gather = c.n_gather;
  up.K = c.d;
  up.Ncols = c.I;
  up.ldA = c.d;
  up.ldC = c.I;
  up.wstride = (int64_t)c.I * c.d;
  up.n_tokens = c.N;
  up.ident_row0 = c.identity_row0;
  up.clip = c.clip;
  up.C = c.h;
  up.Sa = c.save_a;
  up.Su = c.save_u;
  up.sat = c.dtype == MOE_BF16 ? c.sat : nullptr;
  if (c.activation == MOE_SWIGLU) {
    up.Br0 = c.wg; up.Br1 = c.wu; up.Bs0 = c.sg; up.Bs1 = c.su;
  } else {
    up.Br0 = c.wu; up.Bs0 = c.su;
  }
  auto gate_up = [&](const GemmParams& gp, const GemmCfg& cfg, int64_t tiles) {
    return c.activation == MOE_SWIGLU ? launch_gemm<MODE_GATEUP>(gp, c.dtype, cfg, tiles, s)
                                      : launch_gemm<MODE_RELU_UP>(gp, c.dtype, cfg, tiles, s);
  };
  mark(2);
  err = gate_up(up, cfg_up, mt);
  if (err == hipSuccess && split) {
    GemmParams us = up;
    us.plan = plan_s;
    err = gate_up(us, cfg_s, mt_s);
  }
  if (err != hipSuccess) return err;
  mark(3);

  GemmParams dn{};
  dn.A = c.h;
  dn.plan = c.plan;
  dn.G = G;
  dn.n_gather = c.n_gather;
  dn.K = c.I;
  dn.Ncols = c.d;
  dn.ldA = c.I;
  dn.ldC = c.d;
  dn.wstride = (int64_t)c.d * c.I;
  dn.n_tokens = c.N;
  dn.ident_row0 = c.identity_row0;
  dn.Br0 = c.wd;
  dn.Bs0 = c.sd;
  dn.C = c.y_rows;
  dn.sat = c.dtype == MOE_BF16 ? c.sat : nullptr;
  mark(4);
  err = launch_gemm<MODE_DOWN>(dn, c.dtype, cfg_dn, mt, s);
  if (err == hipSuccess && split) {
    GemmParams ds = dn;
    ds.plan = plan_s;
    err = launch_gemm<MODE_DOWN>(ds, c.dtype, cfg_s, mt_s, s);
  }
  mark(5);
  return err;
}

int ffn_plan_rows(const FfnCall& c) {
  return c.dtype == MOE_BF16 ? choose_cfg(c, MODE_GATEUP).bm : kF32BM;
}

hipError_t launch_ffn_plan(const int32_t* offsets, int n_gather, int n_ident, int64_t N,
                           int64_t rows_cap, int64_t ident_row0, int BM, int32_t* plan,
                           hipStream_t s) {
  ffn_plan_kernel<<<1, 1024, 0, s>>>(offsets, n_gather, n_ident, N, rows_cap, ident_row0, BM,
                                     BM, plan, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe
