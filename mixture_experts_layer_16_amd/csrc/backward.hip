// Backward pass of the layer: gradients of L = sum(dy * y) for the routing
// the forward pass decided (selection held fixed: top-k, capacity and reroute
// are piecewise constant, so the router is reached only through the gate
// weights -- the reason "Основы MoE" (ai.flicky.cc), "Как устроен MoE-слой",
// gives the Switch top-1 weight as p_i and not 1).
//
// Per row r of the forward's layout (token t, gate weight g; shared rows g=1):
//   a = x_t W_gate^T, u = x_t W_up^T            recomputed
//   du_h = dy_t W_down                           (h's gradient before g)
//   dg = <h, du_h>, dh = g du_h (0 where the clamp is active)
//   da = dh u silu'(a), du = dh silu(a)          (ReLU: du = dh [u > 0])
//   dW_down += (g dy_t)^T h, dW_gate += da^T x_t, dW_up += du^T x_t
//   dx_t += da W_gate + du W_up
// then the gate weights' gradient dg goes through the (renormalised) softmax
// or sigmoid to dz, dW_router = dz^T x and dx += dz W_router.
//
// The matrix products run on one bf16 MFMA grouped GEMM with register-staged
// loads that can transpose either operand into LDS (operands stored with the
// reduction index as the slow one), fp32 accumulation and fp32 results.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int BW_BN = 256;   // tile columns

// One operand of C[m][n] = sum_k A(m, k) B(n, k).
//   T == 0: element (i, k) at row(i)[k]   (k contiguous; i = m or n)
//   T == 1: element (i, k) at row(k)[i]   (i contiguous)
// row(r) = base + r' * ld, with base = p + g * gstride for routed groups and
// ps + (g - n_gather) * gstride for dense ones; r' = r, except for a dense
// group of an operand whose rows are tokens (dense_tok): r' = r - the group's
// first layout row.  Rows past an extent are clamped; k past K reads zero.
struct Operand {
  const uint16_t* p;
  const uint16_t* ps;
  int64_t gstride;
  int64_t ld;
  int dense_tok;
};

struct BwdGemmParams {
  Operand A, B, A2, B2;      // A2/B2: optional second product into the same C
  int two;                   // use A2/B2
  void* C;                   // row mode: float [rows][ldc]; weight mode: routed groups' matrices
  void* Cs;                  // weight mode: dense groups' matrices
  int out_bf16;              // weight mode: C / Cs are bf16 (partials stay float)
  int64_t ldc, c_gstride;
  int M, N, K, K2;           // extents (row mode: M from the plan; weight mode: K from it)
  int mode;                  // 0: tiles over the plan's rows; 1: K = a group's rows
  const int32_t* plan;       // tile_start[G+1], row_begin[G], rows[G]
  int G;
  int n_gather;              // groups below this are routed experts
  int64_t ident_row0, n_tokens;
  // weight mode: each dense group's rows are cut into `pieces` runs of at most
  // `kchunk` rows (so its tiles take about as long as the routed ones); with
  // more than one piece, piece q of dense group s writes its partial product
  // to Cpart + (s * pieces + q) * c_gstride, to be summed afterwards
  int pieces, kchunk;
  float* Cpart;
};

// ---------------------------------------------------------------------------
// Grouped GEMM with direct-to-LDS copies, either operand transposed.
//
// A block computes a BM x 256 tile of C with 8 waves (4 x 2, each (BM/4) x 128
// of v_mfma_f32_32x32x16_bf16 accumulators), k-slices of 64 in two LDS stages.
// Copies go from global memory straight into LDS (global_load_lds_dwordx4: one
// wave instruction fills 1 KiB = 8 lines of 128 bytes; each lane picks the
// 16-byte global chunk that belongs at its own position), so both layouts
// below are produced without passing through registers:
//   T == 0: one line per row (64 k), chunk c (k 8c .. 8c+7) at position
//           c ^ sw0(line);
//   T == 1: one k-row of the slice takes R/64 lines (R = 256 or BM rows of the
//           operand); quarter q (i 64q .. 64q+63) is line (R/64) k + (q ^ (k & 1))
//           and chunk c of it (i 64q + 8c ..) sits at position c ^ sw1(k).
// T == 0 fragments are one ds_read_b128 per lane.  T == 1 fragments are read
// transposed with ds_read_b64_tr_b16: in each 16-lane group, lane j names the
// 4 consecutive elements of k-row k0 + j/4 at i0 + 4 (j%4), and lane j
// receives element j%4 of lanes 4q + j/4, q = 0..3, i.e. k0 .. k0+3 of i0 + j
// -- two such reads give a lane its 8 consecutive k of one row of the
// fragment, the matrix-core operand layout.  Both swizzles keep the reads of
// a half wave on distinct banks.
//
// The schedule follows the forward kernels: each 16-wide step issues its
// MFMAs with the next step's fragment reads (and, in the last step of a
// slice, the copies of a later slice) between them; one barrier per slice;
// NS stages in a ring.  Results are float32: the B fragment is the first MFMA
// operand, so the accumulators hold C^T with runs of 4 consecutive columns per
// lane, which go through LDS to leave as whole 128-byte row segments.
__device__ __forceinline__ int sw0(int line) { return (line & 7) ^ ((line >> 3) & 1); }
__device__ __forceinline__ int sw1(int k) { return 2 * (k & 3); }

__device__ __forceinline__ void bw_g2lds16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}
__device__ const uint32_t kBwZero[4] = {0u, 0u, 0u, 0u};

template <int TA, int TB, int BM, int BK, int NW, int NS>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_gemm_dl(BwdGemmParams p) {
  constexpr int BN = BW_BN, KS = BK / 16;
  constexpr int LA = BM * BK / 64, LB = BN * BK / 64;   // 128-byte lines per operand and stage
  constexpr int SB = (LA + LB) * 128;          // bytes per stage
  constexpr int NLD = (LA + LB) / (8 * NW);    // copies per thread per slice
  constexpr int JA = LA / (8 * NW);            // the first JA copies are A's
  constexpr int WM = NW / 2;
  constexpr int WROWS = BM / WM, WCOLS = BN / 2;
  constexpr int FM = WROWS / 32, FN = WCOLS / 32;
  constexpr int NRA = FM * (TA ? 2 : 1), NRB = FN * (TB ? 2 : 1);   // read instructions
  static_assert(BM == 128 || BM == 256, "tile rows");
  static_assert(NW == 4 || NW == 8, "waves");
  static_assert(BK == 64 || (BK == 32 && TA == 1 && TB == 1), "k-slice (32: transposed operands)");
  static_assert(JA * 8 * NW == LA && NLD * 8 * NW == LA + LB, "copies cover the stage");
  static_assert(NS >= 2 && (NS - 1) * NLD <= 63 && KS % 2 == 0, "pipeline shape");
  static_assert(NS * SB <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[NS * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- tile decode
  int g, m0, n0, Mlim, Klim;
  int64_t rb;
  char* Cg = static_cast<char*>(p.C);   // this tile's output matrix (bytes)
  bool obf = false;                      // ... holds bf16 (else float)
  const int ntn = (p.N + BN - 1) / BN;
  if (p.mode == 0) {
    const int32_t* tile_start = p.plan;
    const int total = tile_start[p.G] * ntn;
    const int per = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= per) return;
    const int L = (blockIdx.x % kXcds) * per + slot;   // consecutive tiles on one XCD
    if (L >= total) return;
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] * ntn <= L) lo = mid; else hi = mid - 1;
    }
    g = lo;
    // within a group: super-rows of GM m-tiles, m-tile fastest inside one, so
    // the tiles running together on one XCD share weight rows (the large
    // operand) and a few row tiles
    constexpr int GM = 8;
    const int mtg = tile_start[g + 1] - tile_start[g];
    const int local = L - tile_start[g] * ntn;
    const int sr = local / (GM * ntn);
    const int rem = local - sr * GM * ntn;
    const int gm = min(GM, mtg - sr * GM);
    const int nt = rem / gm;
    m0 = (sr * GM + (rem - nt * gm)) * BM;
    n0 = nt * BN;
    rb = p.plan[p.G + 1 + g];
    Mlim = p.plan[p.G + 1 + p.G + g];
    Klim = p.K;
  } else {
    const int ntm = (p.M + BM - 1) / BM;
    const int per = ntm * ntn;
    // virtual groups: the routed experts, then the pieces of the dense groups;
    // they are dealt to the XCDs round-robin (XCD x takes x, x + 8, ...), all
    // tiles of one virtual group on one XCD, so the groups' different lengths
    // average out over the XCDs and each group's operands share one L2
    const int nv = p.n_gather + (p.G - p.n_gather) * p.pieces;
    const int slot = blockIdx.x / kXcds;
    const int gl = slot / per;
    const int gv = (int)(blockIdx.x % kXcds) + kXcds * gl;
    if (gv >= nv) return;
    const int local = slot - gl * per;
    // the smaller operand's tiles vary fastest, so it stays in L2 while the
    // larger one streams through once
    if (p.M <= p.N) {
      m0 = (local % ntm) * BM;
      n0 = (local / ntm) * BN;
    } else {
      m0 = (local / ntn) * BM;
      n0 = (local % ntn) * BN;
    }
    if (gv < p.n_gather) {
      g = gv;
      rb = p.plan[p.G + 1 + g];
      Klim = p.plan[p.G + 1 + p.G + g];
      obf = p.out_bf16;
      Cg = static_cast<char*>(p.C) + g * p.c_gstride * (obf ? 2 : 4);
    } else {
      const int sd = (gv - p.n_gather) / p.pieces, q = (gv - p.n_gather) % p.pieces;
      g = p.n_gather + sd;
      rb = p.plan[p.G + 1 + g] + (int64_t)q * p.kchunk;
      Klim = p.plan[p.G + 1 + p.G + g];
      if (p.pieces > 1) Klim = min(p.kchunk, Klim - q * p.kchunk);
      obf = p.out_bf16 && p.pieces == 1;
      Cg = p.pieces == 1
               ? static_cast<char*>(p.Cs) + (int64_t)sd * p.c_gstride * (obf ? 2 : 4)
               : reinterpret_cast<char*>(p.Cpart + (int64_t)(sd * p.pieces + q) * p.c_gstride);
    }
    Mlim = p.M;
    if (Klim <= 0) {
      // no rows: the gradient of this group's weights (or piece) is zero
      for (int i = tid; i < BM * BN / 4; i += 64 * NW) {
        const int m = m0 + i / (BN / 4), n = n0 + 4 * (i % (BN / 4));
        if (m < p.M && n < p.N) {
          if (obf)
            *reinterpret_cast<uint2*>(Cg + ((int64_t)m * p.ldc + n) * 2) = make_uint2(0u, 0u);
          else
            *reinterpret_cast<float4*>(Cg + ((int64_t)m * p.ldc + n) * 4) =
                make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      return;
    }
  }
  const bool routed = g < p.n_gather;
  const int64_t dense_row0 = p.ident_row0 + (int64_t)(g - p.n_gather) * p.n_tokens;
  auto row_ptr = [&](const Operand& O, int64_t r) -> const char* {
    if (O.dense_tok && !routed) r -= dense_row0;
    const uint16_t* base =
        routed ? O.p + g * O.gstride : O.ps + (int64_t)(g - p.n_gather) * O.gstride;
    return reinterpret_cast<const char*>(base + r * O.ld);
  };

  const uint32_t lds_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(lds) + wave * 1024;
  const int lline = lane >> 3, lpos = lane & 7;

  // fragment read offsets (bytes within a stage) for step kk = 0; a step adds
  // 32 bytes (T == 0) or 16 k-rows (T == 1)
  const int wm = wave % WM, wn = wave / WM;
  const int lr = lane & 31, lh = lane >> 5;
  const int tg = lane >> 4, tj = lane & 15;
  auto tr_off = [&](int region, int lpk, int o, int h) {
    // element (k, o) with k = 8 (tg >> 1) + 4 h + tj / 4 and o + 16 (tg & 1) + 4 (tj & 3)
    const int k = 8 * (tg >> 1) + 4 * h + (tj >> 2);
    const int i = o + 16 * (tg & 1) + 4 * (tj & 3);
    const int q = i >> 6, c = (i >> 3) & 7, b = i & 7;
    return region + (lpk * k + (q ^ (k & 1))) * 128 + ((c ^ sw1(k)) << 4) + b * 2;
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto run = [&](const Operand& OA, const Operand& OB, int K) {
    // ---- copy sources.  Copy j of this wave fills stage line (NW j + wave) 8
    // + lane / 8 at position lane % 8.
    const char* src[NLD];
    int kof[NLD];            // k of the chunk (T == 0) or of the k-row (T == 1)
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const bool isA = j < JA;
      const int T = isA ? TA : TB;
      const int line = (NW * j + wave) * 8 + lline - (isA ? 0 : LA);
      const int rows = isA ? BM : BN;
      const Operand& O = isA ? OA : OB;
      const int lim = isA ? Mlim : p.N;
      const int i0 = isA ? m0 : n0;
      if (T == 0) {
        const int c = lpos ^ sw0(line);
        int i = i0 + line;
        if (i >= lim) i = lim - 1;
        const int64_t r = (isA && p.mode == 0) ? rb + i : (int64_t)i;
        src[j] = row_ptr(O, r) + c * 16;
        kof[j] = 8 * c;
      } else {
        const int lpk = rows / 64;
        const int k = line / lpk;
        const int q = (line % lpk) ^ (k & 1);
        const int c = lpos ^ sw1(k);
        int i = i0 + 64 * q + 8 * c;
        if (i >= lim) i = ((lim + 7) & ~7) - 8;
        const int64_t r = (p.mode == 1 ? rb : 0) + k;
        src[j] = row_ptr(O, r) + (int64_t)i * 2;
        kof[j] = k;
      }
    }
    const int64_t stepA = TA ? (int64_t)BK * OA.ld * 2 : BK * 2;   // bytes per slice
    const int64_t stepB = TB ? (int64_t)BK * OB.ld * 2 : BK * 2;
    const int nsl = (K + BK - 1) / BK;
    auto src_of = [&](int j, int kt) -> const char* {
      const bool ok = kt * BK + kof[j] < K;   // false for slices past the last
      return ok ? src[j] + kt * (j < JA ? stepA : stepB) : reinterpret_cast<const char*>(kBwZero);
    };
    auto issue_slice = [&](int st, int kt) {
      const uint32_t sb = lds_base + st * SB;
#pragma unroll
      for (int j = 0; j < NLD; ++j) bw_g2lds16(src_of(j, kt), sb + NW * 1024 * j);
    };

    int aoff[NRA], boff[NRB];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int o = wm * WROWS + 32 * i;
      if (TA == 0) {
        aoff[i] = (o + lr) * 128 + (((lh) ^ sw0(o + lr)) << 4);
      } else {
        aoff[2 * i] = tr_off(0, BM / 64, o, 0);
        aoff[2 * i + 1] = tr_off(0, BM / 64, o, 1);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int o = wn * WCOLS + 32 * j;
      if (TB == 0) {
        boff[j] = LA * 128 + (o + lr) * 128 + (((lh) ^ sw0(o + lr)) << 4);
      } else {
        boff[2 * j] = tr_off(LA * 128, BN / 64, o, 0);
        boff[2 * j + 1] = tr_off(LA * 128, BN / 64, o, 1);
      }
    }
    // step kk: T == 0 chunk 2 kk + lh (the swizzle is an XOR on the chunk:
    // (2kk + lh) ^ s = ((lh ^ s) ^ 2kk), so the offset moves by XOR 32 kk bytes);
    // T == 1: 16 k-rows further
    auto rd_a = [&](int i, int kk, const char* s) -> u32x4_t {
      if (TA == 0) {
        const int off = aoff[i] ^ (32 * kk);
        return *reinterpret_cast<const u32x4_t*>(s + off);
      } else {
        const int adv = 16 * (BM / 64) * 128 * kk;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)((__attribute__((address_space(3))) char*)(s) + aoff[2 * i] + adv));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)((__attribute__((address_space(3))) char*)(s) + aoff[2 * i + 1] + adv));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        return u32x4_t{l2.x, l2.y, h2.x, h2.y};
      }
    };
    auto rd_b = [&](int j, int kk, const char* s) -> u32x4_t {
      if (TB == 0) {
        const int off = boff[j] ^ (32 * kk);
        return *reinterpret_cast<const u32x4_t*>(s + off);
      } else {
        const int adv = 16 * (BN / 64) * 128 * kk;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)((__attribute__((address_space(3))) char*)(s) + boff[2 * j] + adv));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)((__attribute__((address_space(3))) char*)(s) + boff[2 * j + 1] + adv));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        return u32x4_t{l2.x, l2.y, h2.x, h2.y};
      }
    };
    auto read_frags = [&](int st, int kk, u32x4_t (&af)[FM], u32x4_t (&bf)[FN]) {
      const char* s = lds + st * SB;
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = rd_a(i, kk, s);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = rd_b(j, kk, s);
    };
    // one 16-wide step: MFMA m, then the next step's fragment m (when RD) and
    // this MFMA's share of the copies of slice dkt into stage dst (when DMA)
    auto step = [&](auto RD, auto DMA, const u32x4_t (&af)[FM], const u32x4_t (&bf)[FN],
                    int rst, int rkk, u32x4_t (&na)[FM], u32x4_t (&nb)[FN], int dst, int dkt) {
      constexpr bool kRd = decltype(RD)::value;
      constexpr bool kDma = decltype(DMA)::value;
      constexpr int NM = FM * FN, NF = FM + FN;
      const char* rs = lds + rst * SB;
      const uint32_t sb = lds_base + dst * SB;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int i = m / FN, j = m % FN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, bf[j]), __builtin_bit_cast(bf16x8_t, af[i]), acc[i][j],
            0, 0, 0);
        if constexpr (kRd) {
          // the NF fragments spread over the NM MFMAs
#pragma unroll
          for (int r = m * NF / NM; r < (m + 1) * NF / NM; ++r) {
            if (r < FM) na[r] = rd_a(r, rkk, rs);
            else nb[r - FM] = rd_b(r - FM, rkk, rs);
          }
        }
        if constexpr (kDma) {
#pragma unroll
          for (int d = m * NLD / NM; d < (m + 1) * NLD / NM; ++d)
            bw_g2lds16(src_of(d, dkt), sb + NW * 1024 * d);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;

    if (nsl <= 0) return;
    // NS-stage ring: slice kt lives in stage kt % NS.  Prologue: slices 0 ..
    // NS-1.  At the end of slice kt: wait for slice kt+1 (slices kt+2 ..
    // kt+NS-1 may still be in flight), the barrier that publishes it and frees
    // stage kt % NS, then the last 16-wide step of slice kt with the copies of
    // slice kt+NS into that stage and the first fragment reads of slice kt+1
    // in its shadow.  Slices past the last copy the zero chunk into stages no
    // slice reads, so every wait counts the same number of copies.
    u32x4_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    int st = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q) issue_slice(q, q);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * NLD) : "memory");
    __syncthreads();
    read_frags(0, 0, fa0, fb0);
    for (int kt = 0; kt + 1 < nsl; ++kt) {
      const int nx = (st + 1 == NS) ? 0 : st + 1;
#pragma unroll
      for (int kk = 0; kk + 1 < KS; ++kk) {
        if (kk % 2 == 0) step(T_{}, F_{}, fa0, fb0, st, kk + 1, fa1, fb1, 0, 0);
        else step(T_{}, F_{}, fa1, fb1, st, kk + 1, fa0, fb0, 0, 0);
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * NLD) : "memory");
      __syncthreads();
      step(T_{}, T_{}, fa1, fb1, nx, 0, fa0, fb0, st, kt + NS);
      st = nx;
    }
#pragma unroll
    for (int kk = 0; kk + 1 < KS; ++kk) {
      if (kk % 2 == 0) step(T_{}, F_{}, fa0, fb0, st, kk + 1, fa1, fb1, 0, 0);
      else step(T_{}, F_{}, fa1, fb1, st, kk + 1, fa0, fb0, 0, 0);
    }
    step(F_{}, F_{}, fa1, fb1, 0, 0, fa0, fb0, 0, 0);
    // every copy has landed and every wave is done with the stages before
    // they are refilled (second product) or the block ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  run(p.A, p.B, p.mode == 1 ? Klim : p.K);
  if (p.two) run(p.A2, p.B2, p.mode == 1 ? Klim : p.K2);

  // ---- store: acc[i][j] is the 32 x 32 block of C^T; element v of lane
  // (lr, lh) is row 32 i + lr and column 8 (v / 4) + 4 lh + v % 4 of fragment j,
  // so each lane holds runs of 4 consecutive columns
  {
    // through LDS (free: run() ended with a barrier after its last reads), one
    // 32-column fragment per pass, so each global store instruction writes
    // whole 128-byte row segments (measured: 8% less time for the backward on
    // the 256-expert layer than 32-byte pieces straight from the accumulators)
    constexpr int PS = 32 * 4 + 16;   // LDS row stride in bytes (padded)
    static_assert(NW * WROWS * PS <= NS * SB, "epilogue staging fits the stages");
    char* eb = lds + wave * (WROWS * PS);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          *reinterpret_cast<float4*>(eb + (32 * i + lr) * PS + (8 * vq + 4 * lh) * 4) =
              make_float4(acc[i][j][4 * vq], acc[i][j][4 * vq + 1], acc[i][j][4 * vq + 2],
                          acc[i][j][4 * vq + 3]);
      // the LDS operations of one wave complete in order: the reads see the
      // writes, and the next pass's writes come after these reads
      // non-temporal stores: the results are not read again by this kernel
      // (measured: about 1% less time for the backward)
      if (obf) {
        // bf16: 8 columns per lane, one 16-byte store (half the store
        // instructions of 4-column runs)
#pragma unroll
        for (int q = 0; q < WROWS / 16; ++q) {
          const int row = 16 * q + (lane >> 2), c8 = lane & 3;
          const float4 v0 = *reinterpret_cast<const float4*>(eb + row * PS + c8 * 32);
          const float4 v1 = *reinterpret_cast<const float4*>(eb + row * PS + c8 * 32 + 16);
          const int m = m0 + wm * WROWS + row;
          const int n = n0 + wn * WCOLS + 32 * j + 8 * c8;
          if (m < Mlim && n < p.N) {
            const int64_t e = (p.mode == 0 ? rb + m : (int64_t)m) * p.ldc + n;
            const u32x4_t b = {f32_to_bf16(v0.x) | ((uint32_t)f32_to_bf16(v0.y) << 16),
                               f32_to_bf16(v0.z) | ((uint32_t)f32_to_bf16(v0.w) << 16),
                               f32_to_bf16(v1.x) | ((uint32_t)f32_to_bf16(v1.y) << 16),
                               f32_to_bf16(v1.z) | ((uint32_t)f32_to_bf16(v1.w) << 16)};
            __builtin_nontemporal_store(b, reinterpret_cast<u32x4_t*>(Cg + e * 2));
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < WROWS / 8; ++q) {
          const int row = 8 * q + (lane >> 3), c4 = lane & 7;
          const float4 v = *reinterpret_cast<const float4*>(eb + row * PS + c4 * 16);
          const int m = m0 + wm * WROWS + row;
          const int n = n0 + wn * WCOLS + 32 * j + 4 * c4;
          if (m < Mlim && n < p.N) {
            const int64_t e = (p.mode == 0 ? rb + m : (int64_t)m) * p.ldc + n;
            __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<f32x4_t*>(Cg + e * 4));
          }
        }
      }
    }
  }
}

template <int TA, int TB, int BM, int BK = 64, int NW = 8, int NS = 2>
hipError_t launch_bwd_gemm(const BwdGemmParams& p, int64_t tiles, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  // the decode deals tiles to the XCDs in blocks of ceil(tiles / 8)
  const int64_t blocks = (tiles + kXcds - 1) / kXcds * kXcds;
  bwd_gemm_dl<TA, TB, BM, BK, NW, NS><<<(unsigned)blocks, 64 * NW, 0, s>>>(p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// elementwise steps

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double warp_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double warp_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

// dy (float32) -> bf16, 4 values per thread
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ a,
                                                      uint16_t* __restrict__ b, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(a)[i];
  uint2 o;
  o.x = f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
  o.y = f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
  reinterpret_cast<uint2*>(b)[i] = o;
}

// Routed rows of x and dy in the forward's row layout: xg[r] = x[t], dyg[r] =
// bf16(dy[t]) for t = token_of_row[r], r < offsets[E]; 8 columns per thread.
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dy,
    const int32_t* __restrict__ token_of_row, const int32_t* __restrict__ offsets, int E,
    int64_t N, int d, uint16_t* __restrict__ xg, uint16_t* __restrict__ dyg) {
  const int64_t r = blockIdx.x;
  if (r >= offsets[E]) return;
  int64_t t = token_of_row[r];
  t = t < 0 ? 0 : (t >= N ? N - 1 : t);
  for (int c = 8 * threadIdx.x; c < d; c += 8 * 256) {
    *reinterpret_cast<u32x4_t*>(xg + r * d + c) = *reinterpret_cast<const u32x4_t*>(x + t * d + c);
    const float4 a = *reinterpret_cast<const float4*>(dy + t * d + c);
    const float4 b = *reinterpret_cast<const float4*>(dy + t * d + c + 4);
    u32x4_t o;
    o[0] = f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
    o[1] = f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
    o[2] = f32_to_bf16(b.x) | ((uint32_t)f32_to_bf16(b.y) << 16);
    o[3] = f32_to_bf16(b.z) | ((uint32_t)f32_to_bf16(b.w) << 16);
    *reinterpret_cast<u32x4_t*>(dyg + r * d + c) = o;
  }
}

// slot (t*k + j) of each kept routed row
__global__ __launch_bounds__(256) void slot_of_row_kernel(const int32_t* __restrict__ row_of,
                                                          int32_t* __restrict__ slot, int64_t nk) {
  const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a >= nk) return;
  const int32_t r = row_of[a];
  if (r >= 0 && r < nk) slot[r] = (int32_t)a;
}

// Per layout row r (one block): from a = x W_gate^T, u = x W_up^T and
// du_h = dy W_down (all float32), the row's gate weight g (routed rows; 1 for
// the shared experts' rows):
//   h = clamp(silu(a) u) (SwiGLU) | max(u, 0) (ReLU)
//   dg_r = <h, du_h>
//   dh = g du_h, zero where the clamp is active
//   da = dh u silu'(a), du = dh silu(a)   (ReLU: du = dh [u > 0])
// writes g h, da, du as bf16 and dg_r as float32.
template <bool SAVED>
__global__ __launch_bounds__(256) void bwd_rows_kernel(
    const float* __restrict__ af, const float* __restrict__ uf, const uint16_t* __restrict__ a16,
    const uint16_t* __restrict__ u16, const float* __restrict__ dhu,
    const int32_t* __restrict__ slot, const float* __restrict__ topk_w,
    const int32_t* __restrict__ offsets, int E, int64_t routed_rows, int I, int swiglu,
    float clip, uint16_t* __restrict__ hg, uint16_t* __restrict__ da, uint16_t* __restrict__ du,
    float* __restrict__ dgr) {
  const int64_t r = blockIdx.x;
  float g = 1.f;
  if (r < routed_rows) {
    if (r >= offsets[E]) return;   // unused routed row
    g = topk_w[slot[r]];
  }
  const int64_t o = r * (int64_t)I;
  float part = 0.f;
  for (int i = 4 * threadIdx.x; i < I; i += 4 * 256) {
    const float4 d4 = *reinterpret_cast<const float4*>(dhu + o + i);
    float a[4] = {0.f, 0.f, 0.f, 0.f}, u[4];
    if (SAVED) {
      // the forward's fp16 pre-activations; an infinite u marks an element
      // the forward clamped (sign(u) sign(a) = sign of the clamped h)
      const uint2 u2 = *reinterpret_cast<const uint2*>(u16 + o + i);
      u[0] = f16_to_f32(u2.x & 0xffffu); u[1] = f16_to_f32(u2.x >> 16);
      u[2] = f16_to_f32(u2.y & 0xffffu); u[3] = f16_to_f32(u2.y >> 16);
      if (swiglu) {
        const uint2 a2 = *reinterpret_cast<const uint2*>(a16 + o + i);
        a[0] = f16_to_f32(a2.x & 0xffffu); a[1] = f16_to_f32(a2.x >> 16);
        a[2] = f16_to_f32(a2.y & 0xffffu); a[3] = f16_to_f32(a2.y >> 16);
      }
    } else {
      const float4 u4 = *reinterpret_cast<const float4*>(uf + o + i);
      u[0] = u4.x; u[1] = u4.y; u[2] = u4.z; u[3] = u4.w;
      if (swiglu) {
        const float4 a4 = *reinterpret_cast<const float4*>(af + o + i);
        a[0] = a4.x; a[1] = a4.y; a[2] = a4.z; a[3] = a4.w;
      }
    }
    const float dh_u[4] = {d4.x, d4.y, d4.z, d4.w};
    uint16_t ohg[4], oda[4], odu[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float h, dh, dA = 0.f, dU;
      if (swiglu) {
        const float sg = 1.f / (1.f + expf(-a[q]));
        const float act = a[q] * sg;
        bool pass;
        if (SAVED) {
          // the forward's own clamp decision (see the comment above)
          pass = !__builtin_isinf(u[q]);
          h = pass ? act * u[q] : ((u[q] < 0.f) != __builtin_signbit(a[q]) ? -clip : clip);
        } else {
          const float hpre = act * u[q];
          pass = !(clip > 0.f) || fabsf(hpre) <= clip;
          h = clip > 0.f ? fminf(fmaxf(hpre, -clip), clip) : hpre;
        }
        dh = pass ? g * dh_u[q] : 0.f;
        dU = pass ? dh * act : 0.f;
        dA = pass ? dh * u[q] * (sg * (1.f + a[q] * (1.f - sg))) : 0.f;
      } else {
        h = fmaxf(u[q], 0.f);
        dh = g * dh_u[q];
        dU = u[q] > 0.f ? dh : 0.f;
      }
      part += h * dh_u[q];
      ohg[q] = f32_to_bf16(g * h);
      oda[q] = f32_to_bf16(dA);
      odu[q] = f32_to_bf16(dU);
    }
    uint2 v;
    v.x = ohg[0] | ((uint32_t)ohg[1] << 16);
    v.y = ohg[2] | ((uint32_t)ohg[3] << 16);
    *reinterpret_cast<uint2*>(hg + o + i) = v;
    v.x = odu[0] | ((uint32_t)odu[1] << 16);
    v.y = odu[2] | ((uint32_t)odu[3] << 16);
    *reinterpret_cast<uint2*>(du + o + i) = v;
    if (swiglu) {
      v.x = oda[0] | ((uint32_t)oda[1] << 16);
      v.y = oda[2] | ((uint32_t)oda[3] << 16);
      *reinterpret_cast<uint2*>(da + o + i) = v;
    }
  }
  __shared__ float red[4];
  part = warp_sum(part);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) dgr[r] = (red[0] + red[1]) + (red[2] + red[3]);
}

// Gate-weight gradient to logit gradient, one wave per token (float64):
//   softmax, renormalised:  g = softmax over the chosen;  dz_j = g_j (dg_j - sum g dg)
//   softmax, raw p:         dz = p (dp - <p, dp>), dp = dg on the chosen, 0 elsewhere
//   sigmoid, renormalised:  ds_j = (dg_j - sum g dg) / sum s;  dz_j = ds_j s_j (1 - s_j)
//   sigmoid, raw:           dz_j = dg_j s_j (1 - s_j)
// dg_j is the row's dg for a kept slot and 0 for a dropped one.  Writes dz
// (float32 [N][E]) and its bf16 copy [N][Ep] (zero past E), and dg (nullable).
__global__ __launch_bounds__(256) void gate_bwd_kernel(
    const double* __restrict__ z, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_of, const float* __restrict__ dgr, float* __restrict__ dg_out,
    float* __restrict__ dz, uint16_t* __restrict__ dz16, int64_t N, int E, int Ep, int k,
    int sigmoid, int renorm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;
  const double* zt = z + t * E;
  int e = -1;
  double dgj = 0.0, zj = 0.0;
  if (lane < k) {
    const int32_t ei = idx[t * k + lane];
    const int32_t r = row_of[t * k + lane];
    if (ei >= 0 && ei < E) {
      e = ei;
      zj = zt[e];
      dgj = r >= 0 ? (double)dgr[r] : 0.0;
    }
    if (dg_out) dg_out[t * k + lane] = (float)dgj;
  }
  const bool on = e >= 0;
  double dj = 0.0;        // gradient of the chosen logit (the raw softmax adds to all)
  double M = 0.0, Zs = 1.0, sdp = 0.0;
  if (!sigmoid) {
    if (renorm) {
      const double m = warp_max_d(on ? zj : -INFINITY);
      const double ex = on ? exp(zj - m) : 0.0;
      const double S = warp_sum_d(ex);
      const double gj = S > 0.0 ? ex / S : 0.0;
      const double sgd = warp_sum_d(gj * dgj);
      dj = gj * (dgj - sgd);
    } else {
      double m = -INFINITY;
      for (int i = lane; i < E; i += 64) m = fmax(m, zt[i]);
      M = warp_max_d(m);
      double sm = 0.0;
      for (int i = lane; i < E; i += 64) sm += exp(zt[i] - M);
      Zs = warp_sum_d(sm);
      const double pj = on ? exp(zj - M) / Zs : 0.0;
      sdp = warp_sum_d(pj * dgj);
      dj = pj * dgj;   // plus p_j * (-sdp), added with the rest below
    }
  } else {
    const double sj = on ? 1.0 / (1.0 + exp(-zj)) : 0.0;
    double ds = dgj;
    if (renorm) {
      const double tot = warp_sum_d(sj);
      const double sgd = warp_sum_d(sj * dgj);
      ds = tot > 0.0 ? (dgj - sgd / tot) / tot : 0.0;
    }
    dj = ds * sj * (1.0 - sj);
  }
  const bool raw_soft = !sigmoid && !renorm;
  for (int i = lane; i < Ep; i += 64) {
    double v = 0.0;
    if (i < E && raw_soft) v = -(exp(zt[i] - M) / Zs) * sdp;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(e, j);
      const double dv = __shfl(dj, j);
      if (ej == i) v += dv;
    }
    if (i < E) dz[t * E + i] = (float)v;
    dz16[t * Ep + i] = i < E ? f32_to_bf16((float)v) : 0;
  }
}

// Column sums of dz [N][E] in a fixed order: per-block partials over token
// chunks (float64), then one pass over the partials.
__global__ __launch_bounds__(256) void colsum_partial_kernel(const float* __restrict__ dz,
                                                             double* __restrict__ part, int64_t N,
                                                             int E, int64_t chunk) {
  const int64_t t0 = (int64_t)blockIdx.y * chunk;
  const int64_t t1 = t0 + chunk < N ? t0 + chunk : N;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  double s = 0.0;
  for (int64_t t = t0; t < t1; ++t) s += dz[t * E + e];
  part[(int64_t)blockIdx.y * E + e] = s;
}
__global__ __launch_bounds__(256) void colsum_final_kernel(const double* __restrict__ part,
                                                           int nb, int E, float* __restrict__ out) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  double s = 0.0;
  for (int b = 0; b < nb; ++b) s += part[(int64_t)b * E + e];
  out[e] = (float)s;
}

// dx[t] += sum over t's kept slots j (slot order) of dxp[row_of[t*k+j]]
//          + sum over shared experts s of dxp[N*k + s*N + t]
__global__ __launch_bounds__(256) void dx_combine_kernel(const float* __restrict__ dxp,
                                                         const int32_t* __restrict__ row_of,
                                                         float* __restrict__ dx, int64_t N, int d,
                                                         int k, int S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int d4 = d / 4;
  if (i >= N * d4) return;
  const int64_t t = i / d4;
  const int c = (int)(i - t * d4) * 4;
  float4 acc = *reinterpret_cast<const float4*>(dx + t * d + c);
  for (int j = 0; j < k; ++j) {
    const int32_t r = row_of[t * k + j];
    if (r < 0) continue;
    const float4 v = *reinterpret_cast<const float4*>(dxp + (int64_t)r * d + c);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  for (int s_ = 0; s_ < S; ++s_) {
    const float4 v = *reinterpret_cast<const float4*>(dxp + (N * k + s_ * N + t) * d + c);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *reinterpret_cast<float4*>(dx + t * d + c) = acc;
}

// out[s][i] = sum over q (in order) of part[s][q][i]; n (a multiple of 4)
// elements per matrix, P pieces, blockIdx.y = s; out float or (BF16) bf16
template <bool BF16>
__global__ __launch_bounds__(256) void reduce_pieces_kernel(const float* __restrict__ part,
                                                            int P, int64_t n, void* out,
                                                            int64_t out_stride) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float* src = part + (int64_t)blockIdx.y * P * n + i;
  float4 a = *reinterpret_cast<const float4*>(src);
  for (int q = 1; q < P; ++q) {
    const float4 b = *reinterpret_cast<const float4*>(src + (int64_t)q * n);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  const int64_t o = (int64_t)blockIdx.y * out_stride + i;
  if (BF16)
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) =
        make_uint2(f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16),
                   f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16));
  else
    *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = a;
}

inline unsigned blocks_of(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }
// Dense groups' rows per weight-gradient piece: the experts' (shared) and the
// router's (whose single group has all N rows).
constexpr int kExpertChunk = 2048, kRouterChunk = 512, kMaxPieces = 32;
inline int pieces_of(int64_t N, int chunk) {
  const int64_t p = (N + chunk - 1) / chunk;
  return (int)(p < 1 ? 1 : (p > kMaxPieces ? kMaxPieces : p));
}
inline int chunk_of(int64_t N, int chunk) {
  const int P = pieces_of(N, chunk);
  return (int)(((N + P - 1) / P + 31) / 32 * 32);   // rows per piece, a multiple of 32
}
inline int64_t colsum_blocks(int64_t N) {
  const int64_t nb = (N + 255) / 256;
  return nb < 1 ? 1 : (nb > 1024 ? 1024 : nb);
}

}  // namespace

BwdLayout bwd_ws_layout(const moe_problem* p) {
  const size_t N = (size_t)p->n_tokens, E = (size_t)p->n_experts, k = (size_t)p->top_k;
  const size_t S = (size_t)p->n_shared, d = (size_t)p->d_model, I = (size_t)p->d_expert;
  const size_t nk = N * k, R = nk + N * S, Ep = (E + 7) / 8 * 8;
  const bool swiglu = p->activation == MOE_SWIGLU;
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes ? (bytes + 255) / 256 : 1) * 256;
    return o;
  };
  L.plan = take(plan_bytes((int)(E + S)));
  L.plan_r = take(plan_bytes(1));
  L.slot = take(nk * 4);
  L.dy16 = take(N * d * 2);
  L.xg = take(nk * d * 2);
  L.dyg = take(nk * d * 2);
  L.af = swiglu ? take(R * I * 4) : 0;
  L.uf = take(R * I * 4);
  L.dhu = take(R * I * 4);
  L.hg = take(R * I * 2);
  L.da = swiglu ? take(R * I * 2) : 0;
  L.du = take(R * I * 2);
  L.dgr = take(R * 4);
  L.dxp = take(R * d * 4);
  L.dz = take(N * E * 4);
  L.dz16 = take(N * Ep * 2);
  L.colsum = take((size_t)colsum_blocks((int64_t)N) * E * 8);
  {
    // partial weight gradients of the dense groups' pieces
    const size_t pe = S ? (size_t)pieces_of((int64_t)N, kExpertChunk) : 0;
    const size_t pr = (size_t)pieces_of((int64_t)N, kRouterChunk);
    const size_t a = pe > 1 ? S * pe * d * I : 0;
    const size_t b = pr > 1 ? pr * E * d : 0;
    L.part = take((a > b ? a : b) * 4);
  }
  L.total = off;
  return L;
}

hipError_t launch_backward(const BwdCall& c, hipStream_t s) {
  const int64_t N = c.N;
  const int d = c.d, I = c.I, E = c.E, k = c.k, S = c.S;
  const int Ep = (E + 7) / 8 * 8;
  const int64_t nk = N * k, R = nk + N * S;
  const int G = E + S;
  const bool swiglu = c.activation == MOE_SWIGLU;
  char* base = static_cast<char*>(c.ws);
  const BwdLayout& L = c.L;
  int32_t* plan = reinterpret_cast<int32_t*>(base + L.plan);
  int32_t* plan_r = reinterpret_cast<int32_t*>(base + L.plan_r);
  int32_t* slot = reinterpret_cast<int32_t*>(base + L.slot);
  uint16_t* dy16 = reinterpret_cast<uint16_t*>(base + L.dy16);
  uint16_t* xg = reinterpret_cast<uint16_t*>(base + L.xg);
  uint16_t* dyg = reinterpret_cast<uint16_t*>(base + L.dyg);
  float* af = swiglu ? reinterpret_cast<float*>(base + L.af) : nullptr;
  float* uf = reinterpret_cast<float*>(base + L.uf);
  float* dhu = reinterpret_cast<float*>(base + L.dhu);
  uint16_t* hg = reinterpret_cast<uint16_t*>(base + L.hg);
  uint16_t* da = swiglu ? reinterpret_cast<uint16_t*>(base + L.da) : nullptr;
  uint16_t* du = reinterpret_cast<uint16_t*>(base + L.du);
  float* dgr = reinterpret_cast<float*>(base + L.dgr);
  float* dxp = reinterpret_cast<float*>(base + L.dxp);
  float* dz = c.dz_out ? c.dz_out : reinterpret_cast<float*>(base + L.dz);
  uint16_t* dz16 = reinterpret_cast<uint16_t*>(base + L.dz16);
  double* colsum = reinterpret_cast<double*>(base + L.colsum);
  const uint16_t* x = static_cast<const uint16_t*>(c.x);
  auto W = [](const void* q) { return static_cast<const uint16_t*>(q); };
  hipError_t err;
#define MOE_CHK(e)                     \
  do {                                 \
    err = (e);                         \
    if (err != hipSuccess) return err; \
  } while (0)

  auto mark = [&](int i) {
    if (c.marks[i]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(c.marks[i]), s);
  };
  // Row tiles of BM = 256 rows when the groups are large, else 128 (a group
  // of r rows costs ceil(r / BM) tiles).
  const int bm = (R / G >= 512) ? 256 : 128;
  const int bmr = N >= 512 ? 256 : 128;
  // tile plans: experts + shared experts over the forward's row layout, and
  // one dense group of N rows for the router products
  mark(2 * MOE_BSTAGE_PREP);
  MOE_CHK(launch_ffn_plan(c.offsets, E, S, N, nk, nk, bm, plan, s));
  MOE_CHK(launch_ffn_plan(nullptr, 0, 1, N, 0, 0, bmr, plan_r, s));
  if (S > 0) {
    to_bf16_kernel<<<blocks_of(N * d / 4, 256), 256, 0, s>>>(c.dy, dy16, N * d / 4);
    MOE_CHK(hipGetLastError());
  }
  gather_rows_kernel<<<(unsigned)nk, 256, 0, s>>>(x, c.dy, c.token_of_row, c.offsets, E, N, d,
                                                  xg, dyg);
  MOE_CHK(hipGetLastError());
  slot_of_row_kernel<<<blocks_of(nk, 256), 256, 0, s>>>(c.row_of, slot, nk);
  MOE_CHK(hipGetLastError());

  BwdGemmParams q{};
  q.plan = plan;
  q.G = G;
  q.n_gather = E;
  q.ident_row0 = nk;
  q.n_tokens = N;
  // tiles of the row-mode products: at most one partial tile per group
  const int64_t row_tiles = (nk + bm - 1) / bm + E + S * ((N + bm - 1) / bm);
  auto tn = [](int n) { return (int64_t)((n + BW_BN - 1) / BW_BN); };
#ifndef MOE_BWD_RNS
#define MOE_BWD_RNS 2, 3
#endif
  auto row_gemm = [&](auto TBc, const BwdGemmParams& pp, int64_t tiles) {
    constexpr int TB_ = decltype(TBc)::value;
    constexpr int ns[2] = {MOE_BWD_RNS};   // stages for 256- and 128-row tiles
    return bm == 256 ? launch_bwd_gemm<0, TB_, 256, 64, 8, ns[0]>(pp, tiles, s)
                     : launch_bwd_gemm<0, TB_, 128, 64, 8, ns[1]>(pp, tiles, s);
  };
  using TN = std::integral_constant<int, 0>;
  using TT = std::integral_constant<int, 1>;
  // routed rows come from the gathered copies, dense (shared-expert) rows from
  // the token arrays
  const Operand xin{xg, x, 0, d, 1};
  const Operand dyin{dyg, dy16, 0, d, 1};
  auto Wop = [&](const void* r_, const void* s_, int64_t ld) {
    return Operand{W(r_), W(s_), (int64_t)I * d, ld, 0};
  };

  mark(2 * MOE_BSTAGE_PREP + 1);
  // recompute a = x W_gate^T and u = x W_up^T per row (unless the forward
  // saved them)
  mark(2 * MOE_BSTAGE_RECOMPUTE);
  const bool saved = c.act_u != nullptr;
  q.mode = 0;
  q.K = d;
  q.N = I;
  q.ldc = I;
  q.A = xin;
  if (!saved) {
    if (swiglu) {
      q.B = Wop(c.wg, c.sg, d);
      q.C = af;
      MOE_CHK(row_gemm(TN{}, q, row_tiles * tn(I)));
    }
    q.B = Wop(c.wu, c.su, d);
    q.C = uf;
    MOE_CHK(row_gemm(TN{}, q, row_tiles * tn(I)));
  }
  mark(2 * MOE_BSTAGE_RECOMPUTE + 1);
  // du_h = dy W_down (W_down [d][I]: the reduction index is its row)
  mark(2 * MOE_BSTAGE_DH);
  q.A = dyin;
  q.B = Wop(c.wd, c.sd, I);
  q.C = dhu;
  MOE_CHK(row_gemm(TT{}, q, row_tiles * tn(I)));

  mark(2 * MOE_BSTAGE_DH + 1);
  mark(2 * MOE_BSTAGE_ROWS);
  if (saved)
    bwd_rows_kernel<true><<<(unsigned)R, 256, 0, s>>>(af, uf, c.act_a, c.act_u, dhu, slot,
                                                      c.topk_w, c.offsets, E, nk, I,
                                                      swiglu ? 1 : 0, c.clip, hg, da, du, dgr);
  else
    bwd_rows_kernel<false><<<(unsigned)R, 256, 0, s>>>(af, uf, nullptr, nullptr, dhu, slot,
                                                       c.topk_w, c.offsets, E, nk, I,
                                                       swiglu ? 1 : 0, c.clip, hg, da, du, dgr);
  MOE_CHK(hipGetLastError());

  mark(2 * MOE_BSTAGE_ROWS + 1);
  // weight gradients, one group per expert: K = the group's rows
  mark(2 * MOE_BSTAGE_WGRAD);
  q.mode = 1;
  const Operand hgin{hg, hg, 0, I, 0};
  const Operand dain{da, da, 0, I, 0};
  const Operand duin{du, du, 0, I, 0};
#ifndef MOE_BWD_WCFG
#define MOE_BWD_WCFG 256, 32, 8, 3
#endif
  float* part = reinterpret_cast<float*>(base + L.part);
  q.pieces = S ? pieces_of(N, kExpertChunk) : 1;
  q.kchunk = S ? chunk_of(N, kExpertChunk) : 0;
  q.Cpart = part;
  // launch over the virtual groups (routed experts, then the dense pieces),
  // then sum the pieces of each dense group
  auto wgemm = [&](const BwdGemmParams& pp, int M, int Nn) {
    constexpr int cfg[4] = {MOE_BWD_WCFG};   // tile rows, k-slice, waves, stages
    const int nv = pp.n_gather + (pp.G - pp.n_gather) * pp.pieces;
    const int64_t tiles = (int64_t)(nv + kXcds - 1) / kXcds * kXcds *
                          ((M + cfg[0] - 1) / cfg[0]) * tn(Nn);
    hipError_t e = launch_bwd_gemm<1, 1, cfg[0], cfg[1], cfg[2], cfg[3]>(pp, tiles, s);
    if (e != hipSuccess || pp.pieces == 1 || pp.G == pp.n_gather) return e;
    const int64_t n = (int64_t)M * Nn;
    const dim3 grid(blocks_of(n / 4, 256), (unsigned)(pp.G - pp.n_gather));
    if (pp.out_bf16)
      reduce_pieces_kernel<true><<<grid, 256, 0, s>>>(pp.Cpart, pp.pieces, n, pp.Cs,
                                                      pp.c_gstride);
    else
      reduce_pieces_kernel<false><<<grid, 256, 0, s>>>(pp.Cpart, pp.pieces, n, pp.Cs,
                                                       pp.c_gstride);
    return hipGetLastError();
  };
  // dW_down[e] = sum_r dy_t^T (g h_r)   ([d][I])
  q.M = d; q.N = I; q.ldc = I; q.c_gstride = (int64_t)d * I;
  q.out_bf16 = c.dw_bf16;
  q.A = dyin; q.B = hgin; q.C = c.dw_down; q.Cs = c.dws_down;
  MOE_CHK(wgemm(q, d, I));
  // dW_gate[e] = sum_r da_r^T x_t, dW_up[e] = sum_r du_r^T x_t   ([I][d])
  q.M = I; q.N = d; q.ldc = d; q.c_gstride = (int64_t)I * d;
  q.B = xin;
  if (swiglu) {
    q.A = dain; q.C = c.dw_gate; q.Cs = c.dws_gate;
    MOE_CHK(wgemm(q, I, d));
  }
  q.A = duin; q.C = c.dw_up; q.Cs = c.dws_up;
  MOE_CHK(wgemm(q, I, d));

  mark(2 * MOE_BSTAGE_WGRAD + 1);
  // per-row input gradient dx_r = da W_gate + du W_up ([R][d])
  mark(2 * MOE_BSTAGE_DX);
  q.mode = 0;
  q.N = d; q.ldc = d; q.K = I; q.K2 = I;
  q.C = dxp; q.Cs = nullptr;
  q.out_bf16 = 0;
  if (swiglu) {
    q.A = dain;
    q.B = Wop(c.wg, c.sg, d);
    q.A2 = duin;
    q.B2 = Wop(c.wu, c.su, d);
    q.two = 1;
  } else {
    q.A = duin;
    q.B = Wop(c.wu, c.su, d);
    q.two = 0;
  }
  MOE_CHK(row_gemm(TT{}, q, row_tiles * tn(d)));
  q.two = 0;

  // router: dz from the gate weights' gradient
  gate_bwd_kernel<<<blocks_of(N, 4), 256, 0, s>>>(c.logits, c.topk_idx, c.row_of, dgr, c.dg_out,
                                                  dz, dz16, N, E, Ep, k, c.gating, c.renormalize);
  MOE_CHK(hipGetLastError());
  // dx = dz W_router (written), then the expert rows are added
  BwdGemmParams qr{};
  qr.plan = plan_r;
  qr.G = 1;
  qr.n_gather = 0;
  qr.ident_row0 = 0;
  qr.n_tokens = N;
  qr.mode = 0;
  qr.K = E;
  qr.N = d;
  qr.ldc = d;
  qr.A = Operand{dz16, dz16, 0, Ep, 0};
  qr.B = Operand{W(c.wr), W(c.wr), 0, d, 0};
  qr.C = c.dx;
  const int64_t rtiles = ((N + bmr - 1) / bmr) * tn(d);
  MOE_CHK(bmr == 256 ? (launch_bwd_gemm<0, 1, 256>(qr, rtiles, s))
                     : (launch_bwd_gemm<0, 1, 128>(qr, rtiles, s)));
  // dW_router = dz^T x ([E][d])
  qr.mode = 1;
  qr.M = E;
  qr.N = d;
  qr.ldc = d;
  qr.B = Operand{x, x, 0, d, 0};
  qr.C = c.dw_router;
  qr.Cs = c.dw_router;
  qr.out_bf16 = c.dw_bf16;
  qr.c_gstride = (int64_t)E * d;
  qr.pieces = pieces_of(N, kRouterChunk);
  qr.kchunk = chunk_of(N, kRouterChunk);
  qr.Cpart = part;
  MOE_CHK(wgemm(qr, E, d));
  if (c.d_logit_bias) {
    const int64_t nb = colsum_blocks(N);
    const int64_t chunk = (N + nb - 1) / nb;
    colsum_partial_kernel<<<dim3(blocks_of(E, 256), (unsigned)nb), 256, 0, s>>>(dz, colsum, N, E,
                                                                                 chunk);
    MOE_CHK(hipGetLastError());
    colsum_final_kernel<<<blocks_of(E, 256), 256, 0, s>>>(colsum, (int)nb, E, c.d_logit_bias);
    MOE_CHK(hipGetLastError());
  }
  dx_combine_kernel<<<blocks_of(N * d / 4, 256), 256, 0, s>>>(dxp, c.row_of, c.dx, N, d, k, S);
  MOE_CHK(hipGetLastError());
  mark(2 * MOE_BSTAGE_DX + 1);
#undef MOE_CHK
  return hipSuccess;
}

}  // namespace moe
