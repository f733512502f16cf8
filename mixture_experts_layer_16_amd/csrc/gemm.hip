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
    int64_t rows_cap, int64_t ident_row0, int BM, int32_t* __restrict__ plan) {
  __shared__ int32_t mt[2 * 1024];
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
    row_begin[g] = (int32_t)rb;
    rows[g] = (int32_t)r;
    mt[g] = (int32_t)((r + BM - 1) / BM);
  }
  __syncthreads();
  const int total = block_exclusive_scan_1024(mt, G, tmp);
  for (int g = threadIdx.x; g < G; g += blockDim.x) tile_start[g] = mt[g];
  if (threadIdx.x == 0) tile_start[G] = total;
}

struct Tile {
  int g, m0, n0, M;
  int64_t rb;
  bool ok;
};

// Block -> tile.  Tiles are ordered (group, n-tile, m-tile) so the m-tiles that
// share one weight slab are consecutive; consecutive tiles go to the same XCD
// (blocks are dealt to the 8 XCDs round-robin), so a slab is fetched into that
// XCD's L2 once and reused by its m-tiles.
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
  const int nt = local / mtg;
  const int mtile = local - nt * mtg;
  t.g = g;
  t.m0 = mtile * BM;
  t.n0 = nt * CT;
  t.M = plan[G + 1 + G + g];
  t.rb = plan[G + 1 + g];
  t.ok = true;
  return t;
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
  float clip;
};

// ---------------------------------------------------------------------------
// bf16 grouped GEMM on the matrix cores.
//
// C[m][n] = sum_k A[m][k] * B[n][k]  (both operands contiguous along k).
// Tile 128 rows x 256 weight rows, k-slices of 64 staged in LDS (double
// buffered, 96 KiB), 4 waves in a 2x2 layout, each wave 64 rows x 128 weight
// rows = 2 x 4 v_mfma_f32_32x32x16_bf16 accumulators.  In the gate/up pass the
// 256 weight rows are 128 gate rows and the matching 128 up rows, so one lane
// holds the gate and up value of the same output element and the SwiGLU (and
// clip) is applied in registers before h is written once, in fp16.
// LDS rows are 128 bytes; the 16-byte chunk c of row r sits at chunk c^(r&7) so
// that the 32 rows read by one MFMA operand fetch spread over all banks.
//
// Number formats.  The gate/up pass multiplies bf16 x and bf16 weights; its
// result h is stored in fp16, whose 11-bit significand rounds 8x finer than
// bf16 (|h| is far inside fp16's range; the conversion saturates at +-65504).
// The down pass therefore runs on the fp16 matrix cores: the bf16 W_down tile is
// converted to fp16 while it is staged into LDS -- exact for every bf16 value in
// fp16's normal range, and within 2^-24 absolute below it.  Expert output rows
// are written in fp16 as well.  With bf16 h and rows the rounding alone would
// use most of the 2e-2 * RMS(y) error budget; with fp16 it uses about a tenth.
constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int STAGE = (BM + BN) * BK;   // elements per LDS stage

template <int MODE>
__global__ __launch_bounds__(256, 1) void ffn_gemm_bf16(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * STAGE];
  constexpr int CT = (MODE == MODE_GATEUP) ? BN / 2 : BN;   // output columns per tile
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

  // ---- global -> register loaders: thread owns k-chunk kc of rows r0 + 32 i
  const int kc = tid & 7;
  const int r0 = tid >> 3;
  const int swz = ((kc ^ (r0 & 7)) << 3);
  const uint16_t* ag[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = tl.m0 + r0 + 32 * i;
    if (m >= tl.M) m = tl.M - 1;
    int64_t arow;
    if (MODE == MODE_DOWN) {
      arow = tl.rb + m;
    } else if (routed) {
      arow = p.token_of_row[tl.rb + m];
      arow = arow < 0 ? 0 : (arow >= p.n_tokens ? p.n_tokens - 1 : arow);
    } else {
      arow = m;
    }
    ag[i] = A + arow * p.ldA + kc * 8;
  }
  const uint16_t* bg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = r0 + 32 * i;
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

  u32x4_t ra[4], rbv[8];
  auto gload = [&](int k0) {
    const bool ok = (k0 + kc * 8) < p.K;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ok ? *reinterpret_cast<const u32x4_t*>(ag[i] + k0) : z;
#pragma unroll
    for (int i = 0; i < 8; ++i) rbv[i] = ok ? *reinterpret_cast<const u32x4_t*>(bg[i] + k0) : z;
  };
  auto sstore = [&](int buf) {
    uint16_t* s = sm + buf * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(s + (r0 + 32 * i) * BK + swz) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t v = rbv[i];
      if (MODE == MODE_DOWN) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = bf16x2_to_f16x2(v[q]);
      }
      *reinterpret_cast<u32x4_t*>(s + BM * BK + (r0 + 32 * i) * BK + swz) = v;
    }
  };

  // ---- MFMA fragment addressing
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int l7 = lane & 7;
  int a_off[2], b_off[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_off[i] = (wm * 64 + 32 * i + lr) * BK;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int row;
    if (MODE == MODE_GATEUP) row = (j >> 1) * CT + wn * 64 + 32 * (j & 1) + lr;
    else row = wn * 128 + 32 * j + lr;
    b_off[j] = BM * BK + row * BK;
  }

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (p.K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint16_t* s = sm + cur * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int sw = ((kk * 2 + lh) ^ l7) << 3;
      u32x4_t af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(s + a_off[i] + sw);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const u32x4_t*>(s + b_off[j] + sw);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (MODE == MODE_DOWN)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8_t, af[i]), __builtin_bit_cast(f16x8_t, bf[j]), acc[i][j],
                0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bf[j]),
                acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  32x32 accumulator layout: element v of a lane is row
  // 8*(v/4) + 4*(lane/32) + v%4, column lane%32.
  uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lrow = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
      const int m = tl.m0 + lrow;
      if (m >= tl.M) continue;
      uint16_t* crow = C + (tl.rb + m) * p.ldC;
      if (MODE == MODE_GATEUP) {
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
          const int col = tl.n0 + wn * 64 + 32 * jn + lr;
          if (col < p.Ncols) {
            const float a = acc[i][jn][v];
            const float u = acc[i][jn + 2][v];
            float hv = a / (1.0f + __expf(-a)) * u;
            if (p.clip > 0.f) hv = fminf(fmaxf(hv, -p.clip), p.clip);
            crow[col] = f32_to_f16_sat(hv);
          }
        }
      } else {
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
          const int col = tl.n0 + wn * 128 + 32 * jn + lr;
          if (col < p.Ncols) {
            float vv = acc[i][jn][v];
            if (MODE == MODE_RELU_UP) vv = fmaxf(vv, 0.f);
            crow[col] = f32_to_f16_sat(vv);
          }
        }
      }
    }
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
      r = m;
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

template <int MODE>
hipError_t launch_gemm(const GemmParams& gp, int dtype, int64_t max_mtiles, hipStream_t s) {
  int CT;
  if (dtype == MOE_BF16) CT = (MODE == MODE_GATEUP) ? BN / 2 : BN;
  else CT = kF32BN;
  const int64_t ntn = (gp.Ncols + CT - 1) / CT;
  int64_t blocks = max_mtiles * ntn;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks <= 0) return hipSuccess;
  if (dtype == MOE_BF16) ffn_gemm_bf16<MODE><<<(unsigned)blocks, 256, 0, s>>>(gp);
  else ffn_gemm_f32<MODE><<<(unsigned)blocks, 256, 0, s>>>(gp);
  return hipGetLastError();
}

}  // namespace

int64_t ffn_max_mtiles(int64_t N, int k, int E, int S, int dtype) {
  const int bm = dtype == MOE_BF16 ? kGemmBM : kF32BM;
  int64_t t = 0;
  if (E > 0) t += (N * k + bm - 1) / bm + E;
  t += (int64_t)S * ((N + bm - 1) / bm);
  return t;
}

hipError_t launch_ffn(const FfnCall& c, hipStream_t s) {
  const int G = c.n_gather + c.n_ident;
  if (G <= 0 || c.N <= 0) return hipSuccess;
  const int bm = c.dtype == MOE_BF16 ? kGemmBM : kF32BM;
  const int64_t rows_cap = c.routed_rows;
  auto mark = [&](int i) {
    if (c.marks[i]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(c.marks[i]), s);
  };
  mark(0);
  ffn_plan_kernel<<<1, 1024, 0, s>>>(c.offsets, c.n_gather, c.n_ident, c.N, rows_cap,
                                     c.identity_row0, bm, c.plan);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
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
  up.clip = c.clip;
  up.C = c.h;
  mark(2);
  if (c.activation == MOE_SWIGLU) {
    up.Br0 = c.wg; up.Br1 = c.wu; up.Bs0 = c.sg; up.Bs1 = c.su;
    err = launch_gemm<MODE_GATEUP>(up, c.dtype, c.max_tiles_m, s);
  } else {
    up.Br0 = c.wu; up.Bs0 = c.su;
    err = launch_gemm<MODE_RELU_UP>(up, c.dtype, c.max_tiles_m, s);
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
  dn.Br0 = c.wd;
  dn.Bs0 = c.sd;
  dn.C = c.y_rows;
  mark(4);
  err = launch_gemm<MODE_DOWN>(dn, c.dtype, c.max_tiles_m, s);
  mark(5);
  return err;
}

}  // namespace moe
