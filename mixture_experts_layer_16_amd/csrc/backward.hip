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

constexpr int GB_M = 128, GB_N = 128, GB_K = 32;   // tile and k-slice
constexpr int GB_STAGE = (GB_M + GB_N) * GB_K;     // elements per LDS stage

// LDS row layout: rows of 32 k-values (64 bytes), two per 128-byte line; the
// 16-byte chunk at position q of line l sits at q ^ swz(l) (conflict-free for
// the 32-row fragment reads, as in the forward kernels)
__device__ __forceinline__ int bw_swz(int line) { return ((line >> 1) & 3) ^ ((line & 1) << 1); }
__device__ __forceinline__ int bw_off(int row, int chunk) {   // element offset of (row, chunk*8)
  const int line = row >> 1;
  return line * 64 + ((((row & 1) << 2) + chunk) ^ bw_swz(line)) * 8;
}

// One operand of C[m][n] = sum_k A(m,k) B(n,k).
//   T == 0: element (i, k) at p[row(i) * ld + k]            (k contiguous)
//   T == 1: element (i, k) at p[row(k) * ld + i]            (i contiguous)
// row() applies the optional row map (a gather), else the identity plus a
// base row.  Rows past the tile's extent are clamped; k past the slice's K
// reads zero.
struct Operand {
  const uint16_t* p;    // routed groups (group g at p + g * gstride), or the only matrix
  const uint16_t* ps;   // dense (shared-expert) groups: group g at ps + (g - n_gather) * gstride
  int64_t gstride;      // 0: the same matrix for every group
  int64_t ld;
  int tokens;           // rows are layout rows to turn into token rows: through map for
                        // routed groups, minus the dense group's first row otherwise
  const int32_t* map;   // token_of_row
};

struct BwdGemmParams {
  Operand A, B, A2, B2;      // A2/B2: optional second product into the same C
  int two;                   // use A2/B2
  float* C;                  // row mode: [rows][ldc]; weight mode: routed groups' matrices
  float* Cs;                 // weight mode: dense groups' matrices
  int64_t ldc, c_gstride;
  int M, N, K, K2;           // fixed extents (row mode: M from the plan; weight mode: K)
  int mode;                  // 0: tiles over the plan's rows; 1: K = a group's rows
  const int32_t* plan;       // tile_start[G+1], row_begin[G], rows[G]
  int G;
  int n_gather;              // groups below this are routed experts
  int64_t ident_row0, n_tokens;
};

template <int TA, int TB>
__global__ __launch_bounds__(256, 2) void bwd_gemm_kernel(BwdGemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * GB_STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- tile decode
  int g, m0, n0, Mlim, Klim;
  int64_t rb;
  const int ntn = (p.N + GB_N - 1) / GB_N;
  if (p.mode == 0) {
    const int32_t* tile_start = p.plan;
    const int total = tile_start[p.G] * ntn;
    const int L = blockIdx.x;
    if (L >= total) return;
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] * ntn <= L) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int local = L - tile_start[g] * ntn;
    m0 = (local / ntn) * GB_M;
    n0 = (local % ntn) * GB_N;
    rb = p.plan[p.G + 1 + g];
    Mlim = p.plan[p.G + 1 + p.G + g];
    Klim = p.K;
  } else {
    const int ntm = (p.M + GB_M - 1) / GB_M;
    const int per = ntm * ntn;
    g = blockIdx.x / per;
    if (g >= p.G) return;
    const int local = blockIdx.x - g * per;
    m0 = (local / ntn) * GB_M;
    n0 = (local % ntn) * GB_N;
    rb = p.plan[p.G + 1 + g];
    Klim = p.plan[p.G + 1 + p.G + g];
    if (Klim <= 0) {
      // no rows: the gradient of this group's weights is zero
      float* Cg = g < p.n_gather ? p.C + g * p.c_gstride
                                 : p.Cs + (int64_t)(g - p.n_gather) * p.c_gstride;
      for (int i = tid; i < GB_M * GB_N; i += 256) {
        const int m = m0 + i / GB_N, n = n0 + i % GB_N;
        if (m < p.M && n < p.N) Cg[(int64_t)m * p.ldc + n] = 0.f;
      }
      return;
    }
    Mlim = p.M;
  }

  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // group-dependent operand bases: routed weight groups move by the group
  // stride; in row mode, operands indexed by rows use the plan's row begin
  const bool routed = g < p.n_gather;
  const int64_t dense_row0 = p.ident_row0 + (int64_t)(g - p.n_gather) * p.n_tokens;
  auto run = [&](const Operand& OA, const Operand& OB, int K) {
    // per-thread load plans
    //  T == 0: thread -> rows (tid/4) + 64*i, chunk tid%4: two 16-byte loads
    //  T == 1: thread -> k pair 2*(tid/16), rows 8*(tid%16) .. +7: two loads
    auto row_ptr = [&](const Operand& O, int64_t rr) -> const uint16_t* {
      if (O.tokens) {
        if (routed) {
          rr = O.map[rr];
          rr = rr < 0 ? 0 : (rr >= p.n_tokens ? p.n_tokens - 1 : rr);
        } else {
          rr -= dense_row0;
        }
      }
      const uint16_t* base =
          routed ? O.p + g * O.gstride : O.ps + (int64_t)(g - p.n_gather) * O.gstride;
      return base + rr * O.ld;
    };
    // extents: A's rows are m (limit Mlim), B's rows are n (limit N); in
    // weight mode the k rows are the group's rows (limit Klim)
    u32x4_t ra[2], rbv[2];
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    auto load = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (TA == 0) {
          int m = m0 + (tid >> 2) + 64 * i;
          if (m >= Mlim) m = Mlim - 1;
          const int kk = k0 + (tid & 3) * 8;
          const uint16_t* q = row_ptr(OA, p.mode == 0 ? rb + m : (int64_t)m);
          ra[i] = kk < K ? *reinterpret_cast<const u32x4_t*>(q + kk) : zero;
        } else {
          // 8 consecutive rows; the operand's rows are padded to a multiple of 8
          const int kk = k0 + 2 * (tid >> 4) + i;
          int m = m0 + 8 * (tid & 15);
          if (m >= Mlim) m = ((Mlim + 7) & ~7) - 8;
          if (kk < K) {
            const uint16_t* q = row_ptr(OA, p.mode == 1 ? rb + kk : (int64_t)kk);
            ra[i] = *reinterpret_cast<const u32x4_t*>(q + m);
          } else {
            ra[i] = zero;
          }
        }
        if (TB == 0) {
          int n = n0 + (tid >> 2) + 64 * i;
          if (n >= p.N) n = p.N - 1;
          const int kk = k0 + (tid & 3) * 8;
          const uint16_t* q = row_ptr(OB, n);
          rbv[i] = kk < K ? *reinterpret_cast<const u32x4_t*>(q + kk) : zero;
        } else {
          const int kk = k0 + 2 * (tid >> 4) + i;
          int n = n0 + 8 * (tid & 15);
          if (n >= p.N) n = ((p.N + 7) & ~7) - 8;
          if (kk < K) {
            const uint16_t* q = row_ptr(OB, p.mode == 1 ? rb + kk : (int64_t)kk);
            rbv[i] = *reinterpret_cast<const u32x4_t*>(q + n);
          } else {
            rbv[i] = zero;
          }
        }
      }
    };
    auto store = [&](uint16_t* s) {
      uint16_t* sa = s;
      uint16_t* sb = s + GB_M * GB_K;
      if (TA == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          *reinterpret_cast<u32x4_t*>(sa + bw_off((tid >> 2) + 64 * i, tid & 3)) = ra[i];
      } else {
        // rows 8*(tid%16)+c get the k pair 2*(tid/16), 2*(tid/16)+1
        const int kp = 2 * (tid >> 4);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t lo = (ra[0][c >> 1] >> (16 * (c & 1))) & 0xffffu;
          const uint32_t hi = (ra[1][c >> 1] >> (16 * (c & 1))) & 0xffffu;
          const int row = 8 * (tid & 15) + c;
          *reinterpret_cast<uint32_t*>(sa + bw_off(row, kp >> 3) + (kp & 7)) = lo | (hi << 16);
        }
      }
      if (TB == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          *reinterpret_cast<u32x4_t*>(sb + bw_off((tid >> 2) + 64 * i, tid & 3)) = rbv[i];
      } else {
        const int kp = 2 * (tid >> 4);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t lo = (rbv[0][c >> 1] >> (16 * (c & 1))) & 0xffffu;
          const uint32_t hi = (rbv[1][c >> 1] >> (16 * (c & 1))) & 0xffffu;
          const int row = 8 * (tid & 15) + c;
          *reinterpret_cast<uint32_t*>(sb + bw_off(row, kp >> 3) + (kp & 7)) = lo | (hi << 16);
        }
      }
    };
    auto compute = [&](const uint16_t* s) {
      const uint16_t* sa = s;
      const uint16_t* sb = s + GB_M * GB_K;
#pragma unroll
      for (int kk = 0; kk < GB_K / 16; ++kk) {
        u32x4_t af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const u32x4_t*>(sa + bw_off(wm * 64 + 32 * i + lr, 2 * kk + lh));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bf[j] = *reinterpret_cast<const u32x4_t*>(sb + bw_off(wn * 64 + 32 * j + lr, 2 * kk + lh));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bf[j]),
                acc[i][j], 0, 0, 0);
      }
    };
    const int nsl = (K + GB_K - 1) / GB_K;
    if (nsl <= 0) return;
    load(0);
    store(sm);
    __syncthreads();
    for (int kt = 0; kt < nsl; ++kt) {
      uint16_t* cur = sm + (kt & 1) * GB_STAGE;
      uint16_t* nxt = sm + ((kt + 1) & 1) * GB_STAGE;
      if (kt + 1 < nsl) load((kt + 1) * GB_K);
      compute(cur);
      if (kt + 1 < nsl) store(nxt);
      __syncthreads();
    }
  };
  run(p.A, p.B, p.mode == 1 ? Klim : p.K);
  if (p.two) run(p.A2, p.B2, p.mode == 1 ? Klim : p.K2);

  // ---- store: element v of lane: row 8*(v/4) + 4*lh + v%4, column lr
  float* C = p.C;
  if (p.mode == 1)
    C = routed ? p.C + g * p.c_gstride : p.Cs + (int64_t)(g - p.n_gather) * p.c_gstride;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
      if (m >= Mlim) continue;
      const int64_t crow = (p.mode == 0 ? rb + m : (int64_t)m) * p.ldc;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + 32 * j + lr;
        if (n < p.N) C[crow + n] = acc[i][j][v];
      }
    }
}

template <int TA, int TB>
hipError_t launch_bwd_gemm(const BwdGemmParams& p, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  bwd_gemm_kernel<TA, TB><<<(unsigned)blocks, 256, 0, s>>>(p);
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
__global__ __launch_bounds__(256) void bwd_rows_kernel(
    const float* __restrict__ af, const float* __restrict__ uf, const float* __restrict__ dhu,
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
    const float4 u4 = *reinterpret_cast<const float4*>(uf + o + i);
    const float4 d4 = *reinterpret_cast<const float4*>(dhu + o + i);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (swiglu) {
      const float4 a4 = *reinterpret_cast<const float4*>(af + o + i);
      a[0] = a4.x; a[1] = a4.y; a[2] = a4.z; a[3] = a4.w;
    }
    const float u[4] = {u4.x, u4.y, u4.z, u4.w};
    const float dh_u[4] = {d4.x, d4.y, d4.z, d4.w};
    uint16_t ohg[4], oda[4], odu[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float h, dh, dA = 0.f, dU;
      if (swiglu) {
        const float sg = 1.f / (1.f + expf(-a[q]));
        const float act = a[q] * sg;
        const float hpre = act * u[q];
        const bool pass = !(clip > 0.f) || fabsf(hpre) <= clip;
        h = clip > 0.f ? fminf(fmaxf(hpre, -clip), clip) : hpre;
        dh = pass ? g * dh_u[q] : 0.f;
        dU = dh * act;
        dA = dh * u[q] * (sg * (1.f + a[q] * (1.f - sg)));
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

inline unsigned blocks_of(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }
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

  // tile plans: experts + shared experts over the forward's row layout, and
  // one dense group of N rows for the router products
  MOE_CHK(launch_ffn_plan(c.offsets, E, S, N, nk, nk, GB_M, plan, s));
  MOE_CHK(launch_ffn_plan(nullptr, 0, 1, N, 0, 0, GB_M, plan_r, s));
  to_bf16_kernel<<<blocks_of(N * d / 4, 256), 256, 0, s>>>(c.dy, dy16, N * d / 4);
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
  const int64_t row_tiles = (nk + GB_M - 1) / GB_M + E + S * ((N + GB_M - 1) / GB_M);
  auto tn = [](int n) { return (int64_t)((n + GB_N - 1) / GB_N); };
  const Operand xin{x, x, 0, d, 1, c.token_of_row};
  const Operand dyin{dy16, dy16, 0, d, 1, c.token_of_row};

  // recompute a = x W_gate^T and u = x W_up^T per row
  q.mode = 0;
  q.K = d;
  q.N = I;
  q.ldc = I;
  q.A = xin;
  if (swiglu) {
    q.B = Operand{W(c.wg), W(c.sg), (int64_t)I * d, d, 0, nullptr};
    q.C = af;
    MOE_CHK((launch_bwd_gemm<0, 0>(q, row_tiles * tn(I), s)));
  }
  q.B = Operand{W(c.wu), W(c.su), (int64_t)I * d, d, 0, nullptr};
  q.C = uf;
  MOE_CHK((launch_bwd_gemm<0, 0>(q, row_tiles * tn(I), s)));
  // du_h = dy W_down (W_down [d][I] read with the reduction index slow)
  q.A = dyin;
  q.B = Operand{W(c.wd), W(c.sd), (int64_t)d * I, I, 0, nullptr};
  q.C = dhu;
  MOE_CHK((launch_bwd_gemm<0, 1>(q, row_tiles * tn(I), s)));

  bwd_rows_kernel<<<(unsigned)R, 256, 0, s>>>(af, uf, dhu, slot, c.topk_w, c.offsets, E, nk, I,
                                              swiglu ? 1 : 0, c.clip, hg, da, du, dgr);
  MOE_CHK(hipGetLastError());

  // weight gradients, one group per expert: K = the group's rows
  q.mode = 1;
  const Operand hgin{hg, hg, 0, I, 0, nullptr};
  const Operand dain{da, da, 0, I, 0, nullptr};
  const Operand duin{du, du, 0, I, 0, nullptr};
  auto wblocks = [&](int M, int Nn) {
    return (int64_t)G * ((M + GB_M - 1) / GB_M) * tn(Nn);
  };
  // dW_down[e] = sum_r (g dy_t)^T h_r   ([d][I])
  q.M = d; q.N = I; q.ldc = I; q.c_gstride = (int64_t)d * I;
  q.A = dyin; q.B = hgin; q.C = c.dw_down; q.Cs = c.dws_down;
  MOE_CHK((launch_bwd_gemm<1, 1>(q, wblocks(d, I), s)));
  // dW_gate[e] = sum_r da_r^T x_t, dW_up[e] = sum_r du_r^T x_t   ([I][d])
  q.M = I; q.N = d; q.ldc = d; q.c_gstride = (int64_t)I * d;
  q.B = xin;
  if (swiglu) {
    q.A = dain; q.C = c.dw_gate; q.Cs = c.dws_gate;
    MOE_CHK((launch_bwd_gemm<1, 1>(q, wblocks(I, d), s)));
  }
  q.A = duin; q.C = c.dw_up; q.Cs = c.dws_up;
  MOE_CHK((launch_bwd_gemm<1, 1>(q, wblocks(I, d), s)));

  // per-row input gradient dx_r = da W_gate + du W_up ([R][d])
  q.mode = 0;
  q.N = d; q.ldc = d; q.K = I; q.K2 = I;
  q.C = dxp; q.Cs = nullptr;
  if (swiglu) {
    q.A = dain;
    q.B = Operand{W(c.wg), W(c.sg), (int64_t)I * d, d, 0, nullptr};
    q.A2 = duin;
    q.B2 = Operand{W(c.wu), W(c.su), (int64_t)I * d, d, 0, nullptr};
    q.two = 1;
  } else {
    q.A = duin;
    q.B = Operand{W(c.wu), W(c.su), (int64_t)I * d, d, 0, nullptr};
    q.two = 0;
  }
  MOE_CHK((launch_bwd_gemm<0, 1>(q, row_tiles * tn(d), s)));
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
  qr.A = Operand{dz16, dz16, 0, Ep, 0, nullptr};
  qr.B = Operand{W(c.wr), W(c.wr), 0, d, 0, nullptr};
  qr.C = c.dx;
  MOE_CHK((launch_bwd_gemm<0, 1>(qr, ((N + GB_M - 1) / GB_M) * tn(d), s)));
  // dW_router = dz^T x ([E][d])
  qr.mode = 1;
  qr.M = E;
  qr.N = d;
  qr.ldc = d;
  qr.c_gstride = 0;
  qr.B = Operand{x, x, 0, d, 0, nullptr};
  qr.C = c.dw_router;
  qr.Cs = c.dw_router;
  MOE_CHK((launch_bwd_gemm<1, 1>(qr, (int64_t)((E + GB_M - 1) / GB_M) * tn(d), s)));
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
#undef MOE_CHK
  return hipSuccess;
}

}  // namespace moe
