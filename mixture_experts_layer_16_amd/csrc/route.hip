// Router projection, scoring, selection keys, top-k and gate weights.
//
// Steps 1-3 of "Основы MoE" (ai.flicky.cc), section "Как устроен MoE-слой":
// logits z = x W_g, scores softmax(z) (or the sigmoid of the DeepSeek-V3
// variant mentioned in the same section), the k largest, renormalised weights.
// Selection bias moves only the choice ("Le groupe d'experts (MoE)", section
// "Étape 1: le routeur"; V4.1 page, "L'équilibrage de charge"), one bias set per
// modality (V4.1 page, "La nouveauté de V4.1").
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// ---------------------------------------------------------------------------
// bf16 router logits on the matrix cores.
//
// Each v_mfma_f32_16x16x32_bf16 sums 32 exact bf16 x bf16 products into a
// fresh fp32 partial; the partial is then added into a float64 accumulator.
// The fp32 rounding error is therefore confined to 32-term partial sums and the
// logits come out within ~1e-7 of their scale of the exact dot product, which
// keeps the top-k decision equal to the float64 one except for near-ties.
//
// Block: 4 waves; tile 128 tokens x 64 experts; wave w owns 32 tokens (two
// 16-row fragments, read straight from global memory) and the block's 64
// experts, whose 64 x 128 k-chunk is staged in LDS (double buffered) for all
// four waves.  The loads of chunk c+1 (both operands) are in flight while
// chunk c is multiplied, so each wave keeps 12 16-byte loads per lane
// outstanding instead of waiting on every 32-wide step.  The reduction
// dimension may be split over gridDim.z blocks (small batches); each split
// writes float64 partials [split][N][E] and the top-k kernel adds them in
// split order.  The float64 accumulators see the 32-product partials in k
// order whatever the chunking, so the logits do not depend on it.
constexpr int RT_TOK = 128;
constexpr int RT_EXP = 64;

// RT_STEPS: 32-wide k steps per staged chunk; MINB: blocks per CU the register
// budget allows (two-step chunks need the registers of two blocks per CU)
template <int RT_STEPS, int MINB>
__global__ __launch_bounds__(256, MINB) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, double* __restrict__ zpart,
    int64_t N, int d, int E, int ksplit_len) {
  __shared__ __attribute__((aligned(16))) uint16_t bs[2][RT_STEPS][RT_EXP * 32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tok0 = (int64_t)blockIdx.x * RT_TOK + wave * 32;
  const int e0 = blockIdx.y * RT_EXP;
  const int k_lo = blockIdx.z * ksplit_len;
  const int k_hi = min(d, k_lo + ksplit_len);
  const int r16 = lane & 15;     // A row / B column supplied by this lane
  const int kq = lane >> 4;      // which 8-wide k chunk of the 32-wide step

  const uint16_t* ap[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int64_t arow = tok0 + 16 * i + r16;
    if (arow >= N) arow = N - 1;
    ap[i] = x + arow * (int64_t)d + kq * 8;
  }
  // B staging: thread -> (expert row tid / 4, chunk tid % 4) of each step; position
  // of chunk c of row e in LDS: c ^ ((e >> 2) & 3), conflict-free for the
  // 16-row reads
  const int se = tid >> 2, sc = tid & 3;
  int ge = e0 + se;
  if (ge >= E) ge = E - 1;
  const uint16_t* bsrc = w + (int64_t)ge * d + sc * 8;
  const int sdst = se * 32 + ((sc ^ ((se >> 2) & 3)) << 3);
  int boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 16 * j + r16;
    boff[j] = e * 32 + ((kq ^ ((e >> 2) & 3)) << 3);
  }

  double acc[2][4][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  constexpr int CHK = 32 * RT_STEPS;
  const int nchunks = (k_hi - k_lo + CHK - 1) / CHK;
  // operands of one chunk; 16-byte pieces past k_hi are zero
  auto load = [&](int c, u32x4_t (&a)[RT_STEPS][2], u32x4_t (&b)[RT_STEPS]) {
#pragma unroll
    for (int s = 0; s < RT_STEPS; ++s) {
      const int k0 = k_lo + c * CHK + 32 * s;
      b[s] = (k0 + sc * 8 < k_hi) ? *reinterpret_cast<const u32x4_t*>(bsrc + k0) : zero;
      const bool ok = k0 + kq * 8 < k_hi;
#pragma unroll
      for (int i = 0; i < 2; ++i) a[s][i] = ok ? *reinterpret_cast<const u32x4_t*>(ap[i] + k0) : zero;
    }
  };
  auto stage = [&](int buf, const u32x4_t (&b)[RT_STEPS]) {
#pragma unroll
    for (int s = 0; s < RT_STEPS; ++s) *reinterpret_cast<u32x4_t*>(&bs[buf][s][sdst]) = b[s];
  };
  auto multiply = [&](int buf, const u32x4_t (&a)[RT_STEPS][2]) {
#pragma unroll
    for (int s = 0; s < RT_STEPS; ++s) {
      u32x4_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u32x4_t*>(&bs[buf][s][boff[j]]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t pp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a[s][i]), __builtin_bit_cast(bf16x8_t, b[j]), zero4,
              0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] += (double)pp[v];
        }
    }
  };

  // chunks alternate between two register sets and two LDS buffers
  u32x4_t a0[RT_STEPS][2], b0[RT_STEPS], a1[RT_STEPS][2], b1[RT_STEPS];
  if (nchunks > 0) {
    load(0, a0, b0);
    stage(0, b0);
  }
  if (nchunks > 1) load(1, a1, b1);
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    multiply(0, a0);
    if (c + 1 < nchunks) stage(1, b1);
    if (c + 2 < nchunks) load(c + 2, a0, b0);
    __syncthreads();
    if (c + 1 >= nchunks) break;
    multiply(1, a1);
    if (c + 2 < nchunks) stage(0, b0);
    if (c + 3 < nchunks) load(c + 3, a1, b1);
    __syncthreads();
  }

  // D layout of the 16x16 output: lane holds column (lane & 15), rows 4*(lane>>4)+v
  double* zp = zpart + (int64_t)blockIdx.z * N * E;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 16 * j + r16;
    if (e >= E) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t t = tok0 + 16 * i + 4 * kq + v;
        if (t < N) zp[t * E + e] = acc[i][j][v];
      }
  }
}

// fp32 inputs: products of two floats are exact in float64, so the float64
// FMA chain gives the logits to float64 accuracy.
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, double* __restrict__ z, int64_t N,
    int d, int E) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * E) return;
  const int64_t t = i / E;
  const int e = (int)(i - t * E);
  const float* xr = x + t * d;
  const float* wr = w + (int64_t)e * d;
  double s = 0.0;
  for (int c = 0; c < d; ++c) s = fma((double)xr[c], (double)wr[c], s);
  z[i] = s;
}

// ---------------------------------------------------------------------------
// top-k: one token per wavefront.  Lane l owns experts l, l+64, l+128, ...
// Each of the k rounds is a 64-lane argmax on (key desc, index asc) by xor
// butterflies; lane r keeps the r-th winner.  Keys and scores are float64.
__device__ __forceinline__ bool better(double ka, int ea, double kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}

// J = key slots per lane (E <= 64 * J), a compile-time constant so the keys
// stay in registers.
// The logits arrive as `nsplit` float64 partial sums [split][N][E]; they are
// added in split order, plus the logit offset, and optionally written out.
template <int J>
__global__ __launch_bounds__(256) void topk_kernel(
    const double* zpart, int nsplit, const float* __restrict__ logit_bias,
    double* z_out, const float* __restrict__ sel_bias,
    const uint8_t* __restrict__ modality, int n_bias_sets, int gating, int renormalize,
    int32_t* __restrict__ out_idx, float* __restrict__ out_w, int32_t* __restrict__ out_alt,
    int64_t N, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;
  const int m = (n_bias_sets == 2) ? (int)modality[t] : 0;
  const float* bias = n_bias_sets ? sel_bias + (int64_t)m * E : nullptr;
  const bool sig = (gating == MOE_SIGMOID);

  double key[J], sc[J];
  uint32_t valid = 0;
  // the logits: split-K partials added in split order.  The partials of all J
  // key slots are loaded QB splits at a time (J * QB independent loads in
  // flight), so a batch of tokens split many ways waits for one memory round
  // trip per QB splits rather than per slot and QB splits
  constexpr int QB = J <= 4 ? 4 : (J <= 8 ? 2 : 1);
  double zsum[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    zsum[j] = e < E ? zpart[t * E + e] : 0.0;
  }
  for (int q = 1; q < nsplit; q += QB) {
    double pq[J][QB];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
#pragma unroll
      for (int i = 0; i < QB; ++i)
        pq[j][i] = (e < E && q + i < nsplit) ? zpart[((int64_t)(q + i) * N + t) * E + e] : 0.0;
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int i = 0; i < QB; ++i)
        if (q + i < nsplit) zsum[j] += pq[j][i];
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    key[j] = -INFINITY;
    sc[j] = 0.0;
    if (e < E) {
      double zz = zsum[j];
      if (logit_bias) zz += (double)logit_bias[e];
      if (z_out) z_out[t * E + e] = zz;
      const double s = sig ? 1.0 / (1.0 + exp(-zz)) : zz;   // sigmoid score, or the logit
      double kk = s;
      if (bias) kk += (double)bias[e];
      key[j] = kk;
      sc[j] = s;
      valid |= 1u << j;
    }
  }

  int my_e = 0;          // lane r < k: expert of round r
  double my_s = 0.0;     // its logit (softmax) or sigmoid score
  int my_alt = -1;       // lane q < k: expert of round k + q (the alternates)
  const int ka = out_alt ? min(k, E - k) : 0;
  for (int r = 0; r < k + ka; ++r) {
    double bk = -INFINITY, bs = 0.0;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (valid & (1u << j)) {
        const int e = lane + 64 * j;
        if (better(key[j], e, bk, be)) { bk = key[j]; be = e; bs = sc[j]; }
      }
    }
    const double own_s = bs;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ok = __shfl_xor(bk, off);
      const int oe = __shfl_xor(be, off);
      if (better(ok, oe, bk, be)) { bk = ok; be = oe; }
    }
    const int owner = be & 63;
    const double ws = __shfl(own_s, owner);
    if (lane == owner) valid &= ~(1u << (be >> 6));
    if (r < k) {
      if (lane == r) { my_e = be; my_s = ws; }
    } else if (lane == r - k) {
      my_alt = be;
    }
  }
  if (out_alt && lane < k) out_alt[t * k + lane] = my_alt;

  // gate weights.  Renormalised: softmax over the chosen logits (equal to the
  // renormalised full softmax), or sigmoid scores divided by their sum.  Raw:
  // the full softmax probability of the chosen expert, or its sigmoid score.
  const bool mine = lane < k;
  double g, sum;
  if (!sig) {
    double mx;
    if (renormalize) {
      mx = mine ? my_s : -INFINITY;
    } else {
      mx = -INFINITY;                       // max over every expert's logit
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (lane + 64 * j < E) mx = fmax(mx, sc[j]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
    g = mine ? exp(my_s - mx) : 0.0;
    if (renormalize) {
      sum = g;
    } else {
      sum = 0.0;
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (lane + 64 * j < E) sum += exp(sc[j] - mx);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  } else {
    g = mine ? my_s : 0.0;
    sum = 1.0;
    if (renormalize) {
      sum = g;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    }
  }
  if (mine) {
    out_idx[t * k + lane] = my_e;
    out_w[t * k + lane] = (float)(g / sum);
  }
}

// Parameter-free router: h = splitmix64(id) (S. Vigna's 64-bit mixer); the
// token's experts are h mod E, h mod E + 1, ... (mod E), weights 1/k.
__global__ __launch_bounds__(256) void hash_route_kernel(const int64_t* __restrict__ ids,
                                                         int64_t N, int E, int k,
                                                         int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_w) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N) return;
  uint64_t z = (uint64_t)ids[t] + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  const int base = (int)(z % (uint64_t)E);
  const float w = 1.0f / (float)k;
  for (int j = 0; j < k; ++j) {
    const int e = base + j;
    out_idx[t * k + j] = e >= E ? e - E : e;
    out_w[t * k + j] = w;
  }
}

}  // namespace

hipError_t launch_hash_route(const int64_t* ids, int64_t N, int E, int k, int32_t* idx,
                             float* w, hipStream_t s) {
  hash_route_kernel<<<(unsigned)((N + 255) / 256), 256, 0, s>>>(ids, N, E, k, idx, w);
  return hipGetLastError();
}

int router_splits(int64_t N, int d, int E) {
  const int64_t base = ((N + RT_TOK - 1) / RT_TOK) * ((E + RT_EXP - 1) / RT_EXP);
  int64_t ks = 512 / (base > 0 ? base : 1);
  const int64_t kmax = d / 256 > 1 ? d / 256 : 1;
  if (ks > kmax) ks = kmax;
  if (ks > kMaxRouterSplits) ks = kMaxRouterSplits;
  return ks < 1 ? 1 : (int)ks;
}

hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* w, double* zpart, int nsplit,
                              int64_t N, int d, int E, hipStream_t s) {
  // split length: a multiple of 32 covering d in nsplit pieces
  int len = (d + nsplit - 1) / nsplit;
  len = (len + 31) / 32 * 32;
  const int ns = (d + len - 1) / len;
  dim3 grid((unsigned)((N + RT_TOK - 1) / RT_TOK), (unsigned)((E + RT_EXP - 1) / RT_EXP),
            (unsigned)ns);
  // two-step chunks (more loads in flight per wave) while two blocks per CU
  // hold the whole grid; otherwise one-step chunks at three blocks per CU, so
  // a large grid still runs in one round
  const int64_t blocks = (int64_t)grid.x * grid.y * grid.z;
  if (blocks <= 2 * kCus)
    router_bf16_kernel<2, 2><<<grid, 256, 0, s>>>(x, w, zpart, N, d, E, len);
  else
    router_bf16_kernel<1, 3><<<grid, 256, 0, s>>>(x, w, zpart, N, d, E, len);
  return hipGetLastError();
}

int router_splits_used(int d, int nsplit) {
  int len = (d + nsplit - 1) / nsplit;
  len = (len + 31) / 32 * 32;
  return (d + len - 1) / len;
}

hipError_t launch_router_f32(const float* x, const float* w, double* z, int64_t N, int d, int E,
                             hipStream_t s) {
  const int64_t n = N * E;
  router_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, w, z, N, d, E);
  return hipGetLastError();
}

hipError_t launch_topk(const double* zpart, int nsplit, const float* logit_bias, double* z_out,
                       const float* sel_bias, const uint8_t* modality, int n_bias_sets,
                       int gating, int renormalize, int32_t* idx, float* w, int32_t* alt,
                       int64_t N, int E, int k, hipStream_t s) {
  const unsigned grid = (unsigned)((N + 3) / 4);
  const int J = (E + 63) / 64;
#define MOE_TOPK(JJ)                                                                        \
  topk_kernel<JJ><<<grid, 256, 0, s>>>(zpart, nsplit, logit_bias, z_out, sel_bias, modality, \
                                       n_bias_sets, gating, renormalize, idx, w, alt, N, E, k)
  if (J <= 1) MOE_TOPK(1);
  else if (J <= 2) MOE_TOPK(2);
  else if (J <= 4) MOE_TOPK(4);
  else if (J <= 6) MOE_TOPK(6);
  else if (J <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
