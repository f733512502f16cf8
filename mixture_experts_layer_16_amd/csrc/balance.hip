// Load-balancing statistics of one routed batch and the aux-loss-free update
// of the per-expert selection biases.
//
// Statistics ("Основы MoE", "Вспомогательный лосс Switch Transformer"):
//   f_e = count_e / (N k)          share of the batch's assignments on expert e
//   P_e = mean_t p_te              mean router probability of expert e
//   aux = E * sum_e f_e P_e        1 for a uniform router, E on full collapse
// p_te is the softmax of the token's logits; for sigmoid gating (which has no
// softmax) it is the token's sigmoid scores divided by their sum.
//
// Update ("Le groupe d'experts (MoE)", "Le problème de l'équilibre de la
// charge", step 2; "Mixture-of-Experts" (DeepSeek-V4.1-Flash), "L'équilibrage
// de charge" and the per-modality section): an expert whose demand is above
// its target N_m k / E has its bias lowered by gamma, below raised by gamma,
// on target left alone; with two bias sets each set follows its own
// modality's demand.  The comparison is done exactly in integers
// (count * E against the set's total demand).
//
// Both reductions run in a fixed order (tokens -> per-block partial rows ->
// one block summing the rows in block order), so the results do not depend
// on scheduling.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BAL_THREADS = 256;
constexpr int FIN_THREADS = 1024;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}

// Block b sums p_te over tokens [b*chunk, min(N, (b+1)*chunk)); wave w of the
// block takes every fourth of those tokens, lane l expert l + 64 j.
template <int J>
__global__ __launch_bounds__(BAL_THREADS) void balance_probs_kernel(
    const double* __restrict__ z, int gating, int64_t N, int E, int64_t chunk,
    double* __restrict__ partial) {
  __shared__ double red[BAL_THREADS / 64][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int64_t t1 = t0 + chunk < N ? t0 + chunk : N;
  const bool sig = (gating == MOE_SIGMOID);

  double acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.0;

  for (int64_t t = t0 + wave; t < t1; t += BAL_THREADS / 64) {
    const double* zt = z + t * E;
    double v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? zt[e] : -INFINITY;
    }
    double s = 0.0;
    if (!sig) {
      double mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < J; ++j) mx = fmax(mx, v[j]);
      mx = wave_max(mx);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        v[j] = (lane + 64 * j < E) ? exp(v[j] - mx) : 0.0;
        s += v[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        v[j] = (lane + 64 * j < E) ? 1.0 / (1.0 + exp(-v[j])) : 0.0;
        s += v[j];
      }
    }
    s = wave_sum(s);
#pragma unroll
    for (int j = 0; j < J; ++j) acc[j] += v[j] / s;
  }

#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    if (e < E) red[wave][e] = acc[j];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += BAL_THREADS) {
    double r = red[0][e];
#pragma unroll
    for (int w = 1; w < BAL_THREADS / 64; ++w) r += red[w][e];
    partial[(int64_t)blockIdx.x * E + e] = r;
  }
}

// Fixed-order tree sum of sh[0..n) (n <= FIN_THREADS); the result is in sh[0].
template <typename T>
__device__ void block_tree_sum(T* sh, int n) {
  for (int w = FIN_THREADS / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w && (int)threadIdx.x + w < n) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
}

__global__ __launch_bounds__(FIN_THREADS) void balance_finish_kernel(
    const double* __restrict__ partial, int64_t nblk, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ mod_counts, double* __restrict__ load,
    double* __restrict__ mean_prob, double* __restrict__ aux, float* __restrict__ sel_bias,
    int n_bias_sets, float gamma, int64_t N, int E, int k) {
  __shared__ double shd[FIN_THREADS];
  __shared__ long long shi[FIN_THREADS];
  static_assert(kMaxExperts <= FIN_THREADS, "one thread per expert");
  const int e = threadIdx.x;
  const bool have = e < E;

  // P_e and f_e
  double P = 0.0, f = 0.0;
  if (have && N > 0) {
    if (partial) {
      for (int64_t b = 0; b < nblk; ++b) P += partial[b * E + e];
      P /= (double)N;
    }
    if (counts) f = (double)counts[e] / (double)(N * (int64_t)k);
  }
  if (have && load) load[e] = f;
  if (have && mean_prob) mean_prob[e] = P;
  if (aux) {
    shd[e] = have ? f * P : 0.0;
    __syncthreads();
    block_tree_sum(shd, E);
    if (e == 0) aux[0] = (double)E * shd[0];
  }

  // +-gamma update of each bias set from its own demand
  if (!sel_bias) return;
  for (int m = 0; m < n_bias_sets; ++m) {
    const int32_t* c = (n_bias_sets == 2) ? mod_counts + (int64_t)m * E : counts;
    __syncthreads();
    const long long cnt = have ? (long long)c[e] : 0;
    shi[e] = cnt;
    __syncthreads();
    block_tree_sum(shi, E);
    const long long total = shi[0];
    if (have) {
      const long long diff = cnt * (long long)E - total;
      const float sgn = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
      float* b = sel_bias + (int64_t)m * E + e;
      *b = *b - gamma * sgn;
    }
  }
}

}  // namespace

int64_t balance_blocks(int64_t N) {
  if (N <= 0) return 0;
  const int64_t nb = (N + kBalTokens - 1) / kBalTokens;
  return nb < kBalMaxBlocks ? nb : kBalMaxBlocks;
}

hipError_t launch_balance(const double* z, const int32_t* counts, const int32_t* mod_counts,
                          double* partial, double* load, double* mean_prob, double* aux,
                          float* sel_bias, int n_bias_sets, float gamma, int gating,
                          int64_t N, int E, int k, hipStream_t s) {
  const int64_t nblk = balance_blocks(N);
  const bool need_p = (mean_prob || aux) && nblk > 0;
  if (need_p) {
    const int64_t chunk = (N + nblk - 1) / nblk;
    const int J = (E + 63) / 64;
#define MOE_BAL(JJ) \
  balance_probs_kernel<JJ><<<(unsigned)nblk, BAL_THREADS, 0, s>>>(z, gating, N, E, chunk, partial)
    if (J <= 1) MOE_BAL(1);
    else if (J <= 2) MOE_BAL(2);
    else if (J <= 4) MOE_BAL(4);
    else if (J <= 6) MOE_BAL(6);
    else if (J <= 8) MOE_BAL(8);
    else MOE_BAL(16);
#undef MOE_BAL
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  balance_finish_kernel<<<1, FIN_THREADS, 0, s>>>(need_p ? partial : nullptr, nblk, counts,
                                                  mod_counts, load, mean_prob, aux, sel_bias,
                                                  n_bias_sets, gamma, N, E, k);
  return hipGetLastError();
}

}  // namespace moe
