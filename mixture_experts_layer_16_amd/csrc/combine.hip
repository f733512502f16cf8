// Gate-weighted combine and un-permute back to token order:
//   y_t = sum_{j kept} g_tj * y_rows[row_of[t,j]] + sum_s shared_s(x_t)
// ("Основы MoE", section "Как устроен MoE-слой", step 4; the shared expert is
// added with weight 1 outside the renormalisation and a dropped assignment adds
// nothing, without renormalising the others: "Mixture-of-Experts : routage et
// capacité", "L'idée — Top-k et mélange" and "Cas guidé — trace complète").
//
// One block per token; 128-bit loads and stores; the expert rows are read once,
// with non-temporal loads, while y is stored normally (the caller reads it
// next); float32 sums in a fixed order (j = 0..k-1, then shared experts); the
// output is float32.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// Rows in fp16 (the expert output format of the bf16 path), output fp32.
__global__ __launch_bounds__(256) void combine_f16_kernel(
    const uint16_t* __restrict__ y_rows, const int32_t* __restrict__ row_of,
    const float* __restrict__ topk_w, const uint16_t* __restrict__ y_shared,
    int64_t sh_stride_rows, int S, float* __restrict__ y, int64_t N, int d, int k) {
  __shared__ int32_t rows[kMaxTopK];
  __shared__ float gw[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of[t * k + threadIdx.x];
    gw[threadIdx.x] = topk_w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int nch = d >> 3;
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // the rows of up to 8 slots are loaded together, then added in slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4_t v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int r = j < k ? rows[j] : -1;
        v[jj] = r >= 0 ? __builtin_nontemporal_load(
                             reinterpret_cast<const u32x4_t*>(y_rows + (int64_t)r * d + c * 8))
                       : (u32x4_t){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        if (j >= k || rows[j] < 0) continue;
        const float g = gw[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(g, f16_to_f32((uint16_t)(v[jj][q] & 0xffffu)), acc[2 * q]);
          acc[2 * q + 1] = fmaf(g, f16_to_f32((uint16_t)(v[jj][q] >> 16)), acc[2 * q + 1]);
        }
      }
    }
    for (int s = 0; s < S; ++s) {
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
          y_shared + ((int64_t)s * sh_stride_rows + t) * d + c * 8));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += f16_to_f32((uint16_t)(v[q] & 0xffffu));
        acc[2 * q + 1] += f16_to_f32((uint16_t)(v[q] >> 16));
      }
    }
    f32x4_t* out = reinterpret_cast<f32x4_t*>(y + t * d + c * 8);
    out[0] = (f32x4_t){acc[0], acc[1], acc[2], acc[3]};
    out[1] = (f32x4_t){acc[4], acc[5], acc[6], acc[7]};
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(
    const float* __restrict__ y_rows, const int32_t* __restrict__ row_of,
    const float* __restrict__ topk_w, const float* __restrict__ y_shared,
    int64_t sh_stride_rows, int S, float* __restrict__ y, int64_t N, int d, int k) {
  __shared__ int32_t rows[kMaxTopK];
  __shared__ float gw[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of[t * k + threadIdx.x];
    gw[threadIdx.x] = topk_w[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r >= 0) acc = fmaf(gw[j], y_rows[(int64_t)r * d + c], acc);
    }
    for (int s = 0; s < S; ++s) acc += y_shared[((int64_t)s * sh_stride_rows + t) * d + c];
    y[t * d + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const void* y_rows, const int32_t* row_of,
                          const float* topk_w, const void* y_shared, int64_t shared_stride_rows,
                          int S, void* y, int64_t N, int d, int k, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (!y_shared) S = 0;
  if (dtype == MOE_BF16)
    combine_f16_kernel<<<(unsigned)N, 256, 0, s>>>(
        static_cast<const uint16_t*>(y_rows), row_of, topk_w,
        static_cast<const uint16_t*>(y_shared), shared_stride_rows, S,
        static_cast<float*>(y), N, d, k);
  else
    combine_f32_kernel<<<(unsigned)N, 256, 0, s>>>(
        static_cast<const float*>(y_rows), row_of, topk_w, static_cast<const float*>(y_shared),
        shared_stride_rows, S, static_cast<float*>(y), N, d, k);
  return hipGetLastError();
}

}  // namespace moe
