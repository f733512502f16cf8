// Internal declarations shared by the HIP sources of the MoE-layer library.
// Nothing here is part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// tiling constants shared by the host planner and the kernels

constexpr int kF32BM = 64;         // fp32 path tile
constexpr int kF32BN = 64;
constexpr int kPermTokens = 256;   // tokens per block of the rank kernel
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxShared = 8;
constexpr int kXcds = 8;              // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kCus = 256;             // MI355X: compute units (32 per die)
constexpr int kMaxRouterSplits = 32;  // split-K pieces of the router for small batches
constexpr int kBalTokens = 64;        // tokens per block of the balance-statistics kernel
constexpr int kBalMaxBlocks = 512;    // blocks (and partial rows) of that kernel at most
constexpr int kSmallTokens = 64;      // batches up to this size route and dispatch in one block

// ---------------------------------------------------------------------------
// device workspace layout (byte offsets from the workspace base)

struct WsLayout {
  size_t logits;        // f64 [splits][N][E] router partial sums
  size_t topk_idx;      // i32 [N*k]
  size_t topk_w;        // f32 [N*k]
  size_t counts;        // i32 [E]
  size_t mod_counts;    // i32 [2][E]
  size_t offsets;       // i32 [E+1]
  size_t row_of;        // i32 [N*k]
  size_t token_of_row;  // i32 [N*k]
  size_t drop;          // u8  [N*k]
  size_t lrank;         // i32 [N*k]   block-local ranks
  size_t blk_counts;    // i32 [nblk][E] per-block demand, then per-block bases
  size_t plan;          // i32 [3*G+1] tile plan of the grouped GEMMs
  size_t h;             // act [N*k + N*S][I]   expert hidden activations
  size_t yrows;         // act [N*k + N*S][d]   expert outputs per row
  size_t bal;           // f64 [balance blocks][E] partial probability sums
  size_t alt;           // i32 [N*k]  alternate experts (reroute policy)
  size_t cand;          // i32 [N*k]  offered expert of each dropped slot
  size_t lrank2;        // i32 [N*k]  block-local ranks of the offers
  size_t blk2;          // i32 [nblk][3][E] per-block offers, then bases
  size_t kept1;         // i32 [E]    first-round rows per expert
  size_t total;
};

WsLayout ws_layout(const moe_problem* p);
int64_t perm_blocks(int64_t N);

// plan layout: tile_start[G+1], row_begin[G], rows[G].  The workspace holds
// two plans (the second for the remainder tiles of the direct-to-LDS GEMM),
// plan_stride(G) ints apart.
inline int64_t plan_stride(int G) { return (3 * (int64_t)G + 1 + 63) / 64 * 64; }
inline size_t plan_bytes(int G) { return (size_t)(2 * plan_stride(G)) * 4; }
struct PlanView {
  int32_t* tile_start;
  int32_t* row_begin;
  int32_t* rows;
};
inline PlanView plan_view(int32_t* plan, int G) {
  return PlanView{plan, plan + (G + 1), plan + (G + 1) + G};
}

// ---------------------------------------------------------------------------
// launchers (each enqueues on `stream`, returns hipError_t of the launch)

// Router logits as float64 partial sums over `nsplit` pieces of d
// ([nsplit][N][E]); router_splits() picks nsplit for a problem and
// router_splits_used() the number of pieces actually launched.
int router_splits(int64_t N, int d, int E);
int router_splits_used(int d, int nsplit);
hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* w, double* zpart, int nsplit,
                              int64_t N, int d, int E, hipStream_t s);
hipError_t launch_router_f32(const float* x, const float* w, double* z, int64_t N, int d, int E,
                             hipStream_t s);
// top-k over the summed partials (+ logit offset); z_out (nullable) receives z
// alt (nullable) [N*k]: the experts ranked k+1 .. 2k, -1 past E
hipError_t launch_topk(const double* zpart, int nsplit, const float* logit_bias, double* z_out,
                       const float* sel_bias, const uint8_t* modality, int n_bias_sets,
                       int gating, int renormalize, int32_t* idx, float* w, int32_t* alt,
                       int64_t N, int E, int k, hipStream_t s);
hipError_t launch_hash_route(const int64_t* ids, int64_t N, int E, int k, int32_t* idx,
                             float* w, hipStream_t s);

// Small batches (N <= kSmallTokens, drop policy): demand histograms, capacity,
// ranks, permutation and the grouped-GEMM tile plan (BM-row tiles, no
// remainder plan) in one single-block launch, after the top-k.
struct SmallDispatch {
  const int32_t* idx;               // [N*k] the routing (expert of each assignment)
  const uint8_t* modality;          // nullable (required with mod_counts)
  int32_t *counts, *mod_counts, *offsets, *row_of, *token_of_row, *final_idx;
  uint8_t* drop;
  int64_t C;                        // capacity, < 0 unlimited
  int64_t N;
  int E, k;
  int n_ident;                      // shared experts (dense groups of the plan)
  int64_t ident_row0;               // first row of the dense groups
  int BM;                           // tile rows of the grouped GEMMs
  int32_t* plan;                    // tile plan out
  int32_t* sat;                     // nullable: range count, zeroed here
};
hipError_t launch_dispatch_small(const SmallDispatch& a, hipStream_t s);

hipError_t launch_permute(const int32_t* idx, const uint8_t* modality, int32_t* counts,
                          int32_t* mod_counts, int32_t* offsets, int32_t* row_of,
                          int32_t* token_of_row, uint8_t* drop, int32_t* lrank,
                          int32_t* blk_counts, int64_t N, int E, int k, int64_t C,
                          hipStream_t s);
// final_idx[a] = idx[a] if row_of[a] >= 0 else -1 (the drop policy's final experts)
hipError_t launch_final_idx(const int32_t* idx, const int32_t* row_of, int32_t* final_idx,
                            int64_t nk, hipStream_t s);
// Reroute policy: as launch_permute, then the q-th dropped slot of a token goes
// to alt[t*k+q] if that expert has room; final_idx (nullable) gets the expert
// that processes each slot (-1 if dropped).  Scratch: cand, lrank2 [N*k],
// blk2 [nblk][3][E], kept1 [E].
hipError_t launch_permute_reroute(const int32_t* idx, const int32_t* alt,
                                  const uint8_t* modality, int32_t* counts,
                                  int32_t* mod_counts, int32_t* offsets, int32_t* row_of,
                                  int32_t* token_of_row, uint8_t* drop, int32_t* final_idx,
                                  int32_t* lrank, int32_t* blk_counts, int32_t* cand,
                                  int32_t* lrank2, int32_t* blk2, int32_t* kept1, int64_t N,
                                  int E, int k, int64_t C, hipStream_t s);

// Grouped FFN over G groups.  Groups [0, n_gather) are routed experts whose
// rows come from `offsets` (row r of group g is x[token_of_row[offsets[g]+r]]);
// the remaining groups are dense over all N tokens, one per "identity" weight
// set, writing rows [identity_row0 + i*N, ...).
struct FfnCall {
  int dtype;                   // MOE_BF16 / MOE_F32
  int activation;              // MOE_SWIGLU / MOE_RELU
  float clip;
  int64_t N;                   // tokens
  int d, I;
  int n_gather;                // routed groups (0 for the dense-only call)
  int64_t routed_rows;         // N*k: rows available to the routed groups
  const int32_t* offsets;      // [n_gather+1] device, or NULL
  const int32_t* token_of_row; // device, or NULL
  int n_ident;                 // dense groups
  int64_t identity_row0;       // first row of the dense groups in h / y_rows
  const void* x;
  const void *wg, *wu, *wd;    // routed weights ([n_gather][..])
  const void *sg, *su, *sd;    // dense-group weights ([n_ident][..])
  void* h;                     // [rows][I]
  void* y_rows;                // [rows][d]
  int32_t* plan;               // workspace for the tile plan
  void* marks[6];              // optional hipEvent_t: before/after plan, gate/up, down
  void *save_a, *save_u;       // optional fp16 [rows][I] pre-activations (bf16 path)
  int32_t* sat;                // optional: zeroed by the plan, then the count of
                               // stored h and y_rows values of magnitude 65504
  int plan_ready;              // 1: the tile plan (and the zeroed sat) are already in
                               // `plan` (written by the small-batch dispatch)
};
hipError_t launch_ffn(const FfnCall& c, hipStream_t s);
// Rows per tile of the grouped GEMMs' tile plan for this call.
int ffn_plan_rows(const FfnCall& c);
// The tile plan alone (BM-row tiles, no remainder plan), for other grouped GEMMs.
hipError_t launch_ffn_plan(const int32_t* offsets, int n_gather, int n_ident, int64_t N,
                           int64_t rows_cap, int64_t ident_row0, int BM, int32_t* plan,
                           hipStream_t s);

// Balancing statistics: P_e partial sums per block, then load, P, aux and the
// optional +-gamma update of the selection biases.
int64_t balance_blocks(int64_t N);
hipError_t launch_balance(const double* z, const int32_t* counts, const int32_t* mod_counts,
                          double* partial, double* load, double* mean_prob, double* aux,
                          float* sel_bias, int n_bias_sets, float gamma, int gating,
                          int64_t N, int E, int k, hipStream_t s);

// Backward pass (bf16 operands, float32 gradients).
struct BwdLayout {
  size_t plan, plan_r;     // tile plans: experts + shared; one dense group (router)
  size_t slot;             // i32 [N*k]  slot of each kept routed row
  size_t dy16;             // bf16 [N][d]
  size_t xg, dyg;          // bf16 [N*k][d]  x and dy of each routed row
  size_t af, uf, dhu;      // f32 [R][I]  a, u recomputed; dy W_down per row
  size_t hg, da, du;       // bf16 [R][I] g h, da, du
  size_t dgr;              // f32 [R]     dg of each row
  size_t dxp;              // f32 [R][d]  per-row input gradient
  size_t dz;               // f32 [N][E]
  size_t dz16;             // bf16 [N][Ep]  (E rounded up to 8, zero padded)
  size_t colsum;           // f64 [blocks][E]
  size_t part;             // f32 partial weight gradients of the dense groups' pieces
  size_t total;
};
BwdLayout bwd_ws_layout(const moe_problem* p);
struct BwdCall {
  int64_t N;
  int d, I, E, k, S;
  int gating, activation, renormalize;
  float clip;
  const void* x;                               // bf16 [N][d]
  const void *wr, *wg, *wu, *wd, *sg, *su, *sd;
  const float* dy;                             // f32 [N][d]
  const double* logits;                        // [N][E]
  const int32_t *topk_idx, *offsets, *row_of, *token_of_row;
  const float* topk_w;
  const uint16_t *act_a, *act_u;               // optional fp16 saved pre-activations
  float* dx;
  void *dw_router, *dw_gate, *dw_up, *dw_down, *dws_gate, *dws_up, *dws_down;
  int dw_bf16;                                 // weight gradients in bf16
  float *d_logit_bias, *dz_out, *dg_out;       // nullable
  void* ws;
  BwdLayout L;
  void* marks[2 * MOE_NUM_BSTAGES];            // optional hipEvent_t around each stage
};
hipError_t launch_backward(const BwdCall& c, hipStream_t s);

hipError_t launch_combine(int dtype, const void* y_rows, const int32_t* row_of,
                          const float* topk_w, const void* y_shared, int64_t shared_stride_rows,
                          int S, void* y, int64_t N, int d, int k, hipStream_t s);

// ---------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round to nearest, ties to even
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even, saturating at +-65504
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  f = fminf(fmaxf(f, -65504.0f), 65504.0f);
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// How many of the two fp16 values packed in w have fp16's largest magnitude,
// 65504: every saturated value (beyond the range, or NaN, which the clamp
// sends to -65504) and the in-range ones that round there (|v| > 65488).
__device__ __forceinline__ int f16x2_at_limit(uint32_t w) {
  return ((w & 0x7fffu) == 0x7bffu) + (((w >> 16) & 0x7fffu) == 0x7bffu);
}
// f32_to_f16_sat, adding to n when the result has magnitude 65504 (as above)
__device__ __forceinline__ uint16_t f32_to_f16_sat_n(float f, int& n) {
  const uint16_t b = f32_to_f16_sat(f);
  n += (b & 0x7fffu) == 0x7bffu;
  return b;
}
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
// two packed bf16 -> two packed fp16.  Exact for values in fp16's normal range
// (bf16's 8-bit significand fits in fp16's 11 bits); smaller magnitudes are
// truncated to the fp16 subnormal grid (error < 2^-24); larger ones saturate.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __uint_as_float(w << 16);
  const float hi = __uint_as_float(w & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Exclusive scan of n (<= 2 * blockDim) ints held in LDS `v`; returns the total.
// blockDim.x must be 1024.
__device__ inline int block_exclusive_scan_1024(int32_t* v, int n, int32_t* tmp) {
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int lo = tid * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < n) s += v[lo + i];
  tmp[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (tid >= off) ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int total = tmp[1023];
  int run = tmp[tid] - s;   // exclusive prefix of this thread's chunk
  for (int i = 0; i < per; ++i)
    if (lo + i < n) {
      const int x = v[lo + i];
      v[lo + i] = run;
      run += x;
    }
  __syncthreads();
  return total;
}

}  // namespace moe
