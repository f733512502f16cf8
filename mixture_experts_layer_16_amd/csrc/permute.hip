// Dispatch: per-expert histogram, capacity, token-order ranks and the slot
// permutation.
//
// The capacity rule and the slot order are those of "Mixture-of-Experts :
// routage et capacité" (cours.spawnkit.ai), sections "L'idée — Capacité" and
// "Cas guidé — trace complète": tokens arrive in batch order, expert e keeps its
// first C arrivals (C = ceil(N*k/E * f)) and drops the rest; kept assignments
// are packed expert by expert, in arrival order.
//
// Ranks must follow token order, so they are not taken from atomics (whose
// order follows the hardware).  Three passes:
//   1. rank:    per block of 256 tokens, each wave ranks its 64 tokens' k
//               assignments with ballot-built peer masks (lanes holding the same
//               expert), keeps per-wave running counts in LDS, then turns them
//               into block-local ranks and a per-block histogram (also split by
//               modality);
//   2. scan:    per expert, an exclusive scan of the block histograms (in
//               runs of blocks, one thread per run) gives each block's base
//               rank and the expert's demand; kept = min(demand, C); an
//               exclusive scan over experts gives the offsets;
//   3. scatter: rank = block base + local rank; kept iff rank < C.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int PR_WAVES = kPermTokens / 64;   // 4 waves, 64 tokens each

__device__ __forceinline__ int expert_bits(int E) {
  int b = 1;
  while ((1 << b) < E) ++b;
  return b;
}

// stride of one block's histogram record: [3][E] (all, text, image)
__global__ __launch_bounds__(256) void perm_rank_kernel(
    const int32_t* __restrict__ idx, const uint8_t* __restrict__ modality,
    int32_t* __restrict__ lrank, int32_t* __restrict__ blk, int64_t N, int E, int k) {
  extern __shared__ int32_t lds[];                // cnt[4][E], then mcnt[2][E]
  int32_t* cnt = lds;
  int32_t* mcnt = lds + PR_WAVES * E;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < (PR_WAVES + 2) * E; i += blockDim.x) lds[i] = 0;
  __syncthreads();

  const int64_t NK = N * k;
  const int64_t a_wave = ((int64_t)blockIdx.x * kPermTokens + 64 * wave) * k;
  const int nbits = expert_bits(E);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* wcnt = cnt + wave * E;

  for (int c = 0; c < k; ++c) {
    const int64_t a = a_wave + (int64_t)c * 64 + lane;
    int e = -1;
    if (a < NK) e = idx[a];
    const bool valid = (e >= 0) && (e < E);
    uint64_t peers = __ballot(valid);
#pragma unroll 1
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = valid && ((e >> bit) & 1);
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    if (valid) {
      const int before = __popcll(peers & lt_mask);
      const int old = wcnt[e];
      if (before == 0) wcnt[e] = old + __popcll(peers);   // the group's lowest lane
      lrank[a] = old + before;
      if (modality) atomicAdd(&mcnt[(modality[a / k] ? 1 : 0) * E + e], 1);
    }
  }
  __syncthreads();

  int32_t* rec = blk + (int64_t)blockIdx.x * 3 * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < PR_WAVES; ++w) {
      const int v = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += v;
    }
    rec[e] = run;
    rec[E + e] = mcnt[e];
    rec[2 * E + e] = mcnt[E + e];
  }
  __syncthreads();

  for (int c = 0; c < k; ++c) {
    const int64_t a = a_wave + (int64_t)c * 64 + lane;
    if (a >= NK) break;
    const int e = idx[a];
    if (e >= 0 && e < E) lrank[a] += wcnt[e];
  }
}

// Block-histogram scan, one block of 1024 threads.  Thread t works on expert
// e = t % E and on the c-th (c = t / E) of tpe <= 1024 / E runs of consecutive
// blocks, so neighbouring threads read neighbouring words of a block record.
// Pass 1 sums each run; an expert's run sums are added up in run order (LDS)
// for each run's starting rank; pass 2 walks the run again and writes each
// block's base rank.  Loads go out in batches of 8 blocks.
constexpr int SCAN_BATCH = 8;

__global__ __launch_bounds__(1024) void perm_scan_kernel(
    int32_t* __restrict__ blk, int nblk, int32_t* __restrict__ counts,
    int32_t* __restrict__ mod_counts, int32_t* __restrict__ offsets, int E, int64_t C) {
  __shared__ int32_t kept[kMaxExperts];
  __shared__ int32_t tmp[1024];
  __shared__ int32_t part[3][1024];
  const int tid = threadIdx.x;
  // runs per expert (E <= 1024): as many as the threads allow, but no shorter
  // than one batch of blocks, so the run sums stay few
  const int tpe = max(1, min(1024 / E, (nblk + SCAN_BATCH - 1) / SCAN_BATCH));
  const int e = tid % E, c = tid / E;
  const bool act = c < tpe;
  const int L = (nblk + tpe - 1) / tpe;
  const int b0 = act ? c * L : 0;
  const int b1 = act ? min(nblk, b0 + L) : 0;
  int v = 0, a0 = 0, a1 = 0;
  for (int b = b0; b < b1; b += SCAN_BATCH) {
    int x[SCAN_BATCH], y0[SCAN_BATCH], y1[SCAN_BATCH];
#pragma unroll
    for (int i = 0; i < SCAN_BATCH; ++i) {
      x[i] = y0[i] = y1[i] = 0;
      if (b + i < b1) {
        const int32_t* rec = blk + (int64_t)(b + i) * 3 * E;
        x[i] = rec[e];
        y0[i] = rec[E + e];
        y1[i] = rec[2 * E + e];
      }
    }
#pragma unroll
    for (int i = 0; i < SCAN_BATCH; ++i) {
      v += x[i];
      a0 += y0[i];
      a1 += y1[i];
    }
  }
  part[0][tid] = v;
  part[1][tid] = a0;
  part[2][tid] = a1;
  __syncthreads();
  if (act) {
    int run = 0;   // ranks held by the expert's earlier runs
    for (int q = 0; q < c; ++q) run += part[0][q * E + e];
    for (int b = b0; b < b1; b += SCAN_BATCH) {
      int x[SCAN_BATCH];
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i)
        x[i] = (b + i < b1) ? blk[(int64_t)(b + i) * 3 * E + e] : 0;
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i)
        if (b + i < b1) {
          blk[(int64_t)(b + i) * 3 * E + e] = run;
          run += x[i];
        }
    }
    if (c == tpe - 1) {   // the last run ends at the expert's demand
      int m0 = 0, m1 = 0;
      for (int q = 0; q < tpe; ++q) {
        m0 += part[1][q * E + e];
        m1 += part[2][q * E + e];
      }
      counts[e] = run;
      if (mod_counts) {
        mod_counts[e] = m0;
        mod_counts[E + e] = m1;
      }
      kept[e] = (C < 0 || run < C) ? run : (int)C;
    }
  }
  __syncthreads();
  const int total = block_exclusive_scan_1024(kept, E, tmp);
  for (int e2 = tid; e2 < E; e2 += blockDim.x) offsets[e2] = kept[e2];
  if (tid == 0) offsets[E] = total;
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of_row,
    uint8_t* __restrict__ drop, int64_t N, int E, int k, int64_t C) {
  const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= N * k) return;
  const int e = idx[a];
  if (e < 0 || e >= E) {
    row_of[a] = -1;
    drop[a] = 1;
    return;
  }
  const int64_t t = a / k;
  const int64_t b = t / kPermTokens;
  const int64_t r = (int64_t)blk[b * 3 * E + e] + lrank[a];
  if (C < 0 || r < C) {
    const int row = offsets[e] + (int)r;
    row_of[a] = row;
    token_of_row[row] = (int32_t)t;
    drop[a] = 0;
  } else {
    row_of[a] = -1;
    drop[a] = 1;
  }
}

// ---- reroute policy ("Report sur E2/E3" of the routing slides' overflow
// table): the q-th dropped slot of a token is offered to its alternate
// expert alt[t*k+q]; experts accept offers in token order while they have
// room left after their own first-round rows.

// one thread per token: the candidate expert of each dropped slot (else -1)
__global__ __launch_bounds__(256) void perm_cand_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ alt,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ blk,
    int32_t* __restrict__ cand, int64_t N, int E, int k, int64_t C) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const int64_t b = t / kPermTokens;
  int q = 0;
  for (int j = 0; j < k; ++j) {
    const int64_t a = t * k + j;
    const int e = idx[a];
    int c = -1;
    if (e >= 0 && e < E && C >= 0) {
      const int64_t r = (int64_t)blk[b * 3 * E + e] + lrank[a];
      if (r >= C) {
        c = alt[t * k + q];
        if (c < 0 || c >= E) c = -1;
        ++q;
      }
    }
    cand[a] = c;
  }
}

// one wave per expert: scan the second-round block histograms into bases,
// accept min(offers, room), and lay out offsets = first-round rows followed
// by accepted offers, expert by expert
__global__ __launch_bounds__(1024) void perm_merge_kernel(
    int32_t* __restrict__ blk2, int nblk, int32_t* __restrict__ offsets,
    int32_t* __restrict__ kept1, int E, int64_t C) {
  __shared__ int32_t k1[kMaxExperts];
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t tmp[1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) k1[e] = offsets[e + 1] - offsets[e];
  __syncthreads();
  for (int e = wave; e < E; e += nwaves) {
    int carry = 0;
    for (int b0 = 0; b0 < nblk; b0 += 64) {
      const int b = b0 + lane;
      int v = 0;
      if (b < nblk) v = blk2[(int64_t)b * 3 * E + e];
      int incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      if (b < nblk) blk2[(int64_t)b * 3 * E + e] = carry + incl - v;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) {
      const int64_t room = C - k1[e];
      tot[e] = k1[e] + (int)((int64_t)carry < room ? carry : room);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) kept1[e] = k1[e];
  const int total = block_exclusive_scan_1024(tot, E, tmp);
  for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = tot[e];
  if (threadIdx.x == 0) offsets[E] = total;
}

__global__ __launch_bounds__(256) void perm_scatter_reroute_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cand,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ lrank2, const int32_t* __restrict__ blk2,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ kept1,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of_row,
    uint8_t* __restrict__ drop, int32_t* __restrict__ final_idx, int64_t N, int E, int k,
    int64_t C) {
  const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= N * k) return;
  const int64_t t = a / k;
  const int64_t b = t / kPermTokens;
  const int e = idx[a];
  int row = -1, fe = -1;
  if (e >= 0 && e < E) {
    const int64_t r = (int64_t)blk[b * 3 * E + e] + lrank[a];
    if (C < 0 || r < C) {
      row = offsets[e] + (int)r;
      fe = e;
    } else {
      const int c = cand[a];
      if (c >= 0) {
        const int64_t r2 = (int64_t)blk2[b * 3 * E + c] + lrank2[a];
        if (r2 < C - kept1[c]) {
          row = offsets[c] + kept1[c] + (int)r2;
          fe = c;
        }
      }
    }
  }
  row_of[a] = row;
  drop[a] = row < 0 ? 1 : 0;
  if (row >= 0) token_of_row[row] = (int32_t)t;
  if (final_idx) final_idx[a] = fe;
}

__global__ __launch_bounds__(256) void final_idx_kernel(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ row_of,
                                                        int32_t* __restrict__ final_idx,
                                                        int64_t nk) {
  const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (a < nk) final_idx[a] = row_of[a] >= 0 ? idx[a] : -1;
}

// ---------------------------------------------------------------------------
// Small batches (N <= kSmallTokens): the demand histograms, capacity,
// token-order ranks, the permutation and the grouped-GEMM tile plan in one
// block of 1024 threads, instead of the rank, scan, scatter and plan launches
// -- with a handful of tokens each of those is mostly start-up latency.  The
// results equal the separate kernels' (ranks by the same rule: an assignment's
// rank is the number of earlier assignments, in token-major order, to its
// expert).
__global__ __launch_bounds__(1024) void dispatch_small_kernel(SmallDispatch a) {
  __shared__ int32_t sidx[kSmallTokens * kMaxTopK];
  __shared__ int32_t srank[kSmallTokens * kMaxTopK];
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t mcnt[2 * kMaxExperts];
  __shared__ int32_t kept[kMaxExperts];
  __shared__ int32_t mt[2 * 1024];
  __shared__ int32_t tmp[1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = a.E, k = a.k;
  const int64_t N = a.N;
  const int NK = (int)(N * k);
  for (int e = tid; e < E; e += 1024) {
    cnt[e] = 0;
    mcnt[e] = 0;
    mcnt[E + e] = 0;
  }
  for (int i = tid; i < NK; i += 1024) sidx[i] = a.idx[i];
  __syncthreads();
  // 1. token-order ranks and demand: one wave walks the assignments in order,
  // 64 at a time; lanes naming the same expert find each other with one
  // ballot per bit of the expert index
  if (wave == 0) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < NK; c0 += 64) {
      const int i = c0 + lane;
      const int e = i < NK ? sidx[i] : -1;
      const bool valid = e >= 0 && e < E;
      uint64_t peers = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool on = valid && ((e >> bit) & 1);
        const uint64_t m = __ballot(on);
        peers &= on ? m : ~m;
      }
      if (valid) {
        const int before = __popcll(peers & lt_mask);
        const int old = cnt[e];
        if (before == 0) cnt[e] = old + __popcll(peers);
        srank[i] = old + before;
        if (a.mod_counts) atomicAdd(&mcnt[(a.modality[i / k] ? 1 : 0) * E + e], 1);
      }
    }
  }
  __syncthreads();
  // 2. demand out, kept = min(demand, C), offsets = exclusive prefix sums
  for (int e = tid; e < E; e += 1024) {
    const int c = cnt[e];
    a.counts[e] = c;
    if (a.mod_counts) {
      a.mod_counts[e] = mcnt[e];
      a.mod_counts[E + e] = mcnt[E + e];
    }
    kept[e] = (a.C < 0 || c < a.C) ? c : (int)a.C;
  }
  __syncthreads();
  const int A = block_exclusive_scan_1024(kept, E, tmp);
  for (int e = tid; e < E; e += 1024) a.offsets[e] = kept[e];
  if (tid == 0) a.offsets[E] = A;
  // 3. the permutation (kept[] now holds the offsets)
  for (int i = tid; i < NK; i += 1024) {
    const int e = sidx[i];
    int row = -1;
    if (e >= 0 && e < E && (a.C < 0 || srank[i] < a.C)) {
      row = kept[e] + srank[i];
      a.token_of_row[row] = i / k;
    }
    a.row_of[i] = row;
    a.drop[i] = row < 0 ? 1 : 0;
    if (a.final_idx) a.final_idx[i] = row < 0 ? -1 : e;
  }
  // 4. tile plan of the grouped GEMMs: the routed groups' rows from the
  // offsets, then one dense group of N rows per shared expert
  const int G = E + a.n_ident;
  int32_t* tile_start = a.plan;
  int32_t* row_begin = a.plan + G + 1;
  int32_t* rows = row_begin + G;
  for (int g = tid; g < G; g += 1024) {
    int rb, r;
    if (g < E) {
      rb = kept[g];
      r = (g + 1 < E ? kept[g + 1] : A) - rb;
    } else {
      rb = (int)(a.ident_row0 + (int64_t)(g - E) * N);
      r = (int)N;
    }
    row_begin[g] = rb;
    rows[g] = r;
    mt[g] = (r + a.BM - 1) / a.BM;
  }
  __syncthreads();
  const int total = block_exclusive_scan_1024(mt, G, tmp);
  for (int g = tid; g < G; g += 1024) tile_start[g] = mt[g];
  if (tid == 0) {
    tile_start[G] = total;
    if (a.sat) *a.sat = 0;   // the range count of this call starts at zero
  }
}

}  // namespace

hipError_t launch_dispatch_small(const SmallDispatch& a, hipStream_t s) {
  dispatch_small_kernel<<<1, 1024, 0, s>>>(a);
  return hipGetLastError();
}

int64_t perm_blocks(int64_t N) { return (N + kPermTokens - 1) / kPermTokens; }

hipError_t launch_final_idx(const int32_t* idx, const int32_t* row_of, int32_t* final_idx,
                            int64_t nk, hipStream_t s) {
  final_idx_kernel<<<(unsigned)((nk + 255) / 256), 256, 0, s>>>(idx, row_of, final_idx, nk);
  return hipGetLastError();
}

hipError_t launch_permute_reroute(const int32_t* idx, const int32_t* alt,
                                  const uint8_t* modality, int32_t* counts,
                                  int32_t* mod_counts, int32_t* offsets, int32_t* row_of,
                                  int32_t* token_of_row, uint8_t* drop, int32_t* final_idx,
                                  int32_t* lrank, int32_t* blk_counts, int32_t* cand,
                                  int32_t* lrank2, int32_t* blk2, int32_t* kept1, int64_t N,
                                  int E, int k, int64_t C, hipStream_t s) {
  const int64_t nblk = perm_blocks(N);
  const size_t lds = (size_t)(PR_WAVES + 2) * E * sizeof(int32_t);
  perm_rank_kernel<<<(unsigned)nblk, 256, lds, s>>>(idx, mod_counts ? modality : nullptr,
                                                     lrank, blk_counts, N, E, k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_scan_kernel<<<1, 1024, 0, s>>>(blk_counts, (int)nblk, counts, mod_counts, offsets, E, C);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_cand_kernel<<<(unsigned)((N + 255) / 256), 256, 0, s>>>(idx, alt, lrank, blk_counts,
                                                                 cand, N, E, k, C);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_rank_kernel<<<(unsigned)nblk, 256, lds, s>>>(cand, nullptr, lrank2, blk2, N, E, k);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_merge_kernel<<<1, 1024, 0, s>>>(blk2, (int)nblk, offsets, kept1, E, C);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t nk = N * k;
  perm_scatter_reroute_kernel<<<(unsigned)((nk + 255) / 256), 256, 0, s>>>(
      idx, cand, lrank, blk_counts, lrank2, blk2, offsets, kept1, row_of, token_of_row, drop,
      final_idx, N, E, k, C);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const uint8_t* modality, int32_t* counts,
                          int32_t* mod_counts, int32_t* offsets, int32_t* row_of,
                          int32_t* token_of_row, uint8_t* drop, int32_t* lrank,
                          int32_t* blk_counts, int64_t N, int E, int k, int64_t C,
                          hipStream_t s) {
  const int64_t nblk = perm_blocks(N);
  const size_t lds = (size_t)(PR_WAVES + 2) * E * sizeof(int32_t);
  perm_rank_kernel<<<(unsigned)nblk, 256, lds, s>>>(idx, mod_counts ? modality : nullptr,
                                                     lrank, blk_counts, N, E, k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_scan_kernel<<<1, 1024, 0, s>>>(blk_counts, (int)nblk, counts, mod_counts, offsets, E, C);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t nk = N * k;
  perm_scatter_kernel<<<(unsigned)((nk + 255) / 256), 256, 0, s>>>(
      idx, lrank, blk_counts, offsets, row_of, token_of_row, drop, N, E, k, C);
  return hipGetLastError();
}

}  // namespace moe
