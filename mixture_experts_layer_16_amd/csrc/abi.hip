// C-ABI entry points: host-side validation, exact capacity, workspace layout
// and the launch sequence of each stage.  No allocation, no synchronisation.
#include <math.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

// Scratch of the allocation-free entry point (moe_forward_noalloc): one copy
// per GPU, held until the process ends.  Host code never uses this name as an
// address (on the host it is a stand-in, not device memory): it uses the
// device address hipGetSymbolAddress returns, kept per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

WsLayout ws_layout(const moe_problem* p) {
  const size_t N = (size_t)p->n_tokens, E = (size_t)p->n_experts, k = (size_t)p->top_k;
  const size_t S = (size_t)p->n_shared, d = (size_t)p->d_model, I = (size_t)p->d_expert;
  const size_t esz = p->dtype == MOE_BF16 ? 2 : 4;
  const size_t nk = N * k;
  const size_t nblk = (size_t)perm_blocks((int64_t)N);
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes ? bytes : 1);
    return o;
  };
  const size_t nsplit =
      p->dtype == MOE_BF16
          ? (size_t)router_splits_used(p->d_model, router_splits((int64_t)N, p->d_model, (int)E))
          : 1;
  L.logits = take(nsplit * N * E * 8);
  L.topk_idx = take(nk * 4);
  L.topk_w = take(nk * 4);
  L.counts = take(E * 4);
  L.mod_counts = take(2 * E * 4);
  L.offsets = take((E + 1) * 4);
  L.row_of = take(nk * 4);
  L.token_of_row = take(nk * 4);
  L.drop = take(nk);
  L.lrank = take(nk * 4);
  L.blk_counts = take(nblk * 3 * E * 4);
  L.plan = take(plan_bytes((int)(E + S)));
  L.h = take((nk + N * S) * I * esz);
  L.yrows = take((nk + N * S) * d * esz);
  L.bal = take((size_t)balance_blocks((int64_t)N) * E * 8);
  L.alt = take(nk * 4);
  L.cand = take(nk * 4);
  L.lrank2 = take(nk * 4);
  L.blk2 = take(nblk * 3 * E * 4);
  L.kept1 = take(E * 4);
  L.total = off;
  return L;
}

static int validate(const moe_problem* p) {
  if (!p) return MOE_ERR_NULL;
  if (p->n_tokens < 0 || p->n_tokens > (int64_t(1) << 24)) return MOE_ERR_INVALID;
  if (p->d_model < 1 || p->d_expert < 1) return MOE_ERR_INVALID;
  if (p->n_experts < 1 || p->n_experts > kMaxExperts) return MOE_ERR_INVALID;
  if (p->top_k < 1 || p->top_k > p->n_experts || p->top_k > kMaxTopK) return MOE_ERR_INVALID;
  if (p->n_shared < 0 || p->n_shared > kMaxShared) return MOE_ERR_INVALID;
  if (p->gating != MOE_SOFTMAX && p->gating != MOE_SIGMOID) return MOE_ERR_INVALID;
  if (p->activation != MOE_SWIGLU && p->activation != MOE_RELU) return MOE_ERR_INVALID;
  if (p->dtype != MOE_BF16 && p->dtype != MOE_F32) return MOE_ERR_INVALID;
  if (p->n_bias_sets < 0 || p->n_bias_sets > 2) return MOE_ERR_INVALID;
  if (!(p->act_clip >= 0.0f)) return MOE_ERR_INVALID;             // rejects NaN
  if (isnan(p->capacity_factor)) return MOE_ERR_INVALID;
  if (p->renormalize != 0 && p->renormalize != 1) return MOE_ERR_INVALID;
  if (p->overflow != MOE_OVERFLOW_DROP && p->overflow != MOE_OVERFLOW_REROUTE)
    return MOE_ERR_INVALID;
  if (p->d_model > (1 << 20) || p->d_expert > (1 << 20)) return MOE_ERR_INVALID;
  const int64_t rows = p->n_tokens * (p->top_k + p->n_shared);
  if (rows >= (int64_t(1) << 31)) return MOE_ERR_INVALID;
  if (p->dtype == MOE_BF16 && ((p->d_model % 8) || (p->d_expert % 8))) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static inline bool aligned16(const void* q) { return ((uintptr_t)q & 15u) == 0; }

// C = ceil(f * N * k / E) on the exact binary value of f; >= 1 when f > 0;
// -1 when unlimited.
static int64_t capacity_of(const moe_problem* p) {
  const double f = p->capacity_factor;
  if (!(f > 0.0)) return -1;
  if (isinf(f)) return -1;
  const int64_t nk = p->n_tokens * p->top_k;
  const int64_t E = p->n_experts;
  if (nk == 0) return 1;
  int ex = 0;
  const double fr = frexp(f, &ex);                   // f = fr * 2^ex, fr in [0.5, 1)
  const int64_t mant = (int64_t)ldexp(fr, 53);       // exact 53-bit integer
  const int q = ex - 53;                             // f = mant * 2^q
  __int128 num = (__int128)nk * mant;
  __int128 den = E;
  if (q >= 0) {
    if (q > 40) return INT64_MAX / 2;                 // astronomically large: unlimited in effect
    num <<= q;
  } else {
    if (-q >= 100) return 1;                          // value < 1
    den <<= -q;
  }
  __int128 c = (num + den - 1) / den;
  if (c < 1) c = 1;
  if (c > (__int128)(INT64_MAX / 2)) c = INT64_MAX / 2;
  return (int64_t)c;
}

static inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Router + top-k.  zpart: workspace for the float64 partial logits
// (route_partials_bytes); z_out (nullable): receives the logits.
static int route_splits(const moe_problem* p) {
  return p->dtype == MOE_BF16
             ? router_splits_used(p->d_model,
                                  router_splits(p->n_tokens, p->d_model, p->n_experts))
             : 1;
}
static size_t route_partials_bytes(const moe_problem* p) {
  return (size_t)route_splits(p) * (size_t)p->n_tokens * p->n_experts * 8;
}

// The router's logits as float64 partial sums in zpart; returns the number of
// partials, or 0 if the launch failed.
static int run_router(const moe_problem* p, const void* x, const void* w_router, double* zpart,
                      hipStream_t s) {
  const int64_t N = p->n_tokens;
  hipError_t err;
  int used = 1;
  if (p->dtype == MOE_BF16) {
    const int ns = router_splits(N, p->d_model, p->n_experts);
    used = router_splits_used(p->d_model, ns);
    err = launch_router_bf16(static_cast<const uint16_t*>(x),
                             static_cast<const uint16_t*>(w_router), zpart, ns, N, p->d_model,
                             p->n_experts, s);
  } else {
    err = launch_router_f32(static_cast<const float*>(x), static_cast<const float*>(w_router),
                            zpart, N, p->d_model, p->n_experts, s);
  }
  return err == hipSuccess ? used : 0;
}

static int run_route(const moe_problem* p, const void* x, const void* w_router,
                     const float* logit_bias, const float* sel_bias, const uint8_t* modality,
                     int32_t* idx, float* w, double* zpart, double* z_out, hipStream_t s,
                     int32_t* alt = nullptr) {
  const int used = run_router(p, x, w_router, zpart, s);
  if (!used) return MOE_ERR_HIP;
  const hipError_t err =
      launch_topk(zpart, used, logit_bias, z_out, p->n_bias_sets ? sel_bias : nullptr, modality,
                  p->n_bias_sets, p->gating, p->renormalize, idx, w, alt, p->n_tokens,
                  p->n_experts, p->top_k, s);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

static int check_route_inputs(const moe_problem* p, const void* x, const void* w_router,
                              const float* sel_bias, const uint8_t* modality) {
  if (!x || !w_router) return MOE_ERR_NULL;
  if (p->n_bias_sets > 0 && !sel_bias) return MOE_ERR_NULL;
  if (p->n_bias_sets == 2 && !modality) return MOE_ERR_NULL;
  if (p->dtype == MOE_BF16 && (!aligned16(x) || !aligned16(w_router))) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Saved pre-activations (moe_routing.act_a / act_u): bf16 layers only; SwiGLU
// takes both or neither, ReLU act_u alone; 16-byte aligned.
static int check_acts(const moe_problem* p, const moe_routing* r) {
  if (!r->act_a && !r->act_u) return MOE_OK;
  if (p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (p->activation == MOE_SWIGLU && (!r->act_a || !r->act_u)) return MOE_ERR_NULL;
  if (p->activation == MOE_RELU && (r->act_a || !r->act_u)) return MOE_ERR_INVALID;
  if (!aligned16(r->act_u) || (r->act_a && !aligned16(r->act_a))) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_workspace_size(const moe_problem* p, size_t* bytes) {
  const int st = validate(p);
  if (st) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = ws_layout(p).total;
  return MOE_OK;
}

int moe_capacity(const moe_problem* p, int64_t* C) {
  const int st = validate(p);
  if (st) return st;
  if (!C) return MOE_ERR_NULL;
  *C = capacity_of(p);
  return MOE_OK;
}

int moe_param_counts(const moe_problem* p, int64_t* expert_total, int64_t* expert_active,
                     int64_t* router) {
  const int st = validate(p);
  if (st) return st;
  if (!expert_total || !expert_active || !router) return MOE_ERR_NULL;
  const int64_t m = p->activation == MOE_SWIGLU ? 3 : 2;
  const int64_t per = m * (int64_t)p->d_model * p->d_expert;
  *expert_total = (int64_t)(p->n_experts + p->n_shared) * per;
  *expert_active = (int64_t)(p->top_k + p->n_shared) * per;
  *router = (int64_t)p->d_model * p->n_experts;
  return MOE_OK;
}

int moe_route(const moe_problem* p, const void* x, const void* w_router, const float* logit_bias,
              const float* sel_bias, const uint8_t* modality, int32_t* topk_idx, float* topk_w,
              double* logits, void* ws, size_t ws_bytes, void* stream) {
  int st = validate(p);
  if (st) return st;
  if (!topk_idx || !topk_w) return MOE_ERR_NULL;
  st = check_route_inputs(p, x, w_router, sel_bias, modality);
  if (st) return st;
  // the partial logits go to the workspace, except when there is one partial
  // and the caller's logits buffer can hold it (then the offset is added in place)
  const bool in_place = logits && route_splits(p) == 1;
  const size_t need = in_place ? 0 : route_partials_bytes(p);
  if (need && (!ws || ws_bytes < need)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_NULL;
  if (p->n_tokens == 0) return MOE_OK;
  double* zpart = in_place ? logits : static_cast<double*>(ws);
  return run_route(p, x, w_router, logit_bias, sel_bias, modality, topk_idx, topk_w, zpart, logits,
                   S(stream));
}

int moe_permute(const moe_problem* p, const int32_t* topk_idx, const uint8_t* modality,
                int32_t* counts, int32_t* modality_counts, int32_t* offsets, int32_t* row_of,
                int32_t* token_of_row, uint8_t* drop_mask, void* ws, size_t ws_bytes,
                void* stream) {
  const int st = validate(p);
  if (st) return st;
  if (!topk_idx || !counts || !offsets || !row_of || !token_of_row || !drop_mask)
    return MOE_ERR_NULL;
  if (p->overflow == MOE_OVERFLOW_REROUTE) return MOE_ERR_UNSUPPORTED;
  if (modality_counts && !modality) return MOE_ERR_NULL;
  const int64_t N = p->n_tokens;
  const size_t nk = (size_t)N * p->top_k;
  const size_t lr_bytes = align256(nk * 4 ? nk * 4 : 1);
  const size_t need = lr_bytes + (size_t)perm_blocks(N) * 3 * p->n_experts * 4;
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (N == 0) {
    // nothing routed: zero counts and offsets so the outputs are still defined
    hipError_t e1 = hipMemsetAsync(counts, 0, (size_t)p->n_experts * 4, S(stream));
    hipError_t e2 = hipMemsetAsync(offsets, 0, (size_t)(p->n_experts + 1) * 4, S(stream));
    hipError_t e3 = modality_counts
                        ? hipMemsetAsync(modality_counts, 0, (size_t)2 * p->n_experts * 4, S(stream))
                        : hipSuccess;
    return (e1 || e2 || e3) ? MOE_ERR_HIP : MOE_OK;
  }
  char* base = static_cast<char*>(ws);
  const hipError_t err = launch_permute(
      topk_idx, modality, counts, modality_counts, offsets, row_of, token_of_row, drop_mask,
      reinterpret_cast<int32_t*>(base), reinterpret_cast<int32_t*>(base + lr_bytes), N,
      p->n_experts, p->top_k, capacity_of(p), S(stream));
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_expert_ffn(const moe_problem* p, const void* x, const int32_t* token_of_row,
                   const int32_t* offsets, const void* w_gate, const void* w_up,
                   const void* w_down, void* y_rows, void* ws, size_t ws_bytes, void* stream) {
  const int st = validate(p);
  if (st) return st;
  const bool routed = token_of_row != nullptr;
  if (routed != (offsets != nullptr)) return MOE_ERR_INVALID;
  if (!x || !w_up || !w_down || !y_rows) return MOE_ERR_NULL;
  if (p->activation == MOE_SWIGLU && !w_gate) return MOE_ERR_NULL;
  if (p->dtype == MOE_BF16) {
    if (!aligned16(x) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(y_rows) ||
        (w_gate && !aligned16(w_gate)))
      return MOE_ERR_UNSUPPORTED;
  }
  const int64_t N = p->n_tokens;
  const size_t esz = p->dtype == MOE_BF16 ? 2 : 4;
  const int E = p->n_experts;
  const int G = routed ? E : 1;
  const size_t plan_sz = align256(plan_bytes(G));
  const size_t rows = routed ? (size_t)N * p->top_k : (size_t)N;
  const size_t need = plan_sz + rows * p->d_expert * esz;
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (N == 0) return MOE_OK;
  char* base = static_cast<char*>(ws);
  FfnCall c{};
  c.dtype = p->dtype;
  c.activation = p->activation;
  c.clip = p->act_clip;
  c.N = N;
  c.d = p->d_model;
  c.I = p->d_expert;
  c.x = x;
  c.plan = reinterpret_cast<int32_t*>(base);
  c.h = base + plan_sz;
  c.y_rows = y_rows;
  if (routed) {
    c.n_gather = E;
    c.routed_rows = N * p->top_k;
    c.offsets = offsets;
    c.token_of_row = token_of_row;
    c.wg = w_gate; c.wu = w_up; c.wd = w_down;
    c.n_ident = 0;
    c.identity_row0 = 0;
  } else {
    c.n_gather = 0;
    c.routed_rows = 0;
    c.n_ident = 1;
    c.identity_row0 = 0;
    c.sg = w_gate; c.su = w_up; c.sd = w_down;
  }
  return launch_ffn(c, S(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_combine(const moe_problem* p, const void* y_rows, const int32_t* row_of,
                const float* topk_w, const void* y_shared, void* y, void* stream) {
  const int st = validate(p);
  if (st) return st;
  if (!y_rows || !row_of || !topk_w || !y) return MOE_ERR_NULL;
  if (p->n_shared > 0 && !y_shared) return MOE_ERR_NULL;
  if (p->dtype == MOE_BF16 &&
      (!aligned16(y_rows) || !aligned16(y) || (y_shared && !aligned16(y_shared))))
    return MOE_ERR_UNSUPPORTED;
  if (p->n_tokens == 0) return MOE_OK;
  const hipError_t err = launch_combine(p->dtype, y_rows, row_of, topk_w, y_shared,
                                        p->n_tokens, p->n_shared, y, p->n_tokens, p->d_model,
                                        p->top_k, S(stream));
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_balance(const moe_problem* p, const double* logits, const int32_t* counts,
                const int32_t* modality_counts, double* load, double* mean_prob, double* aux,
                float* sel_bias, float gamma, void* ws, size_t ws_bytes, void* stream) {
  const int st = validate(p);
  if (st) return st;
  if (!(gamma >= 0.0f) || gamma > 3.0e38f) return MOE_ERR_INVALID;   // rejects NaN too
  if (sel_bias && p->n_bias_sets == 0) return MOE_ERR_INVALID;
  if ((mean_prob || aux) && !logits) return MOE_ERR_NULL;
  if ((load || aux) && !counts) return MOE_ERR_NULL;
  if (sel_bias && p->n_bias_sets == 1 && !counts) return MOE_ERR_NULL;
  if (sel_bias && p->n_bias_sets == 2 && !modality_counts) return MOE_ERR_NULL;
  const size_t need = align256((size_t)balance_blocks(p->n_tokens) * p->n_experts * 8);
  if (mean_prob || aux) {
    if (!ws) return MOE_ERR_NULL;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  }
  if (!load && !mean_prob && !aux && !sel_bias) return MOE_OK;
  const hipError_t err =
      launch_balance(logits, counts, modality_counts, static_cast<double*>(ws), load, mean_prob,
                     aux, sel_bias, p->n_bias_sets, gamma, p->gating, p->n_tokens,
                     p->n_experts, p->top_k, S(stream));
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_route_hash(const moe_problem* p, const int64_t* token_ids, int32_t* topk_idx,
                   float* topk_w, void* stream) {
  const int st = validate(p);
  if (st) return st;
  if (!token_ids || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (p->n_tokens == 0) return MOE_OK;
  return launch_hash_route(token_ids, p->n_tokens, p->n_experts, p->top_k, topk_idx, topk_w,
                           S(stream)) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

int moe_forward(const moe_problem* p, const moe_weights* w, const void* x,
                const float* logit_bias, const float* sel_bias, const uint8_t* modality, void* y,
                const moe_routing* routing_out, void* ws, size_t ws_bytes, void* stream) {
  return moe_forward_ex(p, w, x, logit_bias, sel_bias, modality, y, routing_out, nullptr, ws,
                        ws_bytes, stream);
}

// The layer after routing (permute, experts, combine) and, unless a routing
// is given (forced_idx != NULL), the routing itself.
static int forward_impl(const moe_problem* p, const moe_weights* w, const void* x,
                        const float* logit_bias, const float* sel_bias,
                        const uint8_t* modality, void* y, const moe_routing* routing_out,
                        const moe_profile* prof, void* ws, size_t ws_bytes, void* stream,
                        const int32_t* forced_idx, const float* forced_w) {
  int st = validate(p);
  if (st) return st;
  if (!w || !y) return MOE_ERR_NULL;
  if (forced_idx) {
    if (p->overflow == MOE_OVERFLOW_REROUTE) return MOE_ERR_UNSUPPORTED;
    if (!forced_w || !x) return MOE_ERR_NULL;
    if (p->dtype == MOE_BF16 && !aligned16(x)) return MOE_ERR_UNSUPPORTED;
  } else {
    st = check_route_inputs(p, x, w->w_router, sel_bias, modality);
    if (st) return st;
  }
  if (!w->w_up || !w->w_down) return MOE_ERR_NULL;
  if (p->activation == MOE_SWIGLU && !w->w_gate) return MOE_ERR_NULL;
  if (p->n_shared > 0) {
    if (!w->ws_up || !w->ws_down) return MOE_ERR_NULL;
    if (p->activation == MOE_SWIGLU && !w->ws_gate) return MOE_ERR_NULL;
  }
  if (p->dtype == MOE_BF16) {
    const void* ptrs[] = {w->w_gate, w->w_up, w->w_down, w->ws_gate, w->ws_up, w->ws_down, y};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return MOE_ERR_UNSUPPORTED;
  }
  if (routing_out && routing_out->modality_counts && !modality) return MOE_ERR_NULL;
  if (routing_out) {
    st = check_acts(p, routing_out);
    if (st) return st;
  }
  const WsLayout L = ws_layout(p);
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const int64_t N = p->n_tokens;
  if (N == 0) return MOE_OK;

  const hipStream_t s = S(stream);
  char* base = static_cast<char*>(ws);
  const moe_routing none{};
  const moe_routing& r = routing_out ? *routing_out : none;
  double* zpart = reinterpret_cast<double*>(base + L.logits);
  const int32_t* idx;
  const float* gw;
  if (forced_idx) {
    idx = forced_idx;
    gw = forced_w;
  } else {
    int32_t* ridx = r.topk_idx ? r.topk_idx : reinterpret_cast<int32_t*>(base + L.topk_idx);
    float* rw = r.topk_w ? r.topk_w : reinterpret_cast<float*>(base + L.topk_w);
    idx = ridx;
    gw = rw;
  }
  int32_t* counts = r.counts ? r.counts : reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = r.offsets ? r.offsets : reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* row_of = r.row_of ? r.row_of : reinterpret_cast<int32_t*>(base + L.row_of);
  int32_t* tor = r.token_of_row ? r.token_of_row : reinterpret_cast<int32_t*>(base + L.token_of_row);
  uint8_t* drop = r.drop_mask ? r.drop_mask : reinterpret_cast<uint8_t*>(base + L.drop);
  int32_t* mcounts = r.modality_counts;

  auto mark = [&](int i) {
    if (prof && prof->ev[i]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(prof->ev[i]), s);
  };
  const bool reroute = p->overflow == MOE_OVERFLOW_REROUTE;
  int32_t* alt = reinterpret_cast<int32_t*>(base + L.alt);

  const size_t esz = p->dtype == MOE_BF16 ? 2 : 4;
  FfnCall c{};
  c.dtype = p->dtype;
  c.activation = p->activation;
  c.clip = p->act_clip;
  c.N = N;
  c.d = p->d_model;
  c.I = p->d_expert;
  c.n_gather = p->n_experts;
  c.routed_rows = N * p->top_k;
  c.offsets = offsets;
  c.token_of_row = tor;
  c.n_ident = p->n_shared;
  c.identity_row0 = N * p->top_k;
  c.x = x;
  c.wg = w->w_gate; c.wu = w->w_up; c.wd = w->w_down;
  c.sg = w->ws_gate; c.su = w->ws_up; c.sd = w->ws_down;
  c.h = base + L.h;
  c.y_rows = base + L.yrows;
  c.plan = reinterpret_cast<int32_t*>(base + L.plan);
  c.save_a = r.act_a;
  c.save_u = r.act_u;
  c.sat = r.sat_count;
  if (prof) {
    for (int i = 0; i < 6; ++i) c.marks[i] = prof->ev[2 * MOE_STAGE_PLAN + i];
  }

  if (N <= kSmallTokens && !reroute) {
    // small batch: router and top-k, then dispatch and the tile plan in one launch
    mark(2 * MOE_STAGE_ROUTE);
    if (!forced_idx) {
      st = run_route(p, x, w->w_router, logit_bias, sel_bias, modality,
                     const_cast<int32_t*>(idx), const_cast<float*>(gw), zpart, r.logits, s);
      if (st) return st;
    }
    mark(2 * MOE_STAGE_ROUTE + 1);
    mark(2 * MOE_STAGE_PERMUTE);
    SmallDispatch sd{};
    sd.idx = idx;
    sd.modality = modality;
    sd.counts = counts;
    sd.mod_counts = mcounts;
    sd.offsets = offsets;
    sd.row_of = row_of;
    sd.token_of_row = tor;
    sd.final_idx = r.final_idx;
    sd.drop = drop;
    sd.C = capacity_of(p);
    sd.N = N;
    sd.E = p->n_experts;
    sd.k = p->top_k;
    sd.n_ident = p->n_shared;
    sd.ident_row0 = c.identity_row0;
    sd.BM = ffn_plan_rows(c);
    sd.plan = c.plan;
    sd.sat = r.sat_count;
    if (launch_dispatch_small(sd, s) != hipSuccess) return MOE_ERR_HIP;
    mark(2 * MOE_STAGE_PERMUTE + 1);
    c.plan_ready = 1;
  } else {
    mark(2 * MOE_STAGE_ROUTE);
    if (!forced_idx) {
      st = run_route(p, x, w->w_router, logit_bias, sel_bias, modality, const_cast<int32_t*>(idx),
                     const_cast<float*>(gw), zpart, r.logits, s, reroute ? alt : nullptr);
      if (st) return st;
    }
    mark(2 * MOE_STAGE_ROUTE + 1);
    mark(2 * MOE_STAGE_PERMUTE);
    hipError_t perr;
    if (reroute) {
      perr = launch_permute_reroute(
          idx, alt, modality, counts, mcounts, offsets, row_of, tor, drop, r.final_idx,
          reinterpret_cast<int32_t*>(base + L.lrank),
          reinterpret_cast<int32_t*>(base + L.blk_counts),
          reinterpret_cast<int32_t*>(base + L.cand), reinterpret_cast<int32_t*>(base + L.lrank2),
          reinterpret_cast<int32_t*>(base + L.blk2), reinterpret_cast<int32_t*>(base + L.kept1),
          N, p->n_experts, p->top_k, capacity_of(p), s);
    } else {
      perr = launch_permute(idx, modality, counts, mcounts, offsets, row_of, tor, drop,
                            reinterpret_cast<int32_t*>(base + L.lrank),
                            reinterpret_cast<int32_t*>(base + L.blk_counts), N, p->n_experts,
                            p->top_k, capacity_of(p), s);
      if (perr == hipSuccess && r.final_idx)
        perr = launch_final_idx(idx, row_of, r.final_idx, N * p->top_k, s);
    }
    if (perr != hipSuccess) return MOE_ERR_HIP;
    mark(2 * MOE_STAGE_PERMUTE + 1);
  }
  if (launch_ffn(c, s) != hipSuccess) return MOE_ERR_HIP;

  const void* y_shared =
      p->n_shared ? static_cast<const void*>(base + L.yrows +
                                             (size_t)N * p->top_k * p->d_model * esz)
                  : nullptr;
  mark(2 * MOE_STAGE_COMBINE);
  if (launch_combine(p->dtype, base + L.yrows, row_of, gw, y_shared, N, p->n_shared, y, N,
                     p->d_model, p->top_k, s) != hipSuccess)
    return MOE_ERR_HIP;
  mark(2 * MOE_STAGE_COMBINE + 1);
  return MOE_OK;
}

int moe_forward_ex(const moe_problem* p, const moe_weights* w, const void* x,
                   const float* logit_bias, const float* sel_bias, const uint8_t* modality,
                   void* y, const moe_routing* routing_out, const moe_profile* prof, void* ws,
                   size_t ws_bytes, void* stream) {
  return forward_impl(p, w, x, logit_bias, sel_bias, modality, y, routing_out, prof, ws,
                      ws_bytes, stream, nullptr, nullptr);
}

// The current device's copy of the scratch array, looked up once per device
// (thread-safe); NULL with *status set if the lookup fails.
static void* noalloc_scratch(int* status) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = MOE_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      *status = MOE_ERR_HIP;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

int moe_forward_noalloc(const moe_problem* p, const moe_weights* w, const void* x,
                        const float* logit_bias, const float* sel_bias,
                        const uint8_t* modality, void* y, const moe_routing* routing_out,
                        void* stream) {
  int st = validate(p);
  if (st) return st;
  if (ws_layout(p).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = noalloc_scratch(&st);
  if (!ws) return st;
  return forward_impl(p, w, x, logit_bias, sel_bias, modality, y, routing_out, nullptr, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

int moe_forward_routed(const moe_problem* p, const moe_weights* w, const void* x,
                       const int32_t* topk_idx, const float* topk_w, const uint8_t* modality,
                       void* y, const moe_routing* routing_out, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!topk_idx || !topk_w) return MOE_ERR_NULL;
  return forward_impl(p, w, x, nullptr, nullptr, modality, y, routing_out, nullptr, ws,
                      ws_bytes, stream, topk_idx, topk_w);
}

int moe_backward_workspace_size(const moe_problem* p, size_t* bytes) {
  const int st = validate(p);
  if (st) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = bwd_ws_layout(p).total;
  return MOE_OK;
}

int moe_backward(const moe_problem* p, const moe_weights* w, const void* x,
                 const moe_routing* routing, const float* dy, const moe_grads* grads,
                 void* ws, size_t ws_bytes, void* stream) {
  return moe_backward_ex(p, w, x, routing, dy, grads, nullptr, ws, ws_bytes, stream);
}

int moe_backward_ex(const moe_problem* p, const moe_weights* w, const void* x,
                    const moe_routing* routing, const float* dy, const moe_grads* grads,
                    const moe_profile* prof, void* ws, size_t ws_bytes, void* stream) {
  int st = validate(p);
  if (st) return st;
  if (!w || !x || !routing || !dy || !grads) return MOE_ERR_NULL;
  if (p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const bool swiglu = p->activation == MOE_SWIGLU;
  const bool shared = p->n_shared > 0;
  if (!w->w_router || !w->w_up || !w->w_down || (swiglu && !w->w_gate)) return MOE_ERR_NULL;
  if (shared && (!w->ws_up || !w->ws_down || (swiglu && !w->ws_gate))) return MOE_ERR_NULL;
  const moe_routing& r = *routing;
  if (!r.topk_idx || !r.topk_w || !r.logits || !r.offsets || !r.row_of || !r.token_of_row)
    return MOE_ERR_NULL;
  st = check_acts(p, &r);
  if (st) return st;
  const moe_grads& g = *grads;
  if (!g.dx || !g.dw_router || !g.dw_up || !g.dw_down || (swiglu && !g.dw_gate))
    return MOE_ERR_NULL;
  if (shared && (!g.dws_up || !g.dws_down || (swiglu && !g.dws_gate))) return MOE_ERR_NULL;
  if (g.dw_bf16 != 0 && g.dw_bf16 != 1) return MOE_ERR_INVALID;
  {
    const void* ptrs[] = {x,          w->w_router, w->w_gate,  w->w_up,   w->w_down,
                          w->ws_gate, w->ws_up,    w->ws_down, dy,        g.dx,
                          g.dw_router, g.dw_gate,  g.dw_up,    g.dw_down, g.dws_gate,
                          g.dws_up,   g.dws_down};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return MOE_ERR_UNSUPPORTED;
  }
  const BwdLayout L = bwd_ws_layout(p);
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (p->n_tokens == 0) return MOE_OK;
  BwdCall c{};
  c.N = p->n_tokens;
  c.d = p->d_model;
  c.I = p->d_expert;
  c.E = p->n_experts;
  c.k = p->top_k;
  c.S = p->n_shared;
  c.gating = p->gating;
  c.activation = p->activation;
  c.renormalize = p->renormalize;
  c.clip = p->act_clip;
  c.x = x;
  c.wr = w->w_router;
  c.wg = w->w_gate; c.wu = w->w_up; c.wd = w->w_down;
  c.sg = w->ws_gate; c.su = w->ws_up; c.sd = w->ws_down;
  c.dy = dy;
  c.logits = r.logits;
  c.topk_idx = r.topk_idx;
  c.topk_w = r.topk_w;
  c.offsets = r.offsets;
  c.row_of = r.row_of;
  c.token_of_row = r.token_of_row;
  c.act_a = static_cast<const uint16_t*>(r.act_a);
  c.act_u = static_cast<const uint16_t*>(r.act_u);
  c.dx = g.dx;
  c.dw_router = g.dw_router;
  c.dw_gate = g.dw_gate; c.dw_up = g.dw_up; c.dw_down = g.dw_down;
  c.dws_gate = g.dws_gate; c.dws_up = g.dws_up; c.dws_down = g.dws_down;
  c.dw_bf16 = g.dw_bf16;
  c.d_logit_bias = g.d_logit_bias;
  c.dz_out = g.dz;
  c.dg_out = g.dg;
  c.ws = ws;
  c.L = L;
  if (prof)
    for (int i = 0; i < 2 * MOE_NUM_BSTAGES; ++i) c.marks[i] = prof->ev[i];
  return launch_backward(c, S(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_INVALID: return "a size or option is out of range";
    case MOE_ERR_UNSUPPORTED: return "unsupported (alignment or option)";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP kernel launch failed";
    case MOE_ERR_TOO_LARGE:
      return "problem needs more than the 64 MiB fixed scratch of moe_forward_noalloc";
    default: return "unknown status";
  }
}

const char* moe_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"
