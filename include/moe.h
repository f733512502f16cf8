/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts FFN layer forward pass.
 *
 * The layer (one MoE FFN, per token t of a flattened batch x[N][d]):
 *   z_t   = x_t W_g + o                       router logits, one per expert
 *   s_t   = softmax(z_t) | sigmoid(z_t)       scores
 *   key_t = z_t + b   (softmax) | s_t + b[m_t]  (sigmoid)   selection keys
 *   T_t   = the k largest keys, descending, equal keys -> lower expert index
 *   g_tj  = s_tj / sum_{i in T_t} s_ti        renormalised gate weights (no bias)
 *   per expert e the first C tokens in token order are kept, the rest dropped
 *   y_t   = sum_{j kept} g_tj FFN_{e_tj}(x_t) + sum_s FFN_shared_s(x_t)
 *   FFN   = (silu(x W_gate) * (x W_up), clamped to +-act_clip) W_down   (SwiGLU)
 *         | max(x W1, 0) W2                                             (ReLU)
 *
 * Sources of each step (page title, section):
 *   router, softmax, top-k, renormalisation, combine:
 *       "Основы MoE" (ai.flicky.cc), section "Как устроен MoE-слой", steps 1-4;
 *   tie rule (lower index first): same page, section "Практика" (topk_route);
 *   selection bias on the choice only:
 *       "Le groupe d'experts (MoE)" (aiengineeringfromscratch.com), "Étape 1: le routeur";
 *       "Mixture-of-Experts" (mkdocs.reaper.mx, DeepSeek-V4.1-Flash), "L'équilibrage de charge";
 *   one bias set per modality: same V4.1 page, "La nouveauté de V4.1 : l'équilibrage par modalité";
 *   capacity C = ceil(N*k/E * f), token-order drops, shared expert outside the
 *   renormalisation: "Mixture-of-Experts : routage et capacité" (cours.spawnkit.ai),
 *       "L'idée — Capacité", "Cas guidé — trace complète", "L'idée — Top-k et mélange";
 *   SwiGLU with three matrices, clip at 10: V4.1 page, table "Les chiffres de
 *       DeepSeek-V4.1-Flash" and "Le compte des paramètres";
 *   two-layer ReLU expert: "Mixture of Experts" fiche (dataistudio.com), code section.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers marked (device) are HIP device pointers; (host) are host pointers.
 * - All device work is enqueued asynchronously on `stream` (a hipStream_t; NULL =
 *   the null stream).  Nothing synchronises; buffers must stay alive until the
 *   stream work completes.  The library never allocates, frees or keeps a pointer
 *   past the call; the caller owns every buffer.
 * - Inputs x and all weights are bfloat16 (raw 16-bit words) when p->dtype ==
 *   MOE_BF16 and float32 when p->dtype == MOE_F32.  Router logit offsets and
 *   selection biases are always float32; gate weights are float32.
 * - The layer output y is float32 [N][d] for both dtypes (sums are kept in
 *   float32 and not rounded to 16 bits).
 * - Expert output rows ("y_rows", between moe_expert_ffn and moe_combine) are
 *   IEEE fp16 when p->dtype == MOE_BF16 and float32 when MOE_F32.  Internally
 *   the hidden activation h is fp16 as well and the down projection runs on
 *   the fp16 matrix cores, with the bf16 W_down converted to fp16.
 * - Range of the fp16 intermediates (MOE_BF16 only).  h and the expert rows
 *   hold magnitudes up to 65504; a larger (or non-finite) value is stored as
 *   +-65504 -- the layer's result is then wrong for the tokens concerned.
 *   moe_forward counts such values in routing_out->sat_count (see moe_routing):
 *   0 means every intermediate was in range.  This happens only with very
 *   large activations (|x W_gate| |x W_up| beyond ~6.5e4 without a clip); with
 *   act_clip <= 65504, h cannot overflow.  W_down entries convert exactly
 *   when 2^-17 <= |w| <= 65504; smaller ones are truncated to multiples of
 *   2^-24 (absolute error below 6e-8) and larger ones saturate at 65504 --
 *   a property of the weights the caller can check once.
 * - Weight layout is [out][in] (each row is one output unit, contiguous along
 *   the reduction dimension): router [E][d]; gate/up [E][I][d]; down [E][d][I];
 *   shared experts [S][I][d] and [S][d][I].  For ReLU experts w_gate is NULL,
 *   w_up = W1^T and w_down = W2^T.
 * - Assignment arrays are flat [N*k] in token-major order (a = t*k + j).
 * - Return value: MOE_OK or a negative status (see moe_status_string).
 *   Validation happens on the host before any launch; a failed call enqueues
 *   nothing.  Device faults surface at the caller's next synchronisation.
 *   Capacity overflow is NOT an error: it is the drop policy.  N == 0 is a
 *   successful no-op.
 * - Calls are reentrant; overlapping calls must use distinct workspaces.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,          /* a required pointer is NULL */
  MOE_ERR_INVALID = -2,       /* a size or option is out of range */
  MOE_ERR_UNSUPPORTED = -3,   /* valid but not supported (alignment, dtype mix) */
  MOE_ERR_WORKSPACE = -4,     /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = -5,           /* a kernel launch failed (hipGetLastError) */
  MOE_ERR_TOO_LARGE = -6      /* moe_forward_noalloc: the problem needs more than
                                 MOE_NOALLOC_SCRATCH_BYTES of scratch */
};

typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_gating;
typedef enum { MOE_SWIGLU = 0, MOE_RELU = 1 } moe_activation;
typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

/* The problem: the arguments of the layer.  Passed by pointer, read only. */
typedef struct {
  int64_t n_tokens;        /* N >= 0 tokens (rows of x) */
  int32_t d_model;         /* d >= 1; multiple of 8 for MOE_BF16 */
  int32_t n_experts;       /* E routed experts, 1..1024 */
  int32_t top_k;           /* k experts per token, 1..min(E, 32) */
  int32_t d_expert;        /* I expert inner size; multiple of 8 for MOE_BF16 */
  int32_t n_shared;        /* S >= 0 always-on shared experts (inner size I), <= 8 */
  int32_t gating;          /* moe_gating */
  int32_t activation;      /* moe_activation */
  int32_t dtype;           /* moe_dtype of x and the weights */
  int32_t n_bias_sets;     /* 0: no selection bias; 1: bias[E]; 2: bias[2][E] by modality */
  int32_t renormalize;     /* 1: gate weights renormalised over the k chosen;
                              0: the chosen scores as they are (softmax p_i over all
                              E, or the sigmoid score) -- Switch top-1 style */
  float act_clip;          /* > 0: clamp silu(a)*u to [-act_clip, act_clip]; 0: none */
  double capacity_factor;  /* f > 0: C = ceil(N*k/E * f) (exact); <= 0: unlimited */
  int32_t overflow;        /* MOE_OVERFLOW_DROP (0) or MOE_OVERFLOW_REROUTE (1) */
} moe_problem;

/* What happens to an assignment past its expert's capacity (routing slides,
 * table "Politiques de débordement"): DROP -- it adds nothing (row "Abandon");
 * REROUTE -- the q-th dropped slot of a token is offered to the token's
 * (k+1+q)-th best expert (row "Report sur E2/E3"), which accepts offers in
 * token order while it has room left after its own first-choice rows; an
 * accepted slot keeps its gate weight, a refused one is dropped.  REROUTE
 * runs in moe_forward / moe_forward_ex (moe_permute and moe_forward_routed
 * return MOE_ERR_UNSUPPORTED for it: they have no alternate experts). */
enum { MOE_OVERFLOW_DROP = 0, MOE_OVERFLOW_REROUTE = 1 };

/* Expert weights (device).  Routed experts are required; shared ones when S > 0. */
typedef struct {
  const void* w_router;    /* [E][d] */
  const void* w_gate;      /* [E][I][d]; NULL for MOE_RELU */
  const void* w_up;        /* [E][I][d] */
  const void* w_down;      /* [E][d][I] */
  const void* ws_gate;     /* [S][I][d]; NULL for MOE_RELU or S == 0 */
  const void* ws_up;       /* [S][I][d]; NULL when S == 0 */
  const void* ws_down;     /* [S][d][I]; NULL when S == 0 */
} moe_weights;

/* Optional routing outputs of moe_forward (device pointers, each may be NULL). */
typedef struct {
  int32_t* topk_idx;         /* [N*k] */
  float* topk_w;             /* [N*k] */
  int32_t* counts;           /* [E]   demand per expert (before capacity) */
  int32_t* modality_counts;  /* [2][E] demand per modality (n_bias_sets == 2 only) */
  int32_t* offsets;          /* [E+1] prefix sums of kept counts */
  int32_t* row_of;           /* [N*k] slot row, -1 if dropped */
  int32_t* token_of_row;     /* [N*k] valid in [0, offsets[E]) */
  uint8_t* drop_mask;        /* [N*k] 1 if dropped */
  double* logits;            /* [N][E] router logits z (float64) */
  int32_t* final_idx;        /* [N*k] expert that processes each slot (the rerouted
                                one under MOE_OVERFLOW_REROUTE), -1 if dropped */
  /* Pre-activations of the expert FFNs, for moe_backward (MOE_BF16 only; both
   * or neither for SwiGLU, act_u alone for ReLU): IEEE fp16 [N*k + N*S][I],
   * 16-byte aligned, in the layer's row layout (routed rows [0, offsets[E]),
   * then N rows per shared expert from row N*k).  act_a = x W_gate^T,
   * act_u = x W_up^T (SwiGLU) or x W1 before the ReLU.  Written by moe_forward /
   * moe_forward_ex / moe_forward_routed when given; read by moe_backward, which
   * then skips recomputing them. */
  void* act_a;
  void* act_u;
  /* Range status of the fp16 intermediates (device, nullable) int32 [1] out:
   * set to 0 at the start of the expert stage, then the number of hidden (h)
   * and expert-row elements stored as +-65504, fp16's largest magnitude: every
   * element that exceeded the range (|v| > 65504 or not finite) and was
   * saturated, plus any in-range one that rounds there (65488 < |v| <= 65504).
   * Non-zero means y may be wrong for some tokens; the caller may rerun in
   * MOE_F32 or rescale x.  Always 0 for MOE_F32. */
  int32_t* sat_count;
} moe_routing;

/* Bytes of device workspace any call below needs for problem p (host): the
 * router's float64 logits, the routing arrays of steps 1-3 of "Как устроен
 * MoE-слой" ("Основы MoE"), the dispatch arrays of the routing slides' trace
 * ("Cas guidé — trace complète"), and the hidden activations and expert output
 * rows of every kept assignment and shared-expert row (steps 3-4). */
int moe_workspace_size(const moe_problem* p, size_t* bytes);

/* Capacity C = ceil(f * N * k / E) computed exactly on the binary value of f;
 * C >= 1 when f > 0; *C = -1 when unlimited (host).  Routing and capacity
 * slides: "L'idée — Capacité". */
int moe_capacity(const moe_problem* p, int64_t* C);

/* Parameter counts of one layer (host): expert_total = (E+S)*m*d*I and
 * expert_active = (k+S)*m*d*I with m = 3 (SwiGLU) or 2 (ReLU); router = d*E.
 * "Основы MoE", section "Всего параметров и активных параметров". */
int moe_param_counts(const moe_problem* p, int64_t* expert_total,
                     int64_t* expert_active, int64_t* router);

/* Router + scoring + top-k + gate weights (steps 1-3 of "Как устроен MoE-слой").
 *   x         (device) [N][d]
 *   w_router  (device) [E][d]
 *   logit_bias(device, nullable) float32 [E]: added to the logits; moves both
 *             the choice and the weights.
 *   sel_bias  (device, nullable unless n_bias_sets > 0) float32 [n_bias_sets][E]:
 *             moves only the choice.
 *   modality  (device) uint8 [N], 0 = text, 1 = image; required iff n_bias_sets == 2.
 *   topk_idx  (device) int32 [N*k] out: descending key order, ties -> lower index.
 *   topk_w    (device) float32 [N*k] out: renormalised unbiased scores, sum 1.
 *   logits    (device, nullable) float64 [N][E] out: z.
 * Logits are accumulated with float64 folding of short matrix-core partials,
 * so the chosen set is the float64 one except for keys closer than ~1e-7 of
 * their scale. */
int moe_route(const moe_problem* p, const void* x, const void* w_router,
              const float* logit_bias, const float* sel_bias, const uint8_t* modality,
              int32_t* topk_idx, float* topk_w, double* logits,
              void* ws, size_t ws_bytes, void* stream);

/* Histogram, capacity and token-order permutation (routing slides, "Cas guidé
 * — trace complète").  Deterministic: ranks follow token order.
 *   topk_idx        (device) int32 [N*k] in
 *   modality        (device, nullable) uint8 [N]; with modality_counts
 *   counts          (device) int32 [E] out: demand per expert
 *   modality_counts (device, nullable) int32 [2][E] out
 *   offsets         (device) int32 [E+1] out: exclusive prefix sums of min(count, C)
 *   row_of          (device) int32 [N*k] out: offsets[e] + rank, or -1 if dropped
 *   token_of_row    (device) int32 [N*k] out: token of each kept row, [0, offsets[E])
 *   drop_mask       (device) uint8 [N*k] out */
int moe_permute(const moe_problem* p, const int32_t* topk_idx, const uint8_t* modality,
                int32_t* counts, int32_t* modality_counts, int32_t* offsets,
                int32_t* row_of, int32_t* token_of_row, uint8_t* drop_mask,
                void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs over grouped rows: step 3 of "Как устроен MoE-слой" ("Основы
 * MoE": each chosen expert runs on its tokens), with the SwiGLU expert of three
 * matrices and the clip of the V4.1 page ("Mixture-of-Experts", table "Les
 * chiffres de DeepSeek-V4.1-Flash" and "Le compte des paramètres") or the
 * two-layer ReLU expert of the "Mixture of Experts" fiche (code section); the
 * shared expert ("Mixture-of-Experts : routage et capacité", "L'idée — Top-k et
 * mélange") is the dense mode.
 * Routed mode (token_of_row != NULL): for each expert e, rows
 *   [offsets[e], offsets[e+1]) take x[token_of_row[row]] and y_rows[row] =
 *   FFN_e(x[token]).  Weights are the routed [E][..] tensors.
 * Dense mode (token_of_row == NULL, offsets == NULL): one expert (w_gate [I][d],
 *   w_up [I][d], w_down [d][I]) over all N rows: y_rows[t] = FFN(x[t]) -- the
 *   shared expert.
 *   y_rows (device) [N*k][d] (routed) or [N][d] (dense), row format (fp16 for
 *          MOE_BF16, float32 for MOE_F32). */
int moe_expert_ffn(const moe_problem* p, const void* x, const int32_t* token_of_row,
                   const int32_t* offsets, const void* w_gate, const void* w_up,
                   const void* w_down, void* y_rows, void* ws, size_t ws_bytes,
                   void* stream);

/* Gate-weighted combine and un-permute ("Как устроен MoE-слой", step 4):
 *   y[t] = sum_{j: row_of[t*k+j] >= 0} topk_w[t*k+j] * y_rows[row_of[t*k+j]]
 *          + sum_s y_shared[s][t]
 * summed in float32 in that fixed order.  Dropped slots add nothing and the
 * other weights are not renormalised.
 *   y_rows   (device) [*][d] row format; row_of, topk_w (device) [N*k];
 *   y_shared (device, nullable) [S][N][d] row format; y (device) float32 [N][d] out. */
int moe_combine(const moe_problem* p, const void* y_rows, const int32_t* row_of,
                const float* topk_w, const void* y_shared, void* y, void* stream);

/* The whole layer ("Основы MoE", "Как устроен MoE-слой", steps 1-4, with the
 * capacity and drop rule of "Mixture-of-Experts : routage et capacité", "L'idée
 * — Capacité" and "Cas guidé — trace complète", and the shared expert of its
 * "L'idée — Top-k et mélange"): route, permute, routed + shared experts,
 * combine; y is float32 [N][d].  Equal to the staged calls.  routing_out (host
 * struct of device pointers, nullable) receives the intermediate routing
 * arrays for verification and the range status of the fp16 intermediates. */
int moe_forward(const moe_problem* p, const moe_weights* w, const void* x,
                const float* logit_bias, const float* sel_bias, const uint8_t* modality,
                void* y, const moe_routing* routing_out, void* ws, size_t ws_bytes,
                void* stream);

/* Routing replay: the layer with a routing the caller supplies instead of the
 * router's (permute, routed + shared experts, combine; the MoE basics page,
 * "Как устроен MoE-слой", step 4, with the dispatch of the routing slides).
 *   topk_idx (device) int32 [N*k]: expert of each assignment.  Each row should
 *            hold distinct experts; an index outside [0, E) is an assignment to
 *            no expert (not counted, marked dropped, contributes nothing).
 *   topk_w   (device) float32 [N*k]: gate weights, used as given.
 *   modality (device, nullable) uint8 [N]: only for routing_out->modality_counts.
 * w->w_router, logit and selection biases are not used.  routing_out (nullable)
 * receives counts, offsets, row and token maps, drops (its topk_idx, topk_w and
 * logits are not written).  Capacity applies as in moe_forward.  With the
 * indices and weights moe_forward produced, y equals its output bit for bit. */
int moe_forward_routed(const moe_problem* p, const moe_weights* w, const void* x,
                       const int32_t* topk_idx, const float* topk_w, const uint8_t* modality,
                       void* y, const moe_routing* routing_out, void* ws, size_t ws_bytes,
                       void* stream);

/* A router without parameters (the expert-group lesson's hash-router
 * exercise, "Exercices", Medium): h = splitmix64(token_ids[t]) (S. Vigna's
 * 64-bit mixer), experts h mod E, h mod E + 1, ... (mod E), weights 1/k.  Feed
 * the result to moe_forward_routed.
 *   token_ids (device) int64 [N]; topk_idx (device) int32 [N*k] out;
 *   topk_w (device) float32 [N*k] out. */
int moe_route_hash(const moe_problem* p, const int64_t* token_ids, int32_t* topk_idx,
                   float* topk_w, void* stream);

/* Bytes of the fixed device scratch of moe_forward_noalloc: the most
 * workspace (moe_workspace_size) a problem may need to run through it. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same layer, the same kernels and the same results, with no workspace
 * argument and no allocation of any kind.  Its scratch is a file-scope device
 * array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) in the library, one copy per GPU
 * the library runs on, held until the process ends; the first call on a
 * device looks up that device's copy.  Problems whose moe_workspace_size
 * exceeds it return MOE_ERR_TOO_LARGE before anything is enqueued (64 MiB
 * holds decode batches and prefills of a few hundred tokens at the named
 * shapes).  Every call on one GPU shares that GPU's scratch, and its contents
 * stay from the last call: calls that overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  Arguments
 * and results as for moe_forward. */
int moe_forward_noalloc(const moe_problem* p, const moe_weights* w, const void* x,
                        const float* logit_bias, const float* sel_bias,
                        const uint8_t* modality, void* y, const moe_routing* routing_out,
                        void* stream);

/* Stages of moe_forward, in launch order (indices into moe_profile.ev). */
enum {
  MOE_STAGE_ROUTE = 0,      /* router GEMM + top-k */
  MOE_STAGE_PERMUTE = 1,    /* rank, scan, scatter */
  MOE_STAGE_PLAN = 2,       /* grouped-GEMM tile plan */
  MOE_STAGE_GATE_UP = 3,    /* gate/up grouped GEMM + activation */
  MOE_STAGE_DOWN = 4,       /* down grouped GEMM */
  MOE_STAGE_COMBINE = 5,    /* weighted combine + un-permute */
  MOE_NUM_STAGES = 6
};

/* Measurement hook: hipEvent_t handles recorded on the stream immediately
 * before (ev[2*i]) and after (ev[2*i+1]) stage i; NULL entries are skipped.
 * The caller creates, owns and reads the events. */
typedef struct {
  void* ev[2 * MOE_NUM_STAGES];
} moe_profile;

/* moe_forward with an optional measurement hook (prof may be NULL; then it is
 * exactly moe_forward).  Recording events adds stream markers between the
 * stages and nothing else. */
int moe_forward_ex(const moe_problem* p, const moe_weights* w, const void* x,
                   const float* logit_bias, const float* sel_bias, const uint8_t* modality,
                   void* y, const moe_routing* routing_out, const moe_profile* prof,
                   void* ws, size_t ws_bytes, void* stream);

/* Load-balancing statistics of one routed batch and the aux-loss-free bias
 * update (training-time companion of the forward pass).
 * Statistics (MoE basics page, "Вспомогательный лосс Switch Transformer"):
 *   load[e]      = counts[e] / (N k)                 share of assignments
 *   mean_prob[e] = mean over tokens of p_te          softmax of the logits;
 *                  for sigmoid gating the token's sigmoid scores divided by
 *                  their sum
 *   aux[0]       = E * sum_e load[e] * mean_prob[e]  1 when uniform, E on collapse
 * (all float64; with N == 0 every statistic is 0).
 * Update (expert-group lesson, "Le problème de l'équilibre de la charge";
 * DeepSeek-V4.1 page, "L'équilibrage de charge" and its per-modality
 * section): for each bias set m, with c = counts (one set) or
 * modality_counts[m] (two sets) and T_m = sum_e c[e],
 *   sel_bias[m][e] -= gamma * sign(c[e] * E - T_m)
 * in float32, the sign decided exactly in integers; on-target experts keep
 * their bias.
 *   logits          (device) float64 [N][E]: z as moe_route writes it
 *                   (needed for mean_prob / aux)
 *   counts          (device) int32 [E]: demand per expert, as moe_permute
 *                   writes it (needed for load / aux / one-set update)
 *   modality_counts (device) int32 [2][E] (needed for a two-set update)
 *   load, mean_prob (device, nullable) float64 [E] out; aux (device, nullable)
 *                   float64 [1] out
 *   sel_bias        (device, nullable) float32 [n_bias_sets][E], updated in
 *                   place; NULL = no update.  n_bias_sets == 0 with a
 *                   non-NULL sel_bias is MOE_ERR_INVALID.
 *   gamma           update rate, finite and >= 0 (else MOE_ERR_INVALID)
 *   ws, ws_bytes    device workspace (moe_workspace_size is enough); only
 *                   used for mean_prob / aux.
 * Results are deterministic (fixed reduction order). */
int moe_balance(const moe_problem* p, const double* logits, const int32_t* counts,
                const int32_t* modality_counts, double* load, double* mean_prob,
                double* aux, float* sel_bias, float gamma, void* ws, size_t ws_bytes,
                void* stream);

/* Gradients written by moe_backward (device pointers, same layouts as the
 * weights they belong to).  Weight gradients (dw_*, dws_*) are float32, or
 * bf16 (raw 16-bit words, round to nearest even) when dw_bf16 = 1; dx, the
 * logit-offset gradient, dz and dg are float32. */
typedef struct {
  float* dx;            /* [N][d] required */
  void* dw_router;      /* [E][d] required */
  void* dw_gate;        /* [E][I][d] required for MOE_SWIGLU, unused for MOE_RELU */
  void* dw_up;          /* [E][I][d] required */
  void* dw_down;        /* [E][d][I] required */
  void* dws_gate;       /* [S][I][d] required when S > 0 and MOE_SWIGLU */
  void* dws_up;         /* [S][I][d] required when S > 0 */
  void* dws_down;       /* [S][d][I] required when S > 0 */
  float* d_logit_bias;  /* [E] nullable: gradient of the logit offset o (= sum_t dz_t) */
  float* dz;            /* [N][E] nullable: gradient of the logits */
  float* dg;            /* [N*k] nullable: gradient of the gate weights (0 for dropped slots) */
  int32_t dw_bf16;      /* 0: weight gradients float32; 1: bf16 (half the bytes written,
                           which bound the weight-gradient products of small experts) */
} moe_grads;

/* Bytes of device workspace moe_backward needs for problem p (host). */
int moe_backward_workspace_size(const moe_problem* p, size_t* bytes);

/* Backward pass of the layer: the gradients of L = sum(dy * y) for the routing
 * a moe_forward call decided, with that routing held fixed (top-k, capacity and
 * reroute are piecewise constant in the logits, so the router receives its
 * gradient through the gate weights alone -- why the MoE basics page,
 * "Основы MoE", section "Как устроен MoE-слой", keeps p_i as the Switch top-1
 * weight instead of 1).  Chain rule through each step of the forward:
 *   per kept row (token t, weight g) and shared row (g = 1) of expert FFN f:
 *     dW_down += (g dy_t)^T h, dh = g dy_t W_down (0 where the clamp is active),
 *     SwiGLU: da = dh u silu'(a), du = dh silu(a); ReLU: du = dh [u > 0],
 *     dW_gate += da^T x_t, dW_up += du^T x_t, dx_t += da W_gate + du W_up,
 *     dg = <dy_t, f(x_t)>;
 *   gate weights -> logits (softmax renormalised over the chosen, raw softmax
 *   p, sigmoid renormalised or raw): dz; dW_router = dz^T x, dx += dz W_router,
 *   d_logit_bias = sum_t dz_t.  Dropped slots get dg = 0 but still move dz
 *   through the renormalisation.
 * MOE_BF16 only (MOE_F32 returns MOE_ERR_UNSUPPORTED).  The products run on
 * the bf16 matrix cores with float32 accumulation: dy and the per-row
 * gradients (g h, da, du, dz) are rounded to bf16 as operands.
 *   x        (device) bf16 [N][d], the forward's input
 *   w        the forward's weights (w_router required)
 *   routing  (host struct of device pointers) from the moe_forward call:
 *            topk_idx, topk_w, logits, offsets, row_of, token_of_row required
 *            (moe_forward writes them when they are given in routing_out);
 *            act_a / act_u optional: the forward's saved pre-activations, used
 *            instead of recomputing x W_gate^T and x W_up^T
 *   dy       (device) float32 [N][d], gradient of the output y
 *   grads    (host struct of device pointers) outputs, overwritten
 *   ws       (device) moe_backward_workspace_size() bytes
 * dy, dx, x and the weights must be 16-byte aligned.  Results are
 * deterministic (fixed reduction orders, no atomics). */
int moe_backward(const moe_problem* p, const moe_weights* w, const void* x,
                 const moe_routing* routing, const float* dy, const moe_grads* grads,
                 void* ws, size_t ws_bytes, void* stream);

/* Stages of moe_backward, in launch order (indices into moe_profile.ev, as
 * for the forward's stages). */
enum {
  MOE_BSTAGE_PREP = 0,       /* tile plans, routed rows of x and dy gathered */
  MOE_BSTAGE_RECOMPUTE = 1,  /* a = x W_gate^T, u = x W_up^T per row */
  MOE_BSTAGE_DH = 2,         /* dy W_down per row */
  MOE_BSTAGE_ROWS = 3,       /* per-row activation gradients and dg */
  MOE_BSTAGE_WGRAD = 4,      /* dW_down, dW_gate, dW_up grouped GEMMs */
  MOE_BSTAGE_DX = 5,         /* per-row dx, router gradients, dx combine */
  MOE_NUM_BSTAGES = 6
};

/* moe_backward with an optional measurement hook (prof may be NULL; then it is
 * exactly moe_backward).  ev[2*i] and ev[2*i+1] bracket backward stage i. */
int moe_backward_ex(const moe_problem* p, const moe_weights* w, const void* x,
                    const moe_routing* routing, const float* dy, const moe_grads* grads,
                    const moe_profile* prof, void* ws, size_t ws_bytes, void* stream);

/* Text of a status code (static storage). */
const char* moe_status_string(int status);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
