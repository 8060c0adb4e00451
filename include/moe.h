/*
 * moe.h -- C ABI of a mixture-of-experts layer for AMD Instinct MI355X
 * (gfx950): the token-choice forward pass below, and beside it dropless and
 * score-priority capacity, expert-choice routing, the balancing variants and
 * the backward pass (each documented at its entry point).
 *
 * The layer (page titles and sections of the sources it follows):
 *   "Lab 18 -- Mixture of experts" s.1 (layer equation, gate values),
 *   s.2 (load balancing, router z-loss), s.3 (capacity and dropped tokens),
 *   "What to implement"; "Lab 01 -- Router, Load Balancing, Capacity & the
 *   MoE Layer" ("Where to start", "The traps"); "Mixture of Experts --
 *   parameters without the FLOPs" s.2 (the router) and s.3 (capacity);
 *   "Mixture of experts" lecture field map (fp32 router, DeepSeek-V3 sigmoid
 *   affinities and selection bias).
 *
 *   z   = x W_r + logit_bias                      float32, [T,E]
 *   key = z (+ select_bias)          (softmax scores)
 *       = fp32 sigmoid(z) + select_bias  (sigmoid scores)
 *   idx = the k largest keys per token, best first, equal keys to the lower
 *         expert index (-0 equals +0)
 *   g   = softmax over the selected logits (renormalised), or the full
 *         softmax probability (raw, the k = 1 default), or the selected
 *         sigmoid scores normalised over the k (sigmoid)
 *   C   = ceil(cf * T * k / E), or capacity_override when > 0
 *   slot= queue position of (token, choice) in its expert, in priority order
 *         (rank-major: every first choice, then every second choice, token
 *         order inside a rank; or token-major); dropped iff slot >= C
 *   y_t = sum over kept choices of g * FFN_e(x_t)  (+ shared experts);
 *         a token with no kept choice and no shared expert gets y_t = x_t
 *         (or 0 when dropped_output = 1)
 *   L_aux = E * sum_i f_i P_i, f_i = (choices routed to i) / (T k),
 *         P_i = mean full router probability of i;   L_z = mean_t LSE_t^2.
 *         Both are returned without their alpha coefficients.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked [host]. Tensors are dense,
 *     row-major, and at least 16-byte aligned (expert biases included: the
 *     expert GEMMs read them 8 bytes at a time; validation refuses others).
 *   - Storage type of x, expert weights, expert biases and y: MOE_F32 or
 *     MOE_BF16 (raw bf16 bits). The router weight, biases of the router,
 *     logits, probabilities, gates and losses are always float32.
 *   - Expert weights follow the [out_features, in_features] layout:
 *     w_in/w_gate/w_up [E, F, d], w_out [E, d, F], b_in [E, F], b_out [E, d].
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; nothing blocks the host, nothing is copied to
 *     the host, and no device memory is allocated or freed. Results are valid
 *     once the stream has been synchronised.
 *   - The caller owns every buffer, including the workspace `ws` of
 *     moe_workspace_bytes() bytes (256-byte aligned).
 *   - Errors: inputs are validated on the host before anything is launched.
 *     MOE_EINVAL for a bad configuration or argument (capacity_factor < 1,
 *     k < 1, k > E, k > 32, E > 256, T*k >= 2^31, d or F not a multiple of 8,
 *     a required pointer NULL or misaligned); MOE_EUNSUPPORTED for a
 *     combination that is not built; MOE_EHIP when a launch fails.
 *     moe_last_error() returns a message for the calling thread's last
 *     non-OK status.
 *   - Same inputs on the same GPU give bit-identical outputs (no result
 *     depends on the order of atomic operations).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_OK = 0, MOE_EINVAL = 1, MOE_EUNSUPPORTED = 2, MOE_EHIP = 3 } moe_status;
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score;
typedef enum { MOE_GELU = 0, MOE_SWIGLU = 1 } moe_act;
typedef enum { MOE_RANK_MAJOR = 0, MOE_TOKEN_MAJOR = 1, MOE_SCORE_PRIORITY = 2 } moe_priority;
typedef enum { MOE_TOKEN_CHOICE = 0, MOE_EXPERT_CHOICE = 1 } moe_routing;

typedef struct moe_config {
  int64_t T;                  /* tokens (B*S flattened by the caller)                 */
  int32_t d;                  /* model width                                           */
  int32_t E;                  /* routed experts, 1..256                                */
  int32_t k;                  /* experts per token, 1..min(E,32)                       */
  int32_t d_ff;               /* routed expert hidden width F                          */
  int32_t n_shared;           /* shared experts (GELU MLPs), 0 = none                  */
  int32_t d_ff_shared;        /* hidden width of ONE shared expert                     */
  double capacity_factor;     /* >= 1.0, else MOE_EINVAL                               */
  int64_t capacity_override;  /* > 0: use as the capacity C; 0: ceil(cf*T*k/E)         */
  int32_t renormalize;        /* -1: renormalise iff k > 1; 0: raw gates; 1: renorm.   */
  int32_t score;              /* moe_score                                             */
  int32_t act;                /* moe_act of the routed experts                         */
  int32_t dtype;              /* moe_dtype of x, expert weights/biases, y              */
  int32_t priority;           /* moe_priority of the capacity queue                    */
  int32_t dropped_output;     /* 0: fully dropped token -> y = x; 1: y = 0             */
  int32_t dropless;           /* 0: capacity C as above; 1: dropless (see below)       */
  int32_t routing;            /* moe_routing: token choice (above) or expert choice    */
  int32_t save_preact;        /* 1: moe_forward also keeps the expert pre-activations in
                                 its workspace, so moe_backward need not recompute them
                                 (bf16 only)                                          */
} moe_config;

/* Score priority (priority = MOE_SCORE_PRIORITY) ["Lab 18" s.3: who is
 * dropped depends on the priority; V-MoE's batch-prioritised routing ranks
 * assignments by router score]:
 *   - each expert keeps the C assignments with the largest gate (float32, as
 *     moe_route stores it), equal gates to the assignment earlier in the
 *     rank-major queue;
 *   - kept assignments take slots 0.. in rank-major queue order, dropped ones
 *     C.. in the same order (so dropped iff slot >= C still holds);
 *   - the standalone dispatch is moe_dispatch_by_score (moe_dispatch returns
 *     MOE_EINVAL); in dropless mode nothing drops and the rows are numbered
 *     as under rank-major priority. */

/* Dropless mode (dropless = 1) ["Lab 18" s.3, alternatives to dropping: a
 * capacity high enough that nothing is dropped, or block-sparse kernels that
 * remove the limit; "Mixture of experts" lecture, systems section: ragged
 * per-expert matmuls without padding or dropping]:
 *   - capacity_factor and capacity_override are ignored; moe_validate reports
 *     C = T (no expert can receive more than T choices) and no choice is
 *     dropped (dropped[] is all 0, the loss statistics count no drops);
 *   - the choices of expert e occupy the rows [off_e, off_e + counts[e]) of
 *     packed [T*k, ...] buffers, off_e = counts[0] + ... + counts[e-1], in the
 *     same priority order as the capacity queue, with no padding;
 *   - slot[t,j] is that packed ROW (not the position inside the expert);
 *     row_token is [T*k], xe, h and ye are [T*k, ...];
 *   - moe_combine reads ye[slot[t,j]]. */

/* Expert-choice routing (routing = MOE_EXPERT_CHOICE) ["Lab 18" exercise 1
 * and "Common extensions": selection per expert over the tokens, which
 * evens the load by construction and drops nothing, while a token can get
 * several experts or none; "Mixture of experts" lecture, routing families:
 * selection along the expert axis of the token x expert score matrix]:
 *   - C is computed as above (k is then the mean number of experts a token
 *     gets) and every expert takes n = min(C, T) tokens: those with the
 *     largest float32 probability probs[t,e], equal values to the lower
 *     token, held in its rows in token order (row_token [E,C], rows >= n
 *     unused);
 *   - sel[t,e] is token t's row inside expert e, or -1;
 *   - y_t = sum over the experts e that picked t, in e order, of
 *     probs[t,e] * FFN_e(x_t) (+ shared experts); a token no expert picked
 *     gets x_t (or 0, dropped_output = 1) when there is no shared expert;
 *   - L_aux = E * sum_i f_i P_i with f_i = counts_i / sum_j counts_j (1/E);
 *     stats = {E*n picks, 0 dropped, unpicked tokens, E*(C - n) pad slots};
 *   - dropless must be 0 (MOE_EINVAL otherwise). */

/* Check a configuration; on MOE_OK store the capacity C in *capacity [host]
 * (may be NULL). Runs on the host only. ["Lab 18" s.3; "Lab 01" traps] */
MOE_API moe_status moe_validate(const moe_config* cfg, int64_t* capacity);

/* Bytes of workspace moe_forward needs for cfg (0 if cfg is invalid).
 * moe_route, moe_dispatch and moe_aux_losses need at most this much. */
MOE_API size_t moe_workspace_bytes(const moe_config* cfg);

/* Router: logits, probabilities, top-k and gates ["Lab 18" s.1 and "What to
 * implement" 1; "Parameters without the FLOPs" s.2].
 *   x           [T,d] storage type; NULL => `logits` is an INPUT [T,E]
 *   w_router    [d,E] float32 (ignored when x is NULL)
 *   logit_bias  [E] float32 added to the logits, or NULL
 *   select_bias [E] float32 added to the selection key only, or NULL
 *   logits      [T,E] float32: output when x != NULL (may then be NULL)
 *   probs       [T,E] float32 full softmax (or sigmoid scores normalised over
 *               all E), or NULL
 *   idx         [T,k] int32 selected experts, best first          (required)
 *   gates       [T,k] float32 gate of each selected expert        (required)
 *   lse         [T] float32 log-sum-exp of the logits, or NULL
 *   ws          workspace: required when x is bf16 (it holds the router
 *               weight split into three bf16 planes for the matrix cores and
 *               the float32 logits before the epilogue); otherwise may be
 *               NULL (then no loss partials are kept) */
MOE_API moe_status moe_route(const moe_config* cfg, const void* x, const float* w_router,
                     const float* logit_bias, const float* select_bias, float* logits,
                     float* probs, int32_t* idx, float* gates, float* lse, void* ws,
                     void* stream);

/* Capacity and dispatch ["Lab 18" s.3 GShard priority and Tips; "Lab 01"
 * "Where to start" 4; "Parameters without the FLOPs" s.3 static shapes].
 *   x          [T,d] storage type, or NULL (slots only)
 *   idx        [T,k] int32 expert ids (each row distinct, 0..E-1)
 *   slot       [T,k] int32 queue position of each choice
 *   dropped    [T,k] uint8 1 iff slot >= C
 *   counts     [E] int32 choices routed to each expert (before capacity)
 *   row_token  [E,C] int32 token held by each kept slot (rows >= kept_e of
 *              expert e are left untouched), or NULL
 *   xe         [E,C,d] storage type: xe[e,slot] = x[t] for every kept choice
 *              (rows >= kept_e untouched), or NULL
 *   (dropless mode: slot is the packed row, row_token [T*k], xe [T*k,d];
 *   see moe_config)
 *   ws         workspace (required) */
MOE_API moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* idx, int32_t* slot,
                        uint8_t* dropped, int32_t* counts, int32_t* row_token, void* xe,
                        void* ws, void* stream);

/* moe_dispatch without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as moe_dispatch, minus ws.
 * Its scratch (the capacity histograms, k*ceil(T/64)*E int32, plus E and
 * ceil(T/64) int32, 256-byte aligned pieces) lives in a fixed 16 MiB device
 * array inside the library, one per GPU, held until the process ends; a
 * configuration needing more returns MOE_EINVAL before any launch.  Nothing
 * in the scratch needs to start at zero.  Calls that overlap on one GPU (two
 * streams, or two threads) race on that array: serialise them.  The first
 * call on a device looks the array's address up (MOE_EHIP if that fails);
 * no call allocates or frees memory. */
MOE_API moe_status moe_dispatch_noalloc(const moe_config* cfg, const void* x, const int32_t* idx, int32_t* slot,
                                        uint8_t* dropped, int32_t* counts, int32_t* row_token, void* xe,
                                        void* stream);

/* Capacity and dispatch under score priority (cfg->priority must be
 * MOE_SCORE_PRIORITY, token choice; see above): as moe_dispatch, plus
 *   gates   [T,k] float32 score of each choice (moe_route's gates)
 * row_token is required when xe is given. */
MOE_API moe_status moe_dispatch_by_score(const moe_config* cfg, const void* x, const int32_t* idx, const float* gates,
                                         int32_t* slot, uint8_t* dropped, int32_t* counts, int32_t* row_token,
                                         void* xe, void* ws, void* stream);

/* Grouped expert FFN on bf16 MFMA (float32 FMA for MOE_F32)
 * ["Lab 18" s.1 experts, Tips (one grouped matrix multiply over all
 * experts); "Mixture of experts" lecture, expert geometry].
 *   groups          number of experts in this call
 *   rows_per_group  row stride between groups in h and out (and in a when
 *                   not gathered): C for dispatched buffers, T for shared
 *                   experts with groups = 1
 *   rows            [groups] int32 rows to compute in each group (e.g. the
 *                   counts of moe_dispatch; clamped to rows_per_group), or
 *                   NULL for all rows_per_group rows
 *   a               the input rows, storage type: [groups*rows_per_group, d],
 *                   or, with `gather`, the whole [a_rows, d] token matrix
 *   gather          [groups*rows_per_group] int32 or NULL: row m of group g
 *                   is a[gather[g*rows_per_group + m]] (e.g. the row_token
 *                   of moe_dispatch), read straight into the GEMM tiles so
 *                   no dispatched copy of x is needed (this is how
 *                   moe_forward dispatches); entries at or past rows[g] are
 *                   not read.  NULL gives the plain form on dispatched rows.
 *   a_rows          rows of a when gathered (ignored otherwise; bounds the
 *                   gathered reads)
 *   act             moe_act: GELU  h = GELU(a w_in^T + b_in), out = h w_out^T + b_out
 *                            SwiGLU h = SiLU(a w_gate^T) * (a w_in^T), out = h w_out^T
 *                   (an argument rather than cfg->act, so that one config drives
 *                   both the routed experts, whose act is cfg->act, and the
 *                   shared experts, which are GELU MLPs)
 *   w_in            [groups,F,d] (GELU: w_in; SwiGLU: the up projection)
 *   w_gate          [groups,F,d] SwiGLU gate projection, NULL for GELU
 *   b_in            [groups,F] or NULL;   w_out [groups,d,F];  b_out [groups,d] or NULL
 *   h               [groups*rows_per_group, F] hidden activations (storage type)
 *   out             [groups*rows_per_group, d] expert outputs (storage type)
 * Rows at or beyond rows[g] are neither read nor written.  Every operand one
 * launch addresses must hold < 2^30 elements per group (MOE_EINVAL). */
MOE_API moe_status moe_expert_ffn(const moe_config* cfg, int32_t act, int32_t groups,
                                  int64_t rows_per_group, const int32_t* rows, const void* a,
                                  const int32_t* gather, int64_t a_rows, const void* w_in,
                                  const void* w_gate, const void* b_in, const void* w_out,
                                  const void* b_out, int32_t F, void* h, void* out, void* stream);

/* The grouped expert FFN on packed rows (dropless mode): group g's rows are
 * rows [off_g, off_g + rows[g]) of a (or of the gather list), h and out, with
 * off_g = rows[0] + ... + rows[g-1] computed on the device (no padding)
 * ["Mixture of experts" lecture, systems section: ragged per-expert matmuls].
 *   rows        [groups] int32 (required), e.g. the counts of moe_dispatch
 *   total_rows  [host] an upper bound of rows[0] + ... + rows[groups-1]
 *               (sizes the launch; e.g. T*k), >= 0
 *   a           [total rows, d], or with `gather` the [a_rows, d] token
 *               matrix read through gather[off_g + m]
 *   h, out      [total rows, F] and [total rows, d]
 * Other arguments as for moe_expert_ffn; rows past the packed total are
 * neither read nor written. */
MOE_API moe_status moe_expert_ffn_packed(const moe_config* cfg, int32_t act, int32_t groups,
                                         const int32_t* rows, int64_t total_rows, const void* a,
                                         const int32_t* gather, int64_t a_rows, const void* w_in,
                                         const void* w_gate, const void* b_in, const void* w_out,
                                         const void* b_out, int32_t F, void* h, void* out,
                                         void* stream);

/* Gate-weighted combine with residual fallback ["Lab 18" s.1 layer equation
 * and s.3; "Lab 01" "Where to start" 5; "Phase 02" concept map].
 *   y_t = sum_{j not dropped} gates[t,j] * ye[idx[t,j], slot[t,j]] + shared_out[t]
 *   accumulated in float32 in j order, rounded once to the storage type.
 *   With shared_out NULL, a token with every choice dropped gets x_t (or 0).
 *   x [T,d]; ye [E,C,d] (dropless: [T*k,d], row slot[t,j]); shared_out [T,d]
 *   or NULL; y [T,d] (storage type). */
MOE_API moe_status moe_combine(const moe_config* cfg, const void* x, const void* ye,
                       const void* shared_out, const int32_t* idx, const float* gates,
                       const int32_t* slot, const uint8_t* dropped, void* y, void* stream);

/* Expert-choice selection (routing must be MOE_EXPERT_CHOICE, else
 * MOE_EINVAL) ["Lab 18" exercise 1; see the expert-choice block above].
 *   probs      [T,E] float32 router probabilities (moe_route's probs)
 *   row_token  [E,C] int32: the n = min(C,T) tokens expert e picked, in
 *              ascending order, in row e's first n entries (the rest untouched)
 *   sel        [T,E] int32: the row of token t inside expert e, or -1
 *   counts     [E] int32: n for every expert
 *   ws         workspace (required; it holds the [E,T] transposed keys)
 * Feed row_token and counts to moe_expert_ffn (groups E, rows_per_group C,
 * gather row_token) and sel to moe_combine_expert_choice. */
MOE_API moe_status moe_expert_choice(const moe_config* cfg, const float* probs, int32_t* row_token, int32_t* sel,
                                     int32_t* counts, void* ws, void* stream);

/* Expert-choice combine (routing must be MOE_EXPERT_CHOICE):
 *   y_t = sum over e with sel[t,e] >= 0, in e order, of
 *         probs[t,e] * ye[e, sel[t,e]]  + shared_out[t],
 *   accumulated in float32, rounded once to the storage type; a token with
 *   no pick and no shared_out gets x_t (or 0).
 *   x [T,d]; ye [E,C,d]; shared_out [T,d] or NULL; probs [T,E] float32;
 *   sel [T,E] int32 (moe_expert_choice's); y [T,d]. */
MOE_API moe_status moe_combine_expert_choice(const moe_config* cfg, const void* x, const void* ye,
                                             const void* shared_out, const float* probs, const int32_t* sel,
                                             void* y, void* stream);

/* Auxiliary losses from given logits and choices ["Lab 18" s.2 and "What to
 * implement" 2-3; "Lab 01" traps]: losses[0] = E * sum_i f_i P_i,
 * losses[1] = mean_t logsumexp(z_t)^2 (no alpha applied).
 *   logits [T,E] float32; idx [T,k] int32; losses [2] float32; ws required. */
MOE_API moe_status moe_aux_losses(const moe_config* cfg, const float* logits, const int32_t* idx,
                          float* losses, void* ws, void* stream);

/* Sequence-wise balance loss ["Lab 18" s.2, auxiliary-loss-free note: a
 * small sequence-wise balance loss is kept; "Mixture of experts" lecture,
 * DeepSeek section: the same formula over a different balancing unit]:
 *   loss[0] = (1/B) sum_b E * sum_i f_bi P_bi over the B = T/seq_len
 *   sequences b (tokens [b*seq_len, (b+1)*seq_len)), f_bi = the sequence's
 *   choices routed to i / (seq_len*k), P_bi = the mean of its tokens'
 *   probs[t,i]; no alpha.  Fixed-order float64 reductions.
 *   seq_len [host] > 0, dividing T (MOE_EINVAL otherwise; T > 0)
 *   probs [T,E] float32 (e.g. moe_route's probs); idx [T,k] int32;
 *   loss [1] float32; ws required */
MOE_API moe_status moe_sequence_aux_loss(const moe_config* cfg, int64_t seq_len, const float* probs,
                                         const int32_t* idx, float* loss, void* ws, void* stream);

/* Auxiliary-loss-free balancing ["Lab 18" s.2 and its exercise 4; "Mixture
 * of experts" lecture, DeepSeek section]: the selection bias of every
 * expert whose load is above the mean T*k/E drops by gamma, of every expert
 * below it rises by gamma (float32 adds); an expert at the mean keeps it.
 * The bias enters selection only (moe_route's select_bias).
 *   counts       [E] int32 choices routed to each expert before capacity
 *                (moe_dispatch's or moe_forward's counts)
 *   select_bias  [E] float32, updated in place
 *   gamma        [host] step, finite and >= 0 (the lab uses 0.001) */
MOE_API moe_status moe_update_select_bias(const moe_config* cfg, const int32_t* counts, float* select_bias,
                                          float gamma, void* stream);

typedef struct moe_weights {
  const float* w_router;      /* [d,E] float32                                      */
  const float* logit_bias;    /* [E] float32 or NULL                                */
  const float* select_bias;   /* [E] float32 or NULL                                */
  const void* w_in;           /* GELU: [E,F,d]; SwiGLU: w_up [E,F,d]                */
  const void* w_gate;         /* SwiGLU gate [E,F,d]; NULL for GELU                 */
  const void* b_in;           /* [E,F] or NULL                                      */
  const void* w_out;          /* [E,d,F]                                            */
  const void* b_out;          /* [E,d] or NULL                                      */
  /* shared experts are GELU MLPs (no gate matrix), concatenated:          */
  const void* ws_in;          /* [n_shared*Fs, d]                                   */
  const void* bs_in;          /* [n_shared*Fs] or NULL                              */
  const void* ws_out;         /* [d, n_shared*Fs]                                   */
  const void* bs_out;         /* [d] (sum of the shared experts' output biases) or NULL */
} moe_weights;

typedef struct moe_outputs {
  void* y;                    /* [T,d] storage type                        (required) */
  int32_t* idx;               /* [T,k]                                     (required) */
  float* gates;               /* [T,k]                                     (required) */
  int32_t* slot;              /* [T,k]                                     (required) */
  uint8_t* dropped;           /* [T,k]                                     (required) */
  int32_t* counts;            /* [E]                                       (required) */
  float* losses;              /* [2] {L_aux, L_z}                          (required) */
  int32_t* stats;             /* [4] {kept, dropped, fallback tokens, pad slots} or NULL */
  float* logits;              /* [T,E] or NULL                                        */
  float* probs;               /* [T,E] or NULL                                        */
  float* lse;                 /* [T] or NULL                                          */
  int32_t* sel;               /* [T,E] expert choice: row of t in e or -1 (required then;
                                 ignored under token choice)                          */
} moe_outputs;

/* The whole layer: route -> capacity -> dispatch -> routed (and shared)
 * expert FFNs -> combine, with the losses beside, all on `stream`
 * ["Lab 18" "What to implement" 5: MoE.forward(x) -> (y, aux)].
 * Expert choice: route -> expert choice -> routed (and shared) FFNs ->
 * expert-choice combine; idx and gates then receive the router's top-k
 * when given (they may be NULL), slot and dropped are not used, sel is
 * required.
 * Shared experts: pass them concatenated along their hidden dimension
 * (GELU is elementwise, so the sum of the shared experts equals one MLP
 * whose hidden layer is the concatenation of theirs). */
MOE_API moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                       moe_outputs* out, void* ws, void* stream);

/* moe_forward, recording the caller's HIP events (hipEvent_t handles) on
 * `stream` at the boundaries of its phases, so that a caller can time each
 * phase of a real forward pass (a measurement hook; the pass itself is the
 * same).  n_events must be 7 (MOE_EINVAL otherwise); an entry may be NULL
 * (not recorded).  events[0] before the router, [1] after it, [2] after
 * capacity (or the expert-choice selection), [3] after the routed expert FFN
 * (its two grouped GEMM launches), [4] after the shared experts, [5] after
 * the combine, [6] after the losses.  The library creates, waits on and
 * destroys no event. */
MOE_API moe_status moe_forward_events(const moe_config* cfg, const moe_weights* w, const void* x,
                                      moe_outputs* out, void* ws, void* stream, void* const* events,
                                      int32_t n_events);

/* Gradients of the backward pass (storage type unless marked float32). */
typedef struct moe_grads {
  void* dx;                   /* [T,d]                                     (required) */
  float* dw_router;           /* [d,E] float32                             (required) */
  float* dlogit_bias;         /* [E] float32 or NULL                                  */
  void* dw_in;                /* GELU: [E,F,d]; SwiGLU: the up projection  (required) */
  void* dw_gate;              /* SwiGLU [E,F,d] (required then), else ignored         */
  void* db_in;                /* [E,F] or NULL (GELU only)                            */
  void* dw_out;               /* [E,d,F]                                   (required) */
  void* db_out;               /* [E,d] or NULL                                        */
  void* dws_in;               /* shared experts, concatenated: [n_shared*Fs, d]       */
  void* dbs_in;               /* [n_shared*Fs] or NULL                                */
  void* dws_out;              /* [d, n_shared*Fs]                                     */
  void* dbs_out;              /* [d] or NULL: the gradient of EACH shared expert's
                                 output bias (the forward adds their sum)             */
  float* dgates;              /* [T,k] float32 or NULL; expert choice: [T,E], the
                                 gradient of each picked probability (0 elsewhere)    */
  float* dlogits;             /* [T,E] float32 or NULL                                */
} moe_grads;

/* Bytes of backward workspace for cfg (0 if cfg is invalid or not built). */
MOE_API size_t moe_backward_workspace_bytes(const moe_config* cfg);

/* Backward pass of moe_forward ["Lab 18" s.1 (gate values: with raw top-1
 * gates the router learns through the gate) and s.2 (f_i is a count and has
 * no gradient; the balance loss reaches the router through P_i; the z-loss);
 * "Lab 01" "The traps"; "Mixture of experts" lecture, training a router]:
 * the gradients of  L = <dy, y> + alpha_aux * L_aux + alpha_z * L_z.
 *   - top-k selection and capacity are piecewise constant: no gradient; a
 *     dropped choice's gate gets none; a token that fell back to y = x passes
 *     dy to dx; the selection bias has no gradient;
 *   - the float32 rounding of the logits and the storage roundings are taken
 *     as the identity; H and Ye are the forward's stored values, the expert
 *     pre-activations are recomputed, or read from the forward's workspace
 *     when cfg->save_preact is 1 (bit-identical values: the same products
 *     summed in the same order);
 *   - expert choice ["Lab 18" exercise 1 and "Common extensions"]: the gate
 *     of a pick is the router probability itself, so its gradient reaches
 *     the logits through the probabilities' Jacobian (softmax, or the
 *     sigmoid scores normalised over all experts); the picks carry none;
 *   - built for bf16 storage: token choice with a capacity or dropless
 *     (packed rows), or expert choice; MOE_EUNSUPPORTED otherwise.
 *   x, weights    the forward's inputs
 *   fwd           the forward's outputs: idx, gates, slot, dropped, counts and
 *                 logits are read (logits required); expert choice: sel,
 *                 counts, logits, and probs when the forward was given it
 *   fwd_ws        the forward's workspace, unchanged since that call (its
 *                 expert rows, hidden activations and outputs are read)
 *   dy            [T,d] storage type
 *   alpha_aux, alpha_z  [host] loss weights (0 leaves a loss out)
 *   grads         see moe_grads; weight gradients are written, not added to
 *   bws           backward workspace of moe_backward_workspace_bytes() bytes
 * Weight gradients contract over tokens with float32 accumulation in the
 * matrix cores; the router-weight gradient uses the exact three-plane bf16
 * split of dL/dz (as the router does for its weight). */
MOE_API moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                                const moe_outputs* fwd, const void* fwd_ws, const void* dy, float alpha_aux,
                                float alpha_z, moe_grads* grads, void* bws, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
MOE_API const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
