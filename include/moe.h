/*
 * moe.h -- C ABI of the gfx950 fused Mixture-of-Experts layer forward.
 *
 * The layer: top-k routing -> expert-major token dispatch -> grouped GEMM
 * with the gate and up projections fused over one input tile and SwiGLU
 * applied to the accumulators -> down-projection grouped GEMM -> weighted
 * top-k combine, for one GPU that holds every expert.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless their name starts with host_.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream).  The returned status reports argument validation
 *    and launch errors only; a fault inside a kernel surfaces at the
 *    caller's next synchronisation.
 *  - The caller owns every buffer: inputs, outputs, weights and the
 *    workspace memory.  No entry point allocates device memory, except
 *    moe_layer_forward's graph instantiation, once per (token count,
 *    stream) at decode sizes (see moe_workspace_set_graphs).
 *  - A workspace serves one stream at a time (LightMoE README, "MoE
 *    inference": one plan per concurrent stream because workspaces are
 *    reused).  Calls that share a workspace on different streams race.
 *  - Matrices are row-major.  Expert weights are [E, N, K] with K
 *    contiguous, so every projection computes out = A * B^T (LightMoE README,
 *    "Dense GEMM" and "Grouped GEMM").
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_EINVAL 1        /* bad argument (null pointer, bad size, bad enum) */
#define MOE_EUNSUPPORTED 2  /* well-formed but outside what the kernels cover */
#define MOE_ECAPACITY 3     /* exceeds the workspace's max_tokens / capacity */
#define MOE_EHIP 4          /* a HIP runtime call failed */

/* Router score functions (top-k always compares the given fp32 scores). */
#define MOE_SCORE_SOFTMAX 0 /* scores are logits; weights = softmax over the k chosen */
#define MOE_SCORE_SIGMOID 1 /* scores are logits; weights = sigmoid, renormalised over k */
#define MOE_SCORE_PROBS 2   /* scores are probabilities; weights = p / sum of the k */

/* Weight formats (stored codes, quantised offline by the caller). */
#define MOE_W_BF16 0         /* bf16 [E,N,K] */
#define MOE_W_FP8_CHANNEL 1  /* e4m3 [E,N,K] + fp32 scale per output row [E,N] */
#define MOE_W_FP8_BLOCK128 2 /* e4m3 [E,N,K] + fp32 scale per 128x128 block [E,N/128,K/128] */
#define MOE_W_MXFP4 3        /* e2m1 packed [E,N,K/2] (element 2i in the low nibble)
                                + e8m0 scale per 1x32 block [E,N,K/32] (OCP MX v1.0) */

/* Activation formats (quantised on the fly by the layer). */
#define MOE_A_BF16 0         /* no quantisation; the intermediate is rounded to bf16 */
#define MOE_A_FP8_TOKEN 1    /* e4m3, one fp32 scale per row (amax/448) */
#define MOE_A_FP8_G128 2     /* e4m3, one fp32 scale per 1x128 group */
#define MOE_A_MXFP8_G32 3    /* e4m3, one e8m0 scale per 1x32 group (OCP MX v1.0) */

/* Grouped GEMM operations. */
#define MOE_OP_PLAIN 0          /* out[r, n] = sum_k A[r,k] * B0[e,n,k], fp32 out */
#define MOE_OP_GATEUP_ACT 1     /* out[r, n] = act(A*B0^T, A*B1^T), activation format */
#define MOE_OP_GATEUP_SWIGLU MOE_OP_GATEUP_ACT  /* the default activation is SwiGLU */

/* Expert activations, act(g, u) of the gate value g and the up value u
 * (LightMoE README, "Compatibility" and "MoE inference": SwiGLU, bounded
 * SwiGLU with an activation clamp, SwiGLU-OAI, GeGLU, ReGLU, ReLU^2 in the
 * two-weight form).  The pages name them without formulas; L is the desc's
 * act_limit (<= 0 selects 10 for bounded SwiGLU, 7 for SwiGLU-OAI). */
#define MOE_ACT_SWIGLU 0          /* SiLU(g) * u */
#define MOE_ACT_SWIGLU_BOUNDED 1  /* SiLU(min(g, L)) * clamp(u, -L, L) */
#define MOE_ACT_SWIGLU_OAI 2      /* g' sigmoid(1.702 g') (clamp(u, -L, L) + 1), g' = min(g, L) */
#define MOE_ACT_GEGLU 3           /* g (1 + erf(g / sqrt 2)) / 2 * u */
#define MOE_ACT_REGLU 4           /* max(g, 0) * u */
#define MOE_ACT_RELU2 5           /* max(u, 0)^2: no gate projection (w_gate unused, may be
                                     NULL; the GEMM's B0 may be NULL) */

typedef struct moe_ws moe_ws; /* opaque host handle */

/* Shape and formats of one MoE layer (fixed at workspace creation). */
typedef struct moe_layer_desc {
  int hidden;          /* H: multiple of 128 */
  int inter;           /* I: multiple of 128 */
  int num_experts;     /* E: 1..256 routed experts */
  int top_k;           /* k: 1..min(E,16) */
  int shared_experts;  /* 0 or 1 always-on shared expert (weight 1, outside renormalisation) */
  int shared_inter;    /* I of the shared expert; must equal `inter` when shared_experts = 1 */
  int score_fn;        /* MOE_SCORE_* */
  int renormalize;     /* must be 1 (gate weights renormalised over the k chosen) */
  int w_format;        /* MOE_W_* */
  int a_format;        /* MOE_A_*; pairs: BF16/BF16, FP8_CHANNEL/FP8_TOKEN,
                          FP8_BLOCK128/FP8_G128, MXFP4/MXFP8_G32 */
  int max_tokens;      /* T capacity; T*top_k must not exceed 1,048,576 */
  int activation;      /* MOE_ACT_* (0 = SwiGLU) */
  float act_limit;     /* clamp L of the bounded activations; <= 0: their default */
} moe_layer_desc;

/* Caller-owned expert weights, layout [E, N, K] K-contiguous (see formats). */
typedef struct moe_weights {
  const void *w_gate, *w_up, *w_down;   /* [E,I,H], [E,I,H], [E,H,I] codes */
  const void *s_gate, *s_up, *s_down;   /* scales per format, or NULL for bf16 */
  const void *sh_gate, *sh_up, *sh_down;/* shared expert [1,Is,H],[1,Is,H],[1,H,Is] or NULL */
  const void *ss_gate, *ss_up, *ss_down;
} moe_weights;

/* Human-readable text for a status code (static storage). */
MOE_API const char* moe_status_string(int status);
/* Detail of the last error on the calling thread (thread-local storage). */
MOE_API const char* moe_last_error(void);

/* Bytes of device memory a workspace for `desc` needs.  Errors: EINVAL,
 * EUNSUPPORTED for a shape or format pair outside the validation rules. */
MOE_API int moe_workspace_size(const moe_layer_desc* desc, size_t* host_bytes);

/* Build a workspace handle over caller-owned device memory `dev_buf` of
 * `bytes` (at least moe_workspace_size, 256-byte aligned).  The handle is
 * host memory owned by the library; the device buffer stays the caller's and
 * must outlive the handle.  Also loads the kernels on the current device. */
MOE_API int moe_workspace_create(const moe_layer_desc* desc, void* dev_buf, size_t bytes, moe_ws** out);

/* Release the handle (and any graphs it instantiated).  NULL is a no-op. */
MOE_API int moe_workspace_destroy(moe_ws* ws);

/* Top-k routing (Alpha-MoE news page, "How the megakernel works": routing
 * and gating; LightMoE README, "MoE inference": int32 ids distinct per
 * token, fp32 weights).
 *   scores     [T, E] fp32: logits (SOFTMAX/SIGMOID) or probabilities (PROBS)
 *   topk_ids   [T, k] int32 out: the k largest scores in descending order,
 *              ties broken towards the lower expert index (+0 == -0)
 *   renorm     must be 1: the weights are renormalised over the k chosen
 *              (the only form the layer computes; 0 gives EUNSUPPORTED)
 *   topk_w     [T, k] fp32 out: gate weights renormalised over the k
 * T = 0 is a no-op.  Errors: EINVAL (nulls, k < 1, k > min(E,16), E > 256),
 * EUNSUPPORTED (renorm != 1). */
MOE_API int moe_route_topk(const float* scores, int T, int E, int k, int score_fn, int renorm,
                   int32_t* topk_ids, float* topk_w, void* stream);

/* Deterministic expert-major dispatch (LightMoE README, API table and "MoE
 * training": gather indices, m_indptr, inverse slots; "Grouped GEMM":
 * m_indptr has E+1 entries and zero-row experts are valid).  Slots are
 * ordered by expert, then by flat index t*k+j.
 *   topk_ids  [T, k] int32 in, each in [0, E)
 *   counts    [E]   int32 out: rows per expert
 *   m_indptr  [E+1] int32 out: exclusive prefix sum of counts
 *   gather    [T*k] int32 out: slot -> t*k+j
 *   inv       [T*k] int32 out: t*k+j -> slot
 * E must equal the workspace's num_experts and T <= max_tokens.  An id
 * outside [0, E) takes no slot: it is not counted, its inv entry is -1 and
 * m_indptr[E] falls short of T*k by the number of such ids.  The workspace
 * supplies scratch (per-chunk histograms); inv also holds per-chunk ranks
 * between the two launches of large batches.  Errors: EINVAL, ECAPACITY. */
MOE_API int moe_dispatch(moe_ws* ws, const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                 int32_t* m_indptr, int32_t* gather, int32_t* inv, void* stream);

/* moe_dispatch without a workspace, for callers that cannot allocate device
 * memory or create a workspace (code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, outputs and
 * rules as moe_dispatch (E is given here, not taken from a workspace).  Its
 * scratch (group list, block table, per-chunk histograms) is a static device
 * array of about 1.7 MB that the library holds on each GPU it runs on until
 * the process ends; nothing is allocated or freed per call.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race.  Limits: E <= 256,
 * k <= min(E, 16), T*k <= 1,048,576 (ECAPACITY beyond).  Errors: EINVAL,
 * ECAPACITY, EHIP. */
MOE_API int moe_dispatch_noalloc(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                                 int32_t* m_indptr, int32_t* gather, int32_t* inv, void* stream);

/* Grouped GEMM over expert-major rows, one launch for all experts and no
 * padding (pure-Triton MoE commentary, second paragraph: block-id ->
 * (expert, offset) map; LightMoE README, "Grouped GEMM").
 *   op        MOE_OP_PLAIN or MOE_OP_GATEUP_ACT (the workspace's activation)
 *   a         activation rows in the workspace's activation format:
 *             bf16 [rows, K] for A_BF16, else e4m3 codes [rows, K]
 *   a_scale   activation scales: fp32 [rows] (FP8_TOKEN), fp32 [rows, K/128]
 *             (FP8_G128), uint8 e8m0 [rows, K/32] (MXFP8_G32); NULL for bf16
 *   a_gather  NULL: row r of group e is a[m_indptr[e] + r]; else it is
 *             a[a_gather[m_indptr[e] + r] / gather_div] (pass moe_dispatch's
 *             gather and top_k to read token rows in place)
 *   m_indptr  [E+1] int32, m_indptr[E] = total rows R (<= workspace capacity)
 *   N, K      output columns and contraction length; b0/b1 are [E, N, K]
 *             in the workspace's weight format with scales b0_scale/b1_scale
 *             (b1 only for GATEUP_ACT; b0 unused and may be NULL for
 *             MOE_ACT_RELU2)
 *   out       PLAIN: fp32 [R, N].  GATEUP_ACT: h in the activation
 *             format (bf16 [R, N], or e4m3 codes [R, N] + out_scale as for
 *             a_scale with K replaced by N)
 * The tile configuration (streaming, or 32-, 64- or 128-row blocks) is
 * chosen on the device from the group sizes in m_indptr, as in
 * moe_layer_forward (moe_workspace_force_config pins it).  m_indptr is read
 * on the device only: when it is not non-decreasing from 0, or its last
 * entry exceeds the workspace's row capacity, the device computes no rows
 * (out is left as it was) and moe_workspace_check reports EINVAL.
 * Errors: EINVAL, EUNSUPPORTED (N or K not a multiple of 128), ECAPACITY. */
MOE_API int moe_grouped_gemm(moe_ws* ws, int op, const void* a, const void* a_scale,
                     const int32_t* a_gather, int gather_div, const int32_t* m_indptr, int E,
                     int N, int K, const void* b0, const void* b0_scale, const void* b1,
                     const void* b1_scale, void* out, void* out_scale, void* stream);

/* Dynamic activation quantisation of bf16 rows x [T, H] into the
 * workspace's activation format (LightMoE README, "MoE inference": input
 * quantisation): per group, s = amax/448 in fp32 (1 when amax = 0) and
 * q = e4m3_rne(clamp(x/s, +-448)); MX groups use X = 2^(floor(log2 amax)-8).
 *   q [T, H] e4m3 codes out, scale as a_scale of moe_grouped_gemm.
 * Errors: EINVAL, EUNSUPPORTED (bf16 format: nothing to quantise). */
MOE_API int moe_quantize_act(moe_ws* ws, const uint16_t* x_bf16, int T, uint8_t* q, void* scale,
                     void* stream);

/* Weighted top-k combine (LightMoE README, "MoE inference": routing-weight
 * application and deterministic combine):
 *   y[t] = bf16( sum_{j<k} w[t,j] * out_slot[inv[t*k+j]] (+ out_slot[T*k+t]
 *          when the layer has a shared expert) ), j ascending, fp32 sums.
 *   out_slot [T*k (+T), H] fp32; y [T, H] bf16 out.
 * A negative inv entry (an id moe_dispatch dropped) contributes nothing. */
MOE_API int moe_combine(moe_ws* ws, const float* out_slot, const float* topk_w, const int32_t* inv, int T,
                uint16_t* y_bf16, void* stream);

/* The whole layer: x bf16 [T, H] and router scores [T, E] -> y bf16 [T, H].
 * Runs routing, dispatch, activation quantisation, the fused gate/up
 * grouped GEMM with the desc's activation in its epilogue, intermediate requantisation, the down grouped GEMM and the
 * combine.  The tile configuration is chosen on the device from the expert
 * histogram (RaMP abstract: configuration from the runtime routing
 * distribution, not batch size alone).  T = 0 is a no-op.
 * Errors: EINVAL, ECAPACITY (T > max_tokens), EHIP. */
MOE_API int moe_layer_forward(moe_ws* ws, const moe_weights* w, const uint16_t* x_bf16,
                      const float* scores, int T, uint16_t* y_bf16, void* stream);

/* Routing results of the workspace's last moe_layer_forward (device
 * pointers into the workspace, valid until the next call):
 * topk_ids [T,k], topk_w [T,k], counts [E(+1)], m_indptr [E+2 with the
 * shared group], gather, inv.  Any out pointer may be NULL. */
MOE_API int moe_workspace_routing(const moe_ws* ws, const int32_t** topk_ids, const float** topk_w,
                          const int32_t** counts, const int32_t** m_indptr,
                          const int32_t** gather, const int32_t** inv);

/* Block table of the workspace's last dispatch (moe_layer_forward,
 * moe_dispatch or moe_grouped_gemm), device pointers into the workspace:
 * tiles [2 * n] int32 pairs (row group, first row of the block), groups in
 * ascending order, ceil(rows / BM) blocks per group (pure-Triton MoE
 * commentary, second paragraph: block-id -> (expert, offset) map); meta
 * [16] int32 words: [0] active groups, [1] n = table entries, [2] the
 * configuration, [3] largest group, [4] rows, [5] BM, [6] device status
 * (nonzero: m_indptr rejected).  Any out pointer may be NULL. */
MOE_API int moe_workspace_tiles(const moe_ws* ws, const int32_t** tiles, const int32_t** meta);

/* Synchronise `stream` and report the device-side status of the
 * workspace's last dispatch in *device_status: MOE_OK; MOE_EINVAL when the
 * device rejected a caller's m_indptr (moe_grouped_gemm then computed no
 * rows); MOE_EHIP when the single-launch decode layer could not make its
 * whole grid resident and stopped (its output is then incomplete, and the
 * workspace must be created again).  moe_last_error names the reason.
 * Returns EHIP if the synchronisation fails. */
MOE_API int moe_workspace_check(const moe_ws* ws, int* device_status, void* stream);

/* Number of instantiated decode graphs the workspace holds: at most one per
 * (token count, stream), whatever buffers the calls pass. */
MOE_API int moe_workspace_graph_count(const moe_ws* ws, int* host_n);

/* Force the tile configuration (tests and cost-model fitting): -1 = choose
 * from the histogram (default); 0 = streaming decode kernels; 1.. = tiled
 * kernels with a row-block height given by moe_config_rows(cfg). */
MOE_API int moe_workspace_force_config(moe_ws* ws, int cfg_id);

/* Choose the configuration of moe_layer_forward with the fitted wave cost
 * model (1, default) or with the fixed histogram rule (0).  RaMP abstract:
 * a four-parameter wave cost model, fitted once from profiling, picks the
 * fastest configuration from the runtime expert histogram and depends only
 * on the kernels' grid geometry.  Configuration c's predicted time is
 *   th[r][0] + th[r][1]*x1 + th[r][2]*x2 + th[r][3]*x3   (microseconds)
 * with x1 the weight bytes it streams over the 8 TB/s HBM peak, x2 the MFMA
 * work of its padded row blocks over the format's dense MFMA peak, and x3
 * its grid waves (gate/up and down summed); r = c, except r = 4 for the
 * streaming configuration above 16 tokens (another kernel variant).  The
 * host launches the kernels of a candidate set chosen before the histogram
 * exists (moe_workspace_candidates) and the dispatch kernel picks, on the
 * real histogram, the least predicted time within it.  Results do not
 * depend on the configuration beyond the format's tolerance (the K split
 * and summation order differ between configurations).  Clears the
 * workspace's decode graphs. */
MOE_API int moe_workspace_set_config_model(moe_ws* ws, int enable);

/* The configurations (bit c = configuration c) whose kernels
 * moe_layer_forward launches for a batch of T tokens: the one forced, the
 * cost model's candidate set (the set whose best member's predicted time,
 * averaged with weights 0.8 / 0.2 over two routings - T*k rows spread
 * evenly over the experts, and packed into k experts of T rows; a shared
 * expert adds T rows - plus 9 us for every launch beyond the first is
 * least), or
 * the families the histogram rule can land on.  Host only, no GPU work. */
MOE_API int moe_workspace_candidates(const moe_ws* ws, int T, int* host_mask);

/* The fitted parameters th[5][4] compiled into the library (row-major, 20
 * doubles), as moe_workspace_set_config_model describes them. */
MOE_API int moe_config_model_params(double* host_theta20);
/* Configuration used by the last moe_layer_forward (synchronises `stream`). */
MOE_API int moe_workspace_last_config(const moe_ws* ws, int* host_cfg_id, void* stream);
/* Row-block height of a configuration, or -1 if unknown. */
MOE_API int moe_config_rows(int cfg_id);

/* Enable (1, default) or disable (0) hipGraph capture of moe_layer_forward
 * for decode token counts (T <= 128): the first call at each (T, stream)
 * captures and instantiates a graph, later calls with the same pointers
 * replay it, and a call with other pointers re-captures and updates that
 * instance in place (hipGraphExecUpdate; re-instantiated only if the update
 * is refused), so the instances stay one per (T, stream).
 * A call made while `stream` is being captured by the caller (for example
 * a whole model step in one graph) enqueues its kernels into the caller's
 * capture instead; no library call on the path allocates or sets memory,
 * so the captured launches replay like the eager ones. */
MOE_API int moe_workspace_set_graphs(moe_ws* ws, int enable);

/* Enable (1) or disable (0, default) the single-launch decode layer: for
 * batches of at most 16 tokens moe_layer_forward then runs routing,
 * dispatch, both quantisations, both grouped GEMMs and the combine in one
 * persistent kernel (Alpha-MoE news page, "How the megakernel works"),
 * with one grid-wide barrier between the projections.  It applies when
 * hidden and inter are multiples of 512 and no tiled configuration is
 * forced; otherwise, or when disabled, the layer runs its separate kernels.
 * Its grid holds only workgroups that can be resident at once and its
 * barrier's wait is bounded: should the launch not get every workgroup
 * resident (another kernel holding the GPU), it stops and sets the device
 * status that moe_workspace_check reports, rather than waiting for ever.
 * Results equal the separate kernels' streaming configuration bit for bit
 * (GeGLU: within one bf16 step on a few outputs).  It is off by default
 * because on gfx950 it is slower than the separate kernels: every
 * workgroup's device-wide release before the barrier writes back its XCD's
 * L2, which a kernel boundary does once. */
MOE_API int moe_workspace_set_fused_decode(moe_ws* ws, int enable);

/* Profiling: record the caller's HIP events (hipEvent_t, created with
 * timing enabled) immediately before and after the launches of one stage of
 * moe_layer_forward.  Stages: 0 routing + dispatch, 1 input quantisation,
 * 2 gate/up grouped GEMM, 3 intermediate requantisation, 4 down grouped
 * GEMM, 5 combine, 6 the single-launch decode layer (which replaces stages
 * 0-5 when it runs); moe_expert_backward: 7 gate/up recomputation (and the
 * weight transposes of shapes whose hidden or inter size is not a multiple
 * of 256), 8 down input gradient (one launch), 9 per-slot pass, 10 gate/up
 * input gradient (one launch), 11 input gradient combine, 12 down weight
 * gradient, 13 gate and up weight gradients.  NULL events clear the stage.  While any forward stage has
 * events, moe_layer_forward runs its eager path (no graph replay). */
MOE_API int moe_workspace_set_stage_events(moe_ws* ws, int stage, void* ev_begin, void* ev_end);

/* ------------------------------------------------------------------ backward
 * Training-side gradients of the routed expert layer (LightMoE README, "MoE
 * training" and "Highlights": deterministic dispatch, combine, input-,
 * weight- and router-gradient kernels).  bf16 weights and activations only
 * (w_format MOE_W_BF16, a_format MOE_A_BF16), no shared expert, and every
 * activation but ReGLU (the pages' training set excludes it).
 *
 * Bytes of the caller-owned scratch buffer moe_expert_backward needs for a
 * workspace of this description (max_tokens * top_k slots). */
MOE_API int moe_backward_scratch_size(const moe_layer_desc* desc, size_t* bytes);

/* Gradients of a loss L with respect to the layer input, the expert weights
 * and the routing weights, given dy = dL/dy for
 *   y_t = sum_j topk_w[t, j] * W_down[e] act(W_gate[e] x_t, W_up[e] x_t),
 *   e = topk_ids[t, j].
 * Per slot, r = W_down[e]^T dy_t (fp32 accumulation of bf16 operands):
 *   d_topk_w[t, j] = <r, h>,  h = bf16(act(g, u)) recomputed from x
 *   dg = bf16(w r dact/dg), du = bf16(w r dact/du)
 *   dx_t = bf16(sum_j (W_gate[e]^T dg + W_up[e]^T du)), j ascending
 *   d_w_down[e]  = sum over e's slots of bf16(w dy_t) h^T     [E, H, I]
 *   d_w_gate[e]  = sum over e's slots of dg x_t^T             [E, I, H]
 *   d_w_up[e]    = sum over e's slots of du x_t^T             [E, I, H]
 * (expert slots in ascending (t, j) order; experts without tokens get
 * zeros).  Every sum has a fixed order, so results are reproducible bit for
 * bit.  Inputs (device): w->w_gate/w_up/w_down bf16 [E, I, H] / [E, I, H] /
 * [E, H, I] (w_gate unused and may be NULL for ReLU^2); x, dy bf16 [T, H];
 * topk_ids int32 [T, k] (distinct per token, < E), topk_w fp32 [T, k].
 * Outputs (device, caller-owned, fully written): dx bf16 [T, H]; d_w_gate
 * (not written for ReLU^2, may be NULL), d_w_up, d_w_down fp32; d_topk_w
 * fp32 [T, k].  scratch: device memory of at least
 * moe_backward_scratch_size bytes (scratch_bytes); the call allocates
 * nothing.  The workspace's routing buffers are overwritten (dispatch of
 * topk_ids).  T = 0 writes nothing.  Errors: MOE_EUNSUPPORTED for formats,
 * shapes (hidden and inter multiples of 128) or activations outside the
 * list above; MOE_ECAPACITY for T > max_tokens or a short scratch buffer;
 * MOE_EINVAL for NULL pointers. */
MOE_API int moe_expert_backward(moe_ws* ws, const moe_weights* w, const void* x,
                                const int32_t* topk_ids, const float* topk_w, int T, const void* dy,
                                void* dx, float* d_w_gate, float* d_w_up, float* d_w_down,
                                float* d_topk_w, void* scratch, size_t scratch_bytes, void* stream);

/* Router gradient: dL/dscores [T, E] fp32 from d_topk_w = dL/dtopk_w [T, k],
 * for weights renormalised over the k selected experts (the selection is
 * piecewise constant).  With m = sum_j topk_w[t, j] d_topk_w[t, j], a
 * selected expert i gets
 *   MOE_SCORE_SOFTMAX  w_i (dw_i - m)
 *   MOE_SCORE_SIGMOID  s_i (1 - s_i) (dw_i - m) / sum_sel s,  s = sigmoid(score)
 *   MOE_SCORE_PROBS    (dw_i - m) / sum_sel p
 * and every other expert 0 (the whole [T, E] output is written).  All
 * pointers are device pointers; topk_ids/topk_w as moe_route_topk returns
 * them.  Errors: MOE_EINVAL for a bad T, E, k or score_fn or NULL pointers. */
MOE_API int moe_router_backward(const float* scores, const int32_t* topk_ids, const float* topk_w,
                                const float* d_topk_w, int T, int E, int k, int score_fn,
                                float* d_scores, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
