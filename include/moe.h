/*
 * moe.h -- C ABI of libmoe: the forward pass of a sparse mixture-of-experts
 * feed-forward layer with a per-expert capacity limit, on one AMD Instinct
 * MI355X (gfx950) GPU with every expert resident in HBM.
 *
 * Pages this interface follows (titles; sections named, not numbered lines):
 *   [Mixtral explainer] "Mixtral 8x7B and MoE explained" (allinfo.ai.kr)
 *   [MoE wiki]          "Mixture of experts" (wikiprompt.org)
 *   [Routing guide]     "MoE routing, fully explained: Mixtral/DeepSeek
 *                        structure, load balancing, capacity factor"
 *                        (allinfo.ai.kr)
 *
 * The layer, per token x (a row of d values):
 *   1. router scores   l = x . W_gate (+ bias)         [Mixtral explainer]
 *      "Plain explanation" para 3; [Routing guide] "Plain explanation" para 2
 *   2. top-k experts by score (ties: lower index; -0 == +0), gates either
 *      softmax over the k chosen scores (Mixtral) or the full softmax over all
 *      E experts read at the chosen ones (DeepSeek), optionally renormalised
 *      [Mixtral explainer] para 3; [Routing guide] paras 2 and 4
 *   3. dispatch with capacity C = ceil(T*k*cf/E) slots per expert; the
 *      assignments beyond C (the latest in flat order a = t*k + j) are
 *      dropped, sent to spare experts or kept for later rounds
 *      (moe_overflow_t)   [Routing guide] "Plain explanation" paras 3 and 5
 *   4. expert FFN, SwiGLU: y = (silu(x W1[e]) * (x W3[e])) W2[e]
 *      [Mixtral explainer] "Plain explanation" para 2
 *   5. out = sum over kept j of w[t,j] * y[t,j]  +  sum of S shared experts
 *      (gate 1); dropped choices contribute nothing and the surviving gates
 *      are not renormalised   [MoE wiki] "How it works"; [Routing guide]
 *      "Plain explanation" para 4
 *   6. statistics: aux = E * sum_i f_i P_i with f_i = count_i/(T k) before
 *      drops and P_i the mean full softmax; overflow rate; entropy of the
 *      load and mean per-token router entropy (nats)
 *      [Routing guide] "Plain explanation" para 4, "Key insights" item 3
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     allocates nothing on any call.  Scratch memory is the caller's
 *     workspace (cfg->workspace, at least moe_workspace_size(cfg) bytes,
 *     256-byte aligned).  One workspace must not be used by two calls that
 *     may overlap in time.
 *   - All layouts are dense row-major with no padding:
 *       x [T, d]; W_gate [d, E]; W1, W3 [E+S, d, F]; W2 [E+S, F, d];
 *       out [T, d]; logits [T, E] fp32; bias [E] fp32.
 *     The S shared experts follow the E routed experts in W1/W3/W2, which
 *     may instead be given in the packed layout (moe_weight_layout_t).
 *   - x, W_gate, W1, W3, W2 and out share cfg->dtype (fp32 or bf16); router
 *     logits, bias and gate weights are fp32; indices int32.
 *   - x, W_gate, W1, W3, W2, out (and the packed weight buffers) must be
 *     16-byte aligned, as device allocations are; a view that starts
 *     part-way into an allocation may not be, and is rejected (MOE_EINVAL).
 *   - Work is enqueued on cfg->stream (a hipStream_t; NULL = the null
 *     stream) and returns before it finishes, unless a host-side result is
 *     requested (stats != NULL, moe_aux_loss), in which case the call waits
 *     for the stream.
 *   - Return value: MOE_OK (0) or a negative moe_status_t.  Arguments are
 *     checked completely before anything is enqueued.  The reason for the
 *     last failure on the calling thread is in moe_last_error().
 *   - T = 0 is a valid, empty call: nothing is launched and stats are zero.
 *   - With stats == NULL, moe_forward and moe_router_backward only enqueue
 *     kernels on cfg->stream (no allocation, copy, memset or host wait), so
 *     a caller may capture them into a HIP graph and replay it; a replay
 *     reads the inputs' current contents.  Per-kernel timing must be off
 *     while capturing.
 *   - A NaN router score ranks as -infinity (chosen only after every
 *     number; ties by index) and gets gate weight 0.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument: null pointer, size, k > E, ... */
  MOE_EUNSUPPORTED = -2,  /* valid layer the library does not build */
  MOE_EWORKSPACE = -3,    /* workspace missing, too small or misaligned */
  MOE_EHIP = -4           /* a HIP runtime call failed */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_TOPK_THEN_SOFTMAX = 0,  /* Mixtral: softmax over the k chosen logits */
  MOE_SOFTMAX_THEN_TOPK = 1   /* DeepSeek: softmax over all E, read top-k */
} moe_gating_t;

/* How the bf16 down projections (hidden -> model width) are laid out over the
 * GPU.  Both paths run the same MFMA kernels and give results equal to
 * rounding order.  fp32 layers accept AUTO and GROUPED only. */
typedef enum {
  MOE_PATH_AUTO = 0,     /* split K only when the output tiles alone give
                            fewer than 256 workgroups (short batches) */
  MOE_PATH_GROUPED = 1,  /* never split K: one workgroup per output tile */
  MOE_PATH_STREAM = 2    /* always split K toward ~512 workgroups, streaming
                            each expert's weights through many CUs */
} moe_ffn_path_t;

/* What happens to assignments beyond an expert's C slots.  [Routing guide]
 * "Plain explanation" para 3 names the three choices.  In every policy an
 * expert first takes its own assignments in flat order a = t*k + j, up to C.
 *   DROP        the rest contribute nothing.
 *   REROUTE     then the rest, in flat order, each go to the highest-scoring
 *               expert (ties: lower index) that token t did not choose, that
 *               t's earlier assignments were not sent to (a token never
 *               meets one expert twice) and that still has a free slot,
 *               placed after the rows already there, with their own gate
 *               weight; dropped if none has room.
 *               Runs a one-workgroup pass; short batches lose the fused
 *               single-kernel routing.
 *   SEQUENTIAL  nothing is dropped: every assignment is processed by its
 *               expert, as if in rounds of C rows (one launch runs all the
 *               rounds' rows, so the output equals the unlimited layer and
 *               the workspace holds T*k rows); stats report the rounds. */
typedef enum {
  MOE_OVERFLOW_DROP = 0,
  MOE_OVERFLOW_REROUTE = 1,
  MOE_OVERFLOW_SEQUENTIAL = 2
} moe_overflow_t;

/* How W1, W3 and W2 are stored (cfg->weight_layout).  The expert weights are
 * the feed-forward matrices of [Mixtral explainer] "Plain explanation" para
 * 2; the layout changes where each element sits, not what is computed, so a
 * layer gives the same bits with either layout.
 *   ROW_MAJOR  W1, W3 [E+S, d, F] and W2 [E+S, F, d] as described above.
 *   PACKED     the copies moe_pack_weights writes (bf16 layers only): each
 *              expert's matrix cut into blocks of 32 rows x Wb columns (Wb =
 *              128 for W1 and W3, 256 for W2), each block stored as one
 *              contiguous run, column by column (the 32 values of one
 *              column next to each other), so one K step of one output
 *              tile of the expert GEMMs reads whole runs instead of a short
 *              piece of each of 32 rows, already in the k-contiguous order
 *              the matrix-core operands take.  For a [K, N] matrix of
 *              expert e, with N' = N rounded up to Wb, element (k, n) sits at
 *                e*K*N' + ((k/32)*(N'/Wb) + n/Wb)*32*Wb + (n%Wb)*32 + k%32
 *              and the N' - N pad columns hold zeros. */
typedef enum {
  MOE_WEIGHTS_ROW_MAJOR = 0,
  MOE_WEIGHTS_PACKED = 1
} moe_weight_layout_t;

typedef struct {
  int64_t T;             /* tokens in this call, >= 0 */
  int32_t d_model;       /* d */
  int32_t d_ff;          /* F, hidden width of one expert */
  int32_t n_experts;     /* E routed experts, 1..256 */
  int32_t top_k;         /* k, 1..E */
  int32_t n_shared;      /* S always-on shared experts, >= 0 */
  int32_t gating;        /* moe_gating_t */
  int32_t renormalize;   /* DeepSeek gating: divide kept gates by their sum */
  double capacity_factor;/* <= 0: no limit (C = T) */
  int32_t dtype;         /* moe_dtype_t */
  int32_t ffn_path;      /* moe_ffn_path_t */
  const float* logit_bias; /* device [E] fp32 added to the router scores, or NULL */
  void* workspace;       /* device scratch, see moe_workspace_size */
  size_t workspace_bytes;
  void* stream;          /* hipStream_t */
  int32_t overflow;      /* moe_overflow_t (0 = drop) */
  int32_t weight_layout; /* moe_weight_layout_t (0 = row-major) */
  int32_t out_fp32;      /* 0: out in cfg->dtype; 1: out is fp32 [T, d] for
                            either dtype (a bf16 layer then stores the fp32
                            sum it would otherwise round to bf16, RNE) */
} moe_config_t;

typedef struct {
  int64_t capacity;      /* C */
  int64_t assignments;   /* T * k */
  int64_t dropped;       /* assignments no expert processes */
  int64_t* counts;       /* host [E] per-expert assignments before drops, or NULL */
  int64_t* kept;         /* host [E] rows each expert processes (rerouted
                            rows included), or NULL */
  double aux_loss;       /* E * sum f_i P_i, f_i = counts_i / (T k) */
  double aux_loss_kept;  /* same with kept counts */
  double overflow_rate;  /* dropped / (T k) */
  double entropy_load;   /* -sum f_i ln f_i */
  double entropy_token;  /* mean over tokens of -sum_i p_ti ln p_ti */
  int64_t overflowed;    /* sum_i max(counts_i - C, 0): assignments that found
                            their chosen expert full */
  int64_t rerouted;      /* of those, placed on a spare expert (REROUTE) */
  int64_t rounds;        /* max_i ceil(counts_i / C): C-row rounds the busiest
                            chosen expert needs (0 when T = 0) */
} moe_stats_t;

/* Validate cfg without touching the GPU.  Bounds: T >= 0, T*k < 2^31,
 * d, F > 0; bf16 additionally needs d % 64 == 0 and F % 64 == 0
 * (MOE_EUNSUPPORTED otherwise); 1 <= E <= 256; 1 <= k <= E; S >= 0; the
 * enums in range.  The workspace is not checked here. */
int moe_check_config(const moe_config_t* cfg);

/* Bytes of workspace moe_forward / moe_route / moe_route_logits need for
 * cfg (workspace fields ignored).  0 when cfg is invalid. */
size_t moe_workspace_size(const moe_config_t* cfg);

/* Bytes of one packed copy of W1 (the same for W3) and of W2 for cfg's
 * shapes (E+S experts, moe_weight_layout_t PACKED): *w13_bytes =
 * 2*(E+S)*d*F', *w2_bytes = 2*(E+S)*F*d', F' and d' rounded up to 128 and
 * 256.  Host only.  MOE_EUNSUPPORTED for fp32 layers. */
int moe_packed_weight_bytes(const moe_config_t* cfg, size_t* w13_bytes, size_t* w2_bytes);

/* Writes the packed copies (moe_weight_layout_t PACKED) of the row-major
 * bf16 expert weights W1, W3, W2 into W1p, W3p (w13_bytes each) and W2p
 * (w2_bytes), all caller-owned device memory that must not overlap the
 * sources.  Enqueued on cfg->stream; cfg->weight_layout is not read.  Pack
 * once, then pass W1p, W3p, W2p to moe_forward with weight_layout PACKED.
 * MOE_EUNSUPPORTED for fp32 layers, MOE_EINVAL for a NULL pointer. */
int moe_pack_weights(const void* W1, const void* W3, const void* W2, const moe_config_t* cfg,
                     void* W1p, void* W3p, void* W2p);

/* Capacity C for cfg: ceil(T*k*cf/E) with cf read as the shortest decimal
 * that round-trips the double (1.1 means 11/10), or T without a limit.
 * [Routing guide] "Plain explanation" para 5.  -1 when cfg is invalid. */
int64_t moe_capacity(const moe_config_t* cfg);

/* Full layer forward, steps 1-5 (and 6 when stats != NULL).
 *   x [T, d], W_gate [d, E], W1/W3 [E+S, d, F], W2 [E+S, F, d]: inputs
 *   (W1, W3, W2 in cfg->weight_layout: row-major or packed),
 *   out [T, d]: output in cfg->dtype (fp32 when cfg->out_fp32), fully
 *   overwritten.  stats: host struct or NULL.
 * Precision of bf16 layers: products of bf16 values summed in fp32; the
 * hidden rows silu(u) * v are rounded to bf16 once before the down
 * projection; expert rows, gate weights and the weighted sum stay fp32 up to
 * the output, which is rounded once (or not, with out_fp32). */
int moe_forward(const void* x, const void* W_gate, const void* W1,
                const void* W3, const void* W2, const moe_config_t* cfg,
                void* out, moe_stats_t* stats);

/* moe_forward for callers that cannot allocate device memory or bring a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, kernels and results (bit for bit)
 * as moe_forward; cfg->workspace and cfg->workspace_bytes are ignored.
 * Scratch is a fixed 64 MiB array in device memory (67108864 bytes), one per
 * GPU the library runs on, kept until the process ends; its address is
 * looked up on the first call on each device.  A layer whose
 * moe_workspace_size(cfg) exceeds it is refused with MOE_EWORKSPACE before
 * anything is enqueued (e.g. the Mixtral shape up to T = 256 tokens and the
 * 160-expert DeepSeek shape up to T = 64 fit).  Nothing is allocated and,
 * with stats == NULL, nothing but kernels is enqueued.  The kernels write
 * every scratch byte they read, so nothing needs clearing between calls.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (other streams, other threads) race and must be
 * serialised by the caller; moe_router_backward cannot follow this entry
 * point (it needs the forward's workspace). */
int moe_forward_noalloc(const void* x, const void* W_gate, const void* W1,
                        const void* W3, const void* W2, const moe_config_t* cfg,
                        void* out, moe_stats_t* stats);

/* Steps 1-3 (and 6 when stats != NULL): router scores, top-k, gates and
 * dispatch, without the experts.  Outputs (device, caller-owned):
 *   logits   [T, E] fp32  scores seen by top-k (bias included)
 *   topk_idx [T, k] int32 chosen experts, best first
 *   topk_w   [T, k] fp32  gate weights
 *   counts   [E]    int32 assignments per expert before drops
 *   offsets  [E+1]  int32 exclusive prefix sum of kept counts
 *   perm     [T*k]  int32 perm[s] = assignment a = t*k + j held in slot s;
 *                          entries at and after offsets[E] are -1
 *   slot     [T*k]  int32 slot of assignment a, or -1 when dropped; the
 *                          expert that processes it is the e with
 *                          offsets[e] <= slot < offsets[e+1]
 * Any output pointer except topk_idx may be NULL to skip it. */
int moe_route(const void* x, const void* W_gate, const moe_config_t* cfg,
              float* logits, int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets, int32_t* perm,
              int32_t* slot, moe_stats_t* stats);

/* Steps 2-3 (and 6) from caller-supplied router scores logits [T, E] fp32
 * (device), which must already include any bias: cfg->logit_bias must be
 * NULL (MOE_EINVAL otherwise).  Outputs as for moe_route. */
int moe_route_logits(const float* logits, const moe_config_t* cfg,
                     int32_t* topk_idx, float* topk_w, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* slot,
                     moe_stats_t* stats);

/* Step 6's auxiliary load-balancing value alone, E * sum_i f_i P_i, from
 * router scores logits [T, E] fp32 and pre-drop counts [E] int32 (both
 * device).  Uses cfg's T, E, k, stream and workspace; waits for the stream
 * and writes the value to *aux_out (host).  [Routing guide] "Plain
 * explanation" para 4. */
int moe_aux_loss(const float* logits, const int32_t* counts,
                 const moe_config_t* cfg, double* aux_out);

/* Router backward, after moe_forward.  Gradients of
 *   L = sum(dout * out) + aux_coef * aux + entropy_coef * H_tok
 * with respect to the router (H_tok: the mean router entropy, the quantity a
 * training schedule raises early and lowers later, [Routing guide] "Plain
 * explanation" para 4): the gate weights move through their softmax,
 * so in the softmax-over-all order (DeepSeek, not renormalised) every
 * expert's score receives gradient, chosen or not; aux = E sum f_i P_i moves
 * through P_i with the load fractions f_i held fixed, as are the top-k
 * choices and the capacity decisions.  [Routing guide] "Plain explanation"
 * paras 2 and 4.
 *   dw[t,j]       = dout[t] . y[t,j] for an assignment an expert ran, else 0
 *   softmax over the k chosen (Mixtral, or DeepSeek renormalised):
 *       dlogits[t, c_j] = w_j (dw_j - sum_i w_i dw_i), 0 at other experts
 *   softmax over all E read at the chosen ones:
 *       dlogits[t, i]   = p_i (G_i - sum_j w_j dw_j), G_i = dw_j at i = c_j
 *   + aux_coef (E/T) p_i (f_i - sum_m f_m p_m),  f_i = counts_i / (T k)
 *   + entropy_coef (1/T) (-p_i (ln p_i + H_t)),  H_t = -sum_m p_m ln p_m
 *   dW_gate = x^T dlogits, dbias = sum_t dlogits[t], dx = dlogits W_gate^T
 * Must follow moe_forward on the same stream with the same cfg, inputs and
 * workspace, with no other call using that workspace in between: the
 * forward leaves its scores, choices, gates, slots, counts and expert output
 * rows there.  Arguments (device):
 *   x [T, d], W_gate [d, E]  the forward's inputs (x needed for dW_gate,
 *                            W_gate for dx; otherwise may be NULL)
 *   dout     [T, d]  cfg->dtype, gradient of L with respect to out
 *   dlogits  [T, E]  fp32 out (required)
 *   dW_gate  [d, E]  fp32 out, or NULL
 *   dbias    [E]     fp32 out, or NULL (gradient of the score bias)
 *   dx       [T, d]  fp32 out, or NULL: the router's share of dL/dx only
 * Enqueued on cfg->stream; sums run in a fixed order (bitwise reproducible). */
int moe_router_backward(const void* x, const void* W_gate, const void* dout,
                        double aux_coef, double entropy_coef,
                        const moe_config_t* cfg, float* dlogits,
                        float* dW_gate, float* dbias, float* dx);

/* Training side of the router ([Routing guide] "Plain explanation" para 4:
 * the router's entropy is kept high early in training, so tokens try many
 * experts, and lowered later; "Key insights" item 3: the trend of the
 * load-balancing loss is one of the quantities to watch).  Host only: no
 * GPU is touched.
 *
 * moe_entropy_coef: the weight of the mean router entropy H_tok in the loss
 * (the entropy_coef of moe_router_backward) at `step` of `total_steps`:
 * `high` at step 0, falling in a straight line to `low` at step
 * total_steps - 1, held at `high` before and at `low` after; `low` when
 * total_steps <= 1.  The pages give the direction only; the straight line
 * is the plainest shape with it.  NaN for non-finite high or low. */
double moe_entropy_coef(int64_t step, int64_t total_steps, double high, double low);

/* moe_lb_trend: trend of a series of load-balancing losses (the aux_loss
 * of successive forward calls, oldest first; host array of n values):
 * *slope = the least-squares slope of value against step number, per step
 * (sum (i - i_mean)(v_i - v_mean) / sum (i - i_mean)^2), *mean = the mean
 * value.  Negative while the load evens out, near 0 once it has settled.
 * MOE_EINVAL for n < 2, a NULL pointer or a non-finite value (outputs
 * untouched). */
int moe_lb_trend(const double* values, int64_t n, double* slope, double* mean);

/* Debugging aid: workspace canaries.  While enabled (process-wide), the
 * workspace plan puts a 256-byte guard after every region (so
 * moe_workspace_size grows by a few KB; size the workspace after enabling),
 * and every call that uses the workspace first fills the guards with 0xA5
 * (hipMemsetAsync: not for graph capture).  moe_debug_check(cfg) waits for
 * cfg->stream and returns how many guards of cfg->workspace no longer hold
 * the pattern (0: none; moe_last_error names the region before the first
 * overwritten guard), or a negative status.  Off by default. */
int moe_debug_canaries(int enable);
int moe_debug_check(const moe_config_t* cfg);

/* Reason for the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* Per-kernel timing for measurement.  While enabled, every kernel the
 * library launches is bracketed by HIP events on cfg->stream.
 * moe_timing_read waits for those events and returns, for each kernel name,
 * the number of launches and the summed duration in milliseconds since the
 * last reset; names is filled with up to max entries of NUL-terminated
 * names (each at most 63 chars) in a caller buffer of max*64 bytes.
 * Returns the number of distinct kernels (may exceed max). */
int moe_timing_enable(int enable);
/* Restricts timing to the named kernels: a comma-separated list of the names
 * moe_timing_read reports (e.g. "ffn1_swiglu"); NULL or "" times every
 * kernel again.  Each timed kernel adds two event records to the stream, so
 * timing one kernel perturbs the step less than timing all of them. */
int moe_timing_only(const char* names);
int moe_timing_reset(void);
int moe_timing_read(char* names, int64_t* launches, double* total_ms,
                    int max);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
