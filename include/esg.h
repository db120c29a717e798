/*
 * esg.h -- C ABI of the group-sparse SwiGLU feed-forward layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The operations are the ones the eugen_sparse README ("eugen_sparse --
 * sparse SwiGLU FFN in Triton") lists under "What it does": the subsample of
 * gate rows, the grouped top-k selection, the sparse SwiGLU forward and its
 * gradients, and the load-balance bias update; plus the CSR bucketing the
 * same page's "Pitfalls and limitations" section names as a deterministic
 * internal step.  Shape rules follow that page's "Parameters and how to
 * choose them" table.
 *
 * Conventions for every entry point:
 *  - Returns an esg status code (ESG_OK = 0).  Argument and shape errors are
 *    reported before anything is enqueued.
 *  - Device pointers are plain HIP device addresses of contiguous row-major
 *    buffers, 16-byte aligned.  Weights use nn.Linear layout: w_gate and w_up
 *    are [d_ff, d_model], w_down is [d_model, d_ff].  Group g owns neurons
 *    [g*group_size, (g+1)*group_size): rows of w_gate / w_up, columns of
 *    w_down.
 *  - The caller owns every buffer.  The library allocates no device memory and
 *    keeps no state between calls (apart from the optional per-thread kernel
 *    timing below); all scratch comes from caller buffers whose sizes the
 *    *_workspace_size calls give.  Every launch goes to `stream`: the library
 *    creates no stream and no event of its own outside timing.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    nothing synchronises.  Calls on one stream are ordered.
 *  - dtype is ESG_F32 or ESG_BF16 for x, dy, the weights and the outputs
 *    (y, dx, dW).  Group ids and counts are int32; bias, EMA and frequencies
 *    are float32.  Accumulation is float32 in every contraction.
 *  - tokens * k must stay below 2^31 (int32 positions).
 */
#ifndef ESG_H
#define ESG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ESG_OK 0
#define ESG_ERR_INVALID_ARG 1   /* null pointer, misaligned pointer, negative size */
#define ESG_ERR_UNSUPPORTED 2   /* a shape rule is violated or the dtype is unknown */
#define ESG_ERR_WORKSPACE 3     /* a workspace buffer is smaller than required */
#define ESG_ERR_HIP 4           /* a HIP runtime call failed */

/* dtypes */
#define ESG_F32 0
#define ESG_BF16 1

/* bits OR-ed into the optional device status word by the bucketing pass */
#define ESG_STATUS_GROUP_OUT_OF_RANGE 1   /* an id < 0 or >= G was skipped */
#define ESG_STATUS_GROUP_DUPLICATE 2      /* a repeated id in one token was skipped */

/* Human-readable name of a status code (static string). */
const char* esg_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int esg_version(void);

/*
 * Fixed random subset of gate rows per group (eugen_sparse README, "What it
 * does", make_subsample_index; drawn once per layer and kept with the model,
 * "Pitfalls and limitations").
 *
 * Host only.  Writes G*samples_per_group int32 absolute w_gate row ids to the
 * HOST buffer `out` (G = d_ff/group_size): group by group, ascending within a
 * group, each group's ids inside its own row range.  The draw: one SplitMix64
 * stream seeded with `seed`; per group, a partial Fisher-Yates shuffle of
 * 0..group_size-1 with draw i taking (next() mod (group_size-i)) as the swap
 * offset; the first samples_per_group ids are kept.  Deterministic per seed.
 * Errors: ESG_ERR_INVALID_ARG (out NULL), ESG_ERR_UNSUPPORTED (shape rules, or
 * samples_per_group outside 1..group_size).
 */
int esg_make_subsample_index(int d_ff, int group_size, int samples_per_group, uint64_t seed,
                             int32_t* out);

/*
 * Grouped top-k selection (eugen_sparse README, "What it does",
 * grouped_topk_select).  For every token t:
 *   E[t,g] = sum over the group's gate rows r of |SiLU(x[t] . w_gate[r])|,
 *   the rows being sub[g*spg .. g*spg+spg) when `sub` is given, else all
 *   group_size rows of group g;
 *   s[t,g] = E[t,g] + bias[g] (bias may be NULL = 0; selection only);
 *   idx[t, 0..k) = the k groups with the largest s, equal scores ordered by
 *   ascending group id, written in ascending group id.
 * x: [tokens, d_model] dtype; w_gate: [d_ff, d_model] dtype; sub: device
 * int32 [G*spg] or NULL (then spg is ignored); bias: device float [G] or NULL;
 * idx_out: device int32 [tokens, k]; counts_out: device int32 [G] or NULL --
 * overwritten with the number of tokens that selected each group.
 * The energy is accumulated in float32; the ranking uses float32 scores.
 * No gradient.  Constraints: G <= 1024.
 */
int esg_grouped_topk_select(const void* x, const void* w_gate, int dtype, int tokens, int d_model,
                            int d_ff, int group_size, int k, const int32_t* sub, int samples_per_group,
                            const float* bias, int32_t* idx_out, int32_t* counts_out, void* stream);

/*
 * The same selection (same definition as above, bitwise the same idx_out and
 * counts_out) with a device workspace of at least
 * esg_grouped_topk_select_workspace_size() bytes (16-byte aligned; the
 * library's use of it ends with the call's work on `stream`).  Batches too
 * small to give every CU a 32-token workgroup then spread each token block's
 * groups over several workgroups, which write an fp32 [tokens, G] energy
 * table there, and rank in a second launch (decode-sized batches).  A NULL or
 * too small workspace selects exactly as esg_grouped_topk_select.
 * Errors as esg_grouped_topk_select; ESG_ERR_INVALID_ARG for a misaligned
 * workspace.
 */
int esg_grouped_topk_select_workspace_size(int tokens, int d_ff, int group_size, size_t* workspace_bytes);
int esg_grouped_topk_select_ws(const void* x, const void* w_gate, int dtype, int tokens, int d_model,
                               int d_ff, int group_size, int k, const int32_t* sub, int samples_per_group,
                               const float* bias, int32_t* idx_out, int32_t* counts_out, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Deterministic CSR bucketing of routed (token, slot) pairs by group (the
 * eugen_sparse README, "Pitfalls and limitations", states that the CSR
 * bucketing is deterministic).  Pairs are ordered by (group, token):
 *   offsets[G+1]      exclusive prefix sums of the per-group counts;
 *   perm_token[T*k]   the token at each bucket position;
 *   inv[T*k]          the bucket position of pair (t, j) at t*k+j.
 * Ids outside [0, G) and repeats of an id within a token are skipped: their
 * inv entry is -1, they are not counted, and the matching ESG_STATUS_* bit is
 * OR-ed into *status_dev (device int32, may be NULL; never cleared here).
 * With skipped pairs, perm_token holds offsets[G] valid entries.
 * scratch: device buffer of esg_bucket_workspace_size() bytes.
 */
int esg_bucket_workspace_size(int tokens, int k, int groups, size_t* scratch_bytes);
int esg_bucket_by_group(const int32_t* idx, int tokens, int k, int groups, int32_t* offsets,
                        int32_t* perm_token, int32_t* inv, int32_t* status_dev, void* scratch,
                        size_t scratch_bytes, void* stream);

/*
 * Workspace sizes for the FFN.  `saved` is written by the forward and read by
 * the backward of the same call pair (routing in CSR form and the compact
 * gate/up pre-activations of the selected groups); it must not change in
 * between.  `fwd_scratch` and `bwd_scratch` are free between calls.  dense=1
 * sizes the all-groups-active path (idx = NULL, k must equal G): it saves
 * nothing and its forward needs no scratch; its backward scratch holds the
 * recomputed dg, du, a of one chunk of at most 8192 tokens (3 * 2 bytes per
 * neuron per token) plus, when there is more than one chunk, float32
 * accumulators for the three weight gradients.  fwd_scratch is what a
 * forward with `saved` needs; a forward with saved = NULL needs at most that
 * (bf16 training layouts with 128-neuron blocks pad each group's bucket to a
 * whole pair of 128-position tiles for the backward; inference pads to one
 * tile).  The routed backward's scratch holds dg, du and a of every bucket
 * position, the bf16 partial rows of dx and, for bf16 128-neuron blocks whose
 * buckets could exceed 1.5 times the mean, float32 slots for the weight
 * gradients of such buckets summed in chunks.  Errors: as for the forward;
 * ESG_ERR_UNSUPPORTED for a dense shape the dense kernels do not cover.
 */
int esg_sparse_swiglu_workspace_size(int tokens, int d_model, int d_ff, int group_size, int k,
                                     int dtype, int dense, size_t* saved_bytes,
                                     size_t* fwd_scratch_bytes, size_t* bwd_scratch_bytes);

/*
 * Forward (eugen_sparse README, "What it does", sparse_swiglu_ffn):
 *   y[t] = sum over g in idx[t] of (SiLU(x[t] W_gate[g]^T) * (x[t] W_up[g]^T)) W_down[:,g]^T
 * x: [tokens, d_model]; idx: device int32 [tokens, k] (distinct ids per token;
 * see esg_bucket_by_group for what happens otherwise); y: [tokens, d_model]
 * overwritten.  The gated activation of a group never leaves the chip; the k
 * per-token contributions are written as partial rows and summed in slot order
 * in float32 without atomics, so the result is bitwise reproducible.
 * status_dev: as in esg_bucket_by_group.
 * saved = NULL selects inference (forward only): nothing is kept for a
 * backward, the routing is held in the scratch instead (fwd_scratch_bytes
 * covers it), and y is bitwise the same as with saved given.
 *
 * Dense limit: idx = NULL with k = G means every group is active, i.e. the
 * plain SwiGLU block (the README's layer with all groups selected).  It runs
 * a fused kernel in which the [tokens, d_ff] intermediate never exists in
 * device memory (forward only: the dense backward below recomputes gate/up
 * and holds dg, du, a of one token chunk in its scratch); saved and scratch
 * are unused (may be NULL).  Supported for
 * bf16 with d_model <= 2048; other dense shapes return ESG_ERR_UNSUPPORTED,
 * and k != G with idx = NULL returns ESG_ERR_INVALID_ARG.
 */
int esg_sparse_swiglu_fwd(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                          int dtype, int tokens, int d_model, int d_ff, int group_size, int k,
                          const int32_t* idx, void* y, void* saved, size_t saved_bytes, void* scratch,
                          size_t scratch_bytes, int32_t* status_dev, void* stream);

/*
 * The inference forward (the call above with saved = NULL) for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no scratch argument: its
 * scratch is a device array of ESG_NOALLOC_SCRATCH_BYTES (128 MiB) built into
 * the library, one per device the library runs on, held until the process
 * ends.  Arguments and results are those of esg_sparse_swiglu_fwd with
 * saved = NULL; y is bitwise the same.  Shapes whose inference-forward
 * scratch exceeds ESG_NOALLOC_SCRATCH_BYTES return ESG_ERR_WORKSPACE before
 * anything is enqueued (every batch from 1 to 2482 tokens fits at the 1.3B
 * shape, k = 11 of 43 groups of 128; 1 to 10355 at the 128M shape, k = 8 of
 * 32 groups of 64: decode and short prefill batches).  It calls no allocator.
 * All calls on one device share that device's array, so calls that overlap
 * on one device (concurrent streams or threads) race; calls ordered on one
 * stream do not.  The first call on a device looks up the array's device
 * address (hipGetSymbolAddress) with that device current; ESG_ERR_HIP if that
 * fails.
 */
#define ESG_NOALLOC_SCRATCH_BYTES (128u << 20)
int esg_sparse_swiglu_fwd_noalloc(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                                  int dtype, int tokens, int d_model, int d_ff, int group_size, int k,
                                  const int32_t* idx, void* y, int32_t* status_dev, void* stream);

/*
 * Backward of the forward above with the routing held fixed (hard top-k: the
 * README's pitfalls note that only selected groups receive weight gradients
 * and the routing gets none).  With A = SiLU(Hg)*Hu on the selected groups:
 *   dA = dy W_down (selected groups), dHu = dA*SiLU(Hg),
 *   dHg = dA*Hu*SiLU'(Hg), dx = dHg W_gate + dHu W_up,
 *   dW_gate = dHg^T x, dW_up = dHu^T x, dW_down = dy^T A.
 * dy, dx: [tokens, d_model]; dw_gate, dw_up: [d_ff, d_model]; dw_down:
 * [d_model, d_ff]; all overwritten (not accumulated).  Rows/columns of groups
 * that no token selected are written as exact zeros.  `saved` and `idx` must
 * be those of the matching forward call.  No atomics: bitwise reproducible.
 * Dense limit (idx = NULL, k = G): the gate/up pre-activations are recomputed
 * per token chunk (the forward saved nothing; `saved` is unused and may be
 * NULL); the weight gradients are summed over chunks in float32 in chunk
 * order.  Same support rules as the dense forward.
 */
int esg_sparse_swiglu_bwd(const void* dy, const void* x, const void* w_gate, const void* w_up,
                          const void* w_down, int dtype, int tokens, int d_model, int d_ff,
                          int group_size, int k, const int32_t* idx, const void* saved,
                          size_t saved_bytes, void* dx, void* dw_gate, void* dw_up, void* dw_down,
                          void* scratch, size_t scratch_bytes, void* stream);
/*
 * The same backward with a caller-owned second stream: for the routed path,
 * after dh and the dx partials, the weight gradients run on aux_stream while
 * the slot-order sum of dx runs on `stream`; aux_stream waits for `stream`
 * first and `stream` waits for aux_stream at the end (two events created and
 * destroyed inside the call), so on return every result is ordered on
 * `stream` as with esg_sparse_swiglu_bwd.  aux_stream NULL or equal to
 * `stream`: identical to esg_sparse_swiglu_bwd.  Works under stream capture
 * (the event pair forks and joins the captured stream).  Results are bitwise
 * the same either way.
 */
int esg_sparse_swiglu_bwd_overlap(const void* dy, const void* x, const void* w_gate, const void* w_up,
                                  const void* w_down, int dtype, int tokens, int d_model, int d_ff,
                                  int group_size, int k, const int32_t* idx, const void* saved,
                                  size_t saved_bytes, void* dx, void* dw_gate, void* dw_up, void* dw_down,
                                  void* scratch, size_t scratch_bytes, void* stream, void* aux_stream);

/*
 * Load-balance bias update (eugen_sparse README, "What it does",
 * update_load_balance_bias; constants in "Parameters and how to choose
 * them"), once per optimizer step, in place on device float32 [groups]:
 *   ema  <- ema + (1 - momentum) * (current_freq - ema)
 *   bias <- clamp(bias + gamma * sign(target_freq - ema), -bias_max, bias_max)
 * with sign(0) = 0, computed in float32 without fused multiply-add.
 * current_freq[g] is the fraction of tokens that chose group g in the step
 * (it sums to k); target_freq is normally k / G.
 * The _from_counts form takes the int32 per-group counts of a selection call
 * and the token count, and uses current_freq = counts / tokens.
 */
int esg_update_load_balance_bias(float* bias, float* freq_ema, const float* current_freq,
                                 float target_freq, float gamma, float bias_max, float momentum,
                                 int groups, void* stream);
int esg_update_load_balance_bias_from_counts(float* bias, float* freq_ema, const int32_t* counts,
                                             int tokens, float target_freq, float gamma,
                                             float bias_max, float momentum, int groups,
                                             void* stream);

/*
 * The same update with the counts taken from the routing a training forward
 * stored in `saved` (esg_sparse_swiglu_fwd with a non-NULL `saved`): its CSR
 * group offsets give count[g] = offsets[g+1] - offsets[g], the number of valid
 * (token, group) pairs routed to g, equal to the selection's counts when the
 * routing came from esg_grouped_topk_select.  A training step that updates the
 * bias can then select without counts (no counts fill, no count atomics).
 * Shape arguments as given to that forward; saved_bytes at least its
 * saved size.  Errors: ESG_ERR_INVALID_ARG (NULL pointers, tokens <= 0),
 * ESG_ERR_UNSUPPORTED (shape rules), ESG_ERR_WORKSPACE (saved too small).
 */
int esg_update_load_balance_bias_from_routing(float* bias, float* freq_ema, const void* saved, size_t saved_bytes,
                                              int tokens, int d_model, int d_ff, int group_size, int k, int dtype,
                                              float target_freq, float gamma, float bias_max, float momentum,
                                              void* stream);

/*
 * LeakyReLU(0.5)-squared MLP with a stored activation gradient (parameter-golf
 * pull request 1105, "1. Fused MLP Kernels"; architecture table A.7: d_model
 * 512, width 3.5 x 512 = 1792).  bf16 tensors, fp32 accumulation:
 *   forward   pre = x . W_up^T (not stored);
 *             act_grad = 2*pre if pre > 0 else 0.5*pre;
 *             post = 0.5 * act_grad * pre     (= LeakyReLU(0.5)(pre)^2);
 *             y = post . W_down^T
 *   backward  dpre = (dy . W_down) * act_grad  (the product fused into the
 *             GEMM epilogue); dx = dpre . W_up; dW_up = dpre^T . x;
 *             dW_down = dy^T . post
 * post and act_grad are computed from the fp32 pre and rounded once to bf16;
 * dpre is rounded to bf16 before its two products.  The weight gradients are
 * deterministic: token splits add their fp32 partials in a fixed order.
 *
 * x, y, dy, dx: device bf16 [tokens, d_model]; w_up, dw_up: [d_ff, d_model];
 * w_down, dw_down: [d_model, d_ff] (nn.Linear layout).  The gradients are
 * overwritten (tokens == 0 writes zero weight gradients).
 * saved: device buffer of saved_bytes holding post then act_grad ([tokens,
 * d_ff] bf16 each, 256-byte aligned), written by the forward for the backward.
 * scratch: device buffer of scratch_bytes for the backward (dpre and the fp32
 * partials of the weight gradients).
 * Errors: ESG_ERR_INVALID_ARG (null pointer, negative size),
 * ESG_ERR_UNSUPPORTED (d_model or d_ff not a multiple of 8, or a tensor of
 * 2^31 bytes or more), ESG_ERR_WORKSPACE (a buffer below its size).
 */
int esg_leaky_mlp_workspace_size(int tokens, int d_model, int d_ff, size_t* saved_bytes, size_t* scratch_bytes);
int esg_leaky_mlp_fwd(const void* x, const void* w_up, const void* w_down, int tokens, int d_model, int d_ff,
                      void* y, void* saved, size_t saved_bytes, void* stream);
int esg_leaky_mlp_bwd(const void* dy, const void* x, const void* w_up, const void* w_down, int tokens, int d_model,
                      int d_ff, const void* saved, void* dx, void* dw_up, void* dw_down, void* scratch,
                      size_t scratch_bytes, void* stream);

/*
 * Multi-head sub-network FFN core of FlashFFN (FlashFFN README, "Overview" and
 * "Model configurations"): for every token t and head h,
 *   O[t,h] = sum_e R[t,h,e] * ((SiLU(Q[t,h] K[h,e]^T) * (Q[t,h] U[h,e]^T)) V[h,e])
 * with per-head sub-networks K, U, V of shape [d_sub, d_head] each.  The fused
 * forward keeps the [d_sub] intermediate and the fp32 [d_head] output
 * accumulator on chip; the intermediate, scaled by R, is rounded to bf16
 * before its product with V.
 * q, out: device bf16 [tokens, heads, d_head]; r: device float [tokens, heads,
 * subnets]; k, u, v: device bf16 [heads, subnets, d_sub, d_head].  Q is the
 * caller's (normalised) head input and R its router weights; producing them,
 * and the projections around the core, are not part of this call.
 * out is overwritten; tokens == 0 enqueues nothing.
 * esg_mhffn_supported returns 1 when d_head == 128, d_sub is a multiple of 8,
 * subnets <= 32 and every tensor is below 2^31 bytes, else 0.
 * Errors: ESG_ERR_INVALID_ARG (null or misaligned pointer, negative size),
 * ESG_ERR_UNSUPPORTED (shape outside esg_mhffn_supported).
 */
int esg_mhffn_supported(int tokens, int heads, int d_head, int subnets, int d_sub);
int esg_mhffn_fwd(const void* q, const float* r, const void* k, const void* u, const void* v, int tokens, int heads,
                  int d_head, int subnets, int d_sub, void* out, void* stream);
/*
 * Gradients of the same core given dout = dL/dO [tokens, heads, d_head]
 * (bf16): dq (bf16, like q), dr (float, like r), dk, du, dv (bf16, like k).
 * All are overwritten (tokens == 0: dk, du, dv zero, nothing else written).
 * Nothing is saved by the forward: both backward kernels recompute the
 * sub-networks' pre-activations.  Per token t, head h, sub-network e, with
 * a = SiLU(h1) h2 and g = dO V^T: dR = sum_n a g; da = R g; dh2 = da SiLU(h1);
 * dh1 = da h2 SiLU'(h1); dQ = sum_e (dh1 K + dh2 U); dK = dh1^T Q;
 * dU = dh2^T Q; dV = (R a)^T dO.  dh1, dh2 and R a are rounded to bf16 before
 * their products; sums over tokens and sub-networks run in fp32 in a fixed
 * order (deterministic).  Same shape rules and errors as esg_mhffn_fwd.
 */
int esg_mhffn_bwd(const void* dout, const void* q, const float* r, const void* k, const void* u, const void* v,
                  int tokens, int heads, int d_head, int subnets, int d_sub, void* dq, float* dr, void* dk, void* du,
                  void* dv, void* stream);

/*
 * Sigmoid top-k routing with an expert bias (Megatron-Core developer guide,
 * "core.inference.moe.sigmoid_topk": the description of _sigmoid_topk_kernel
 * and the API of sigmoid_topk_routing).  Per token row t and expert e:
 *   s[t,e]   = sigmoid(logits[t,e]), the fp64 value rounded once to fp32;
 *   key[t,e] = s[t,e] + expert_bias[e * bias_stride]   (one fp32 addition).
 * The row's k-th largest key is taken in the total order of fp32 values
 * (-0.0 below +0.0); indices[t] lists the experts whose key is above it in
 * ascending expert order, then the experts whose key equals it in ascending
 * order, k in all.  The weights use the unbiased scores:
 *   probs[t,j] = s[t,i_j] / ((((s_0 + s_1) + s_2) + ...) + 1e-20f),
 * the sum folded left in output order, then times scaling_factor if
 * apply_scaling != 0; every operation is a separately rounded fp32 one.
 * The bias serves the selection only.  Rows are independent and the launch
 * does not depend on `tokens`, so each row's result is independent of the
 * batch (bitwise).
 *
 * logits: device float [tokens, num_experts] row-major (finite values);
 * expert_bias: device float, element e at expert_bias[e * bias_stride]
 * (bias_stride >= 1; finite values); probs: device float [tokens, topk];
 * indices: device int64 [tokens, topk].  Both outputs are overwritten.
 * tokens == 0 enqueues nothing.
 * Errors: ESG_ERR_INVALID_ARG (null pointer with tokens > 0, tokens < 0,
 * bias_stride < 1), ESG_ERR_UNSUPPORTED (shape outside
 * esg_sigmoid_topk_supported, or tokens * topk >= 2^31).
 * esg_sigmoid_topk_supported returns 1 when 1 <= topk <= min(32,
 * num_experts) and num_experts <= 2048, else 0.
 */
int esg_sigmoid_topk_supported(int num_experts, int topk);
int esg_sigmoid_topk_routing(const float* logits, const float* expert_bias, int bias_stride, int tokens,
                             int num_experts, int topk, float scaling_factor, int apply_scaling, float* probs,
                             int64_t* indices, void* stream);

/*
 * Measurement helper (not part of the method): a rate probe of the bf16
 * matrix cores.  Launches `blocks` workgroups of 256 threads on `stream`;
 * every wavefront runs `iters` rounds of eight independent
 * v_mfma_f32_16x16x32_bf16 on register operands, i.e.
 * blocks * 4 * iters * 8 * 16384 FLOPs with no memory traffic, and writes
 * one float per thread to `out` (device, blocks * 256 floats, caller-owned).
 * Time it with events on `stream` to measure the achievable MFMA peak.
 * Returns ESG_ERR_INVALID_ARG for blocks or iters < 1 or out NULL.
 */
int esg_mfma_rate_probe(int blocks, int iters, float* out, void* stream);

/*
 * Kernel timing (instrumentation, off by default).  When enabled, every
 * kernel the library launches from the calling host thread is bracketed by
 * HIP events recorded on its launch stream.  esg_timing_read synchronises on
 * the recorded events and returns the summed duration in milliseconds and the
 * launch count of the kernel named `kernel` since the last reset.  The state
 * (on/off flag, recorded events) belongs to the calling host thread: threads
 * time their own launches independently, and a thread that never enables
 * timing pays one flag test per launch.
 */
int esg_timing_enable(int on);
int esg_timing_reset(void);
int esg_timing_read(const char* kernel, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* ESG_H */
