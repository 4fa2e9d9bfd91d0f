/*
 * gdn_hybrid.h -- C ABI of the MI355X (gfx950) hybrid attention layer:
 * a gated delta-rule (GDN) linear recurrence over the tokens outside a fixed
 * cache budget, plus softmax attention over sink tokens and a sliding window,
 * the two outputs summed; with the GLA diagonal-gate variant and the fused
 * RoPE -> short conv -> L2 norm preparation of Q/K/V.
 *
 * Sources (cited by page title and section):
 *   [P1] "The Key to Going Linear: Analysis-Driven Transformer Linearization"
 *        (summary page of arXiv 2607.07706v1):
 *        - 线性注意力替换机制: the GLA update S_t = G_t S_{t-1} + k_t v_t^T and
 *          the GDN update S_t = (I - b_t k_t k_t^T) G_t S_{t-1} + b_t k_t v_t^T;
 *        - 从 softmax 到 delta 规则的一阶近似: softmax logits q.k / sqrt(d);
 *        - 填补近似缺口的实用设计: budget = 8 sinks (always attended) + a
 *          sliding window; the linear path covers all other tokens;
 *        - 实践建议 items 2-3: fixed budget split; kernel-8 short conv on
 *          Q/K/V after RoPE and before L2 normalisation.
 *   [P2] "線性化 Transformer 但不掉品質", section 方法到底怎麼做: sink tokens,
 *        short convolutions, fixed-budget cache routing.
 *   [P3] "Untangling Component Imbalance in Hybrid Linear Attention
 *        Conversion Methods", section 核心思路: the hybrid combines a linear
 *        branch with sliding-window softmax; linear-only / softmax-only use.
 *
 * Definitions used by every entry point (positions t are 0-based, budget
 * N = n_sink + window, G = H / Hkv, query head h reads KV head h / G):
 *   softmax set  A(t) = { i <= t : i < n_sink or i > t - window }
 *   linear set   L(t) = { i : n_sink <= i <= t - window }
 *   GDN  (per query head, a_i and b_i scalars):
 *        S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T,  i >= n_sink
 *   GLA  (alpha_i a d_k-vector in (0,1)): S_i = Diag(alpha_i) S_{i-1} + k_i v_i^T
 *   o_lin[t] = S_{t-window}^T q_t   (0 while t - window < n_sink)
 *   o_swa[t] = sum_{i in A(t)} softmax_i(q_t . k_i / sqrt(d_k)) v_i
 *   o[t]     = o_lin[t] + o_swa[t]            (a plain sum)
 * S is d_k x d_v (column-vector convention); the state starts at zero.
 *
 * Conventions of all calls:
 *   - Every pointer is a DEVICE pointer owned by the caller; the library never
 *     allocates, frees or retains it, and never synchronises.
 *   - Tensors are dense, row-major (last index fastest), in the layouts given.
 *     Outputs must not alias inputs.  Every tensor pointer is 16-byte aligned
 *     (GDN_EINVAL otherwise): the kernels move rows in 16-byte pieces.
 *   - q/k/v/o and the K/V cache use `dtype` (GDN_F32 or GDN_BF16); gates a, b
 *     and states are always fp32.  d_k = d_v = d in {64, 128}.
 *   - `stream` is a hipStream_t (NULL: the null stream).  Calls are
 *     asynchronous on it.
 *   - Arguments are validated on the host before anything is launched; on an
 *     error nothing is launched and no output is touched.  Return values:
 *     GDN_OK, GDN_EINVAL (bad pointer/shape/flag), GDN_EUNSUPPORTED (valid
 *     but not implemented, e.g. fp32 linear branch at d = 128),
 *     GDN_EWORKSPACE (workspace too small), GDN_ELAUNCH (the HIP launch
 *     failed; hipGetLastError() is reported through gdn_hybrid_last_hip_error).
 *   - Preconditions the caller guarantees (not checked): keys and queries of
 *     the GDN path are L2-normalised (or come from shortconv_qkv); a in (0,1],
 *     b in [0,1]; decode positions pos[b] >= 0 and the cache/state hold the
 *     sequence's prefix up to pos[b] - 1.
 *   - No global mutable state besides the last HIP error code and the
 *     test-only fault setting below: calls are thread-safe as far as HIP
 *     launches are.
 *   - Waits inside a launch: the one-launch few-chain prefill (see
 *     gdn_hybrid_prefill_workspace) hands each chunk from preparation
 *     workgroups to scan workgroups, and the scan's rows to softmax
 *     workgroups, through flags in the workspace.  Every such wait is on
 *     workgroups earlier in the grid (dispatched in order, so already
 *     resident) and is bounded in time (0.1 s by default).  If a bound ever
 *     expires (e.g. another workload starves the producers), the rows and
 *     states computed from the missing data are written as NaN, never as
 *     silently wrong values.
 */
#ifndef GDN_HYBRID_H
#define GDN_HYBRID_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;
/* recurrence of the linear branch (page "The Key to Going Linear", section
   线性注意力替换机制): GDN_DELTA the gated delta rule with one scalar gate
   a_t per token and head; GDN_GLA the diagonal-gate linear update; and
   GDN_DELTA_DIAG the delta rule with the diagonal gate,
   S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1} + b_t k_t v_t^T, whose
   gates are per channel (a [.., dk], as GLA) and b per token and head */
typedef enum { GDN_DELTA = 0, GDN_GLA = 1, GDN_DELTA_DIAG = 2 } gdn_update;

/* flags of gdn_hybrid_prefill / gdn_hybrid_decode */
enum {
  GDN_BRANCH_LINEAR = 1,   /* add o_lin to o                                   */
  GDN_BRANCH_SOFTMAX = 2,  /* add o_swa to o                                   */
  GDN_WRITE_STATE = 4,     /* prefill only: write the final state to state_out */
  GDN_ACCUMULATE = 8,      /* prefill only: add the selected branches to the
                              values o already holds instead of overwriting */
  /* Two-phase prefill (gated delta rule or GLA, linear branch or state
     selected, at least one stream chunk, and a launch plan with a separate
     chunk-preparation launch: every plan except the bf16 one-launch path
     for fewer chains than compute units, which returns GDN_EUNSUPPORTED
     for either flag).  GDN_PREPARE_ONLY runs only the state-independent
     chunk preparation into the workspace (o and state_out untouched);
     GDN_PREPARED skips it, the workspace holding what a GDN_PREPARE_ONLY
     call with the same arguments (other flags equal) wrote, with k, a and b
     unchanged since.  Setting both is GDN_EINVAL. */
  GDN_PREPARE_ONLY = 16,
  GDN_PREPARED = 32
};

/* flags of shortconv_qkv */
enum { GDN_ROPE = 1, GDN_L2NORM = 2 };

enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,
  GDN_EUNSUPPORTED = -2,
  GDN_EWORKSPACE = -3,
  GDN_ELAUNCH = -4
};

/* Library version as major*10000 + minor*100 + patch. */
int gdn_hybrid_version(void);

/* Static text for a return code. */
const char* gdn_hybrid_strerror(int code);

/* hipError_t of the last failed launch in this process (0 if none). */
int gdn_hybrid_last_hip_error(void);

/*
 * Test-only fault injection for the bounded waits described above
 * (process-wide; affects launches issued after the call).  faults: bit 0 =
 * the preparation publishes no chunk-ready flags, bit 1 = the scan publishes
 * no row-done flags, so every wait on them runs into its bound and the
 * affected rows / states come out as NaN while every kernel still exits.
 * wait_us: the bound of each wait in microseconds (default 100000).
 * faults = 0, wait_us = 100000 restores normal operation.
 * Errors: GDN_EINVAL if faults is outside 0..3 or wait_us outside
 * 1..1000000.
 */
int gdn_hybrid_set_test_faults(int faults, int wait_us);

/*
 * Workspace bytes gdn_hybrid_prefill needs for these arguments (written to
 * *bytes).  Non-zero when the linear branch or the state is requested and
 * T > n_sink + window: the state-independent part of every 64-token chunk is
 * computed for all chunks in parallel and stored there, so the sequential
 * scan over chunks only does the state-dependent products.  With
 * nch = ceil((T - window - n_sink) / 64) and elt the size of `dtype`:
 *   GDN_DELTA, few chains (bf16 and B * H * dk / 64 < 256): B * H * nch *
 *     ((64 * 64 + 2 * 64 * dk) * elt + 64 * dk * 4 + 128 * 4 + 8 + dk / 2)
 *     bytes
 *     (Wm, the decayed K^T, the decayed causal scores, the inverse of the
 *     chunk's unit lower-triangular system applied to b * V in fp32, the
 *     gate prefix sums: every state-independent chunk product, and flags
 *     that hand each chunk from the preparation to the scan and from the
 *     scan to the softmax branch; about 150 MB for B=1, H=32, T=4096).  With
 *     both branches, no GDN_ACCUMULATE and a multiple of 4 query heads per
 *     KV head, the whole layer is one launch.  The flags need
 *     no initialisation; a workspace must not be shared by calls that may
 *     run concurrently;
 *   GDN_DELTA otherwise: B * H * nch * (2 * 64 * 64 * elt + 128 * 4) bytes
 *     (the inverse scaled by b and by b * gamma, the gate prefix sums);
 *   GDN_GLA: B * H * nch * ((2 * 64 * dk + 64 * 64) * elt + dk * 4) bytes
 *     (gate-scaled Q and K^T, the intra-chunk scores, the chunk decay);
 *   GDN_DELTA_DIAG: B * H * nch * ((3 * 64 * dk + 2 * 64 * 64) * elt +
 *     dk * 4) bytes (as GDN_GLA, plus the inverse scaled by b and its
 *     product with the gate-scaled K).
 * Errors: GDN_EINVAL if bytes is NULL or the shape arguments are invalid.
 */
int gdn_hybrid_prefill_workspace(int B, int T, int H, int Hkv, int dk, int dv,
                                 int n_sink, int window, int dtype, int update,
                                 int flags, size_t* bytes);

/*
 * Prefill of whole sequences starting at position 0 ([P1] 线性注意力替换机制,
 * 填补近似缺口的实用设计; the sum of the two branches as defined above).
 *
 *   q          [B, T, H, dk]    dtype
 *   k          [B, T, Hkv, dk]  dtype
 *   v          [B, T, Hkv, dv]  dtype
 *   a          GDN: [B, T, H] fp32 (scalar gate); GLA, GDN_DELTA_DIAG:
 *              [B, T, H, dk] fp32 (one gate per channel)
 *   b          GDN, GDN_DELTA_DIAG: [B, T, H] fp32; GLA: ignored (may be NULL)
 *   o          [B, T, H, dv]    dtype, written (every row) unless flags has
 *              neither branch bit (then it may be NULL)
 *   state_out  [B, H, dk, dv] fp32: S after token T-1-window (zero if none),
 *              the state a following decode step continues from; written iff
 *              flags & GDN_WRITE_STATE (else may be NULL)
 *   n_sink >= 0, window >= 1; flags: any combination of GDN_BRANCH_LINEAR,
 *   GDN_BRANCH_SOFTMAX, GDN_WRITE_STATE (at least one) and GDN_ACCUMULATE.
 *   With GDN_ACCUMULATE, o must hold initialised values and receives
 *   o += (selected branches); calling once with GDN_BRANCH_LINEAR and once
 *   with GDN_BRANCH_SOFTMAX | GDN_ACCUMULATE gives the same o as one call
 *   with both branches (each call then launches a single kernel).
 *   workspace / workspace_bytes: device buffer of at least the size reported
 *   by gdn_hybrid_prefill_workspace, 256-byte aligned, owned by the caller
 *   and free for reuse once the call's work on `stream` is done (may be
 *   NULL / 0 when that size is 0).  GDN_EWORKSPACE if it is missing or too
 *   small, GDN_EINVAL if misaligned.
 * Supported: d in {64, 128} for bf16; the linear branch (or the state) in
 * fp32 only at d = 64 (GDN_EUNSUPPORTED otherwise).
 * Preconditions (not checked): gates a in (0, 1], b in [0, 1].  GDN gates
 * may decay at any rate.  GLA and GDN_DELTA_DIAG operands are formed
 * relative to a reference token every 16 tokens, so results are exact (to
 * rounding) while the product of any 8 consecutive gates of one channel
 * stays above e^-80 (a mean gate above about 5e-5).
 */
int gdn_hybrid_prefill(const void* q, const void* k, const void* v,
                       const float* a, const float* b,
                       void* o, float* state_out,
                       int B, int T, int H, int Hkv, int dk, int dv,
                       int n_sink, int window, int dtype, int update, int flags,
                       void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * One decode step for B sequences, each at its own position t = pos[b]
 * ([P1] 填补近似缺口的实用设计; [P2] fixed-budget cache routing).
 * Per sequence: the token e = t - window leaves the window; if e >= n_sink
 * it is folded into the state with its own cached gates; o_lin = S^T q_t;
 * o_swa is the softmax over the sinks and the window (t-window, t], the new
 * token included; o = o_lin + o_swa (as selected by flags); the new k, v and
 * gates are stored in slot(t); pos[b] += 1.
 *
 *   q          [B, H, dk]        dtype
 *   k, v       [B, Hkv, dk|dv]   dtype    (the new token)
 *   a          GDN [B, H] fp32; GLA, GDN_DELTA_DIAG [B, H, dk] fp32
 *   b          GDN, GDN_DELTA_DIAG [B, H] fp32; GLA: ignored (may be NULL)
 *   state      [B, H, dk, dv] fp32, in/out
 *   k_cache, v_cache [B, Hkv, n_sink + window, d] dtype, in/out.  Token i
 *              lives in slot i if i < n_sink, else in slot
 *              n_sink + (i - n_sink) mod window.
 *   a_cache    GDN [B, window, H] fp32; GLA, GDN_DELTA_DIAG [B, window, H, dk]
 *              fp32, in/out
 *   b_cache    GDN, GDN_DELTA_DIAG [B, window, H] fp32 (GLA: ignored, may be
 *              NULL), in/out.
 *              Gates of token i >= n_sink live at ring index
 *              (i - n_sink) mod window.
 *   pos        [B] int32, in/out: position of the new token; incremented.
 *   o          [B, H, dv] dtype, out
 *   flags      GDN_BRANCH_LINEAR and/or GDN_BRANCH_SOFTMAX (the state and
 *              cache are updated either way).
 * Supported: d in {64, 128}; G <= 16; G * (n_sink + window) <= 12288.
 */
int gdn_hybrid_decode(const void* q, const void* k, const void* v,
                      const float* a, const float* b,
                      float* state,
                      void* k_cache, void* v_cache,
                      float* a_cache, float* b_cache,
                      int* pos, void* o,
                      int B, int H, int Hkv, int dk, int dv,
                      int n_sink, int window, int dtype, int update, int flags,
                      void* stream);

/*
 * Inference-time hybridisation ([P3] 关键设计 (1): the two branches' weights
 * set their contributions at inference): gdn_hybrid_prefill and
 * gdn_hybrid_decode with o = w_lin * o_lin + w_swa * o_swa on the selected
 * branches (GDN_ACCUMULATE: o += that).  Weights (1, 1) are the plain sum the
 * calls above compute; (1, 0) and (0, 1) give what the single-branch flags
 * give.  Arguments, layouts and return codes as in those calls; non-finite
 * weights are GDN_EINVAL.
 */
int gdn_hybrid_prefill_weighted(const void* q, const void* k, const void* v,
                                const float* a, const float* b,
                                void* o, float* state_out,
                                int B, int T, int H, int Hkv, int dk, int dv,
                                int n_sink, int window, int dtype, int update, int flags,
                                float w_lin, float w_swa,
                                void* workspace, size_t workspace_bytes,
                                void* stream);
int gdn_hybrid_decode_weighted(const void* q, const void* k, const void* v,
                               const float* a, const float* b,
                               float* state,
                               void* k_cache, void* v_cache,
                               float* a_cache, float* b_cache,
                               int* pos, void* o,
                               int B, int H, int Hkv, int dk, int dv,
                               int n_sink, int window, int dtype, int update, int flags,
                               float w_lin, float w_swa,
                               void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gdn_hybrid_prefill without a workspace argument.  Arguments, layouts,
 * flags and results are those of gdn_hybrid_prefill; the kernels are the
 * same.  The chunk workspace is a library-owned device array of
 * gdn_hybrid_noalloc_max_workspace() bytes (256 MiB) per GPU, created when
 * the library's device code is loaded on that GPU and held until the
 * process ends; the call itself allocates and frees nothing.  Its address
 * is looked up on the first call on each device (the current device at the
 * time of the call; the stream must belong to it).  Nothing in the array
 * needs clearing between calls (the workspace's hand-off flags carry a
 * per-call value).  Every call on one GPU shares that GPU's array, so calls
 * whose work may overlap on one GPU (other streams, other host threads)
 * race: serialise them.
 * Errors: as gdn_hybrid_prefill, and GDN_EWORKSPACE when the workspace
 * these arguments need (gdn_hybrid_prefill_workspace) exceeds the array.
 */
int gdn_hybrid_prefill_noalloc(const void* q, const void* k, const void* v,
                               const float* a, const float* b,
                               void* o, float* state_out,
                               int B, int T, int H, int Hkv, int dk, int dv,
                               int n_sink, int window, int dtype, int update, int flags,
                               void* stream);
/* Bytes of the per-GPU array gdn_hybrid_prefill_noalloc uses. */
size_t gdn_hybrid_noalloc_max_workspace(void);

/*
 * Backward pass of the prefill (the training path; [P1] 实践建议 item 4
 * trains the linearised layers, [P1] 线性注意力替换机制 gives the recurrence
 * differentiated): the gradients of
 *     L = sum(d_o * o) + sum(d_state * S_final),
 *     o = w_lin o_lin + w_swa o_swa   (both branches, no cache),
 * for o and S_final as gdn_hybrid_prefill_weighted computes them from q, k,
 * v, a, b (state starting at zero).
 *   d_o      [B,T,H,d]     upstream gradient of o (dtype of q)
 *   d_state  [B,H,d,d]     upstream gradient of the final state, fp32; NULL
 *                          means zero
 *   dq       [B,T,H,d]     fp32, dL/dq
 *   dk, dv   [B,T,Hkv,d]   fp32, dL/dk, dL/dv (summed over the G query heads
 *                          of each KV head)
 *   da, db   [B,T,H]       fp32, dL/da, dL/db (zero where the recurrence
 *                          does not read them)
 * Every output is overwritten.  Supported: update = GDN_DELTA, dtype =
 * GDN_BF16, d_k = d_v = 128 (GDN_EUNSUPPORTED otherwise); any B, T, H, Hkv,
 * n_sink >= 0, window >= 1.  The workspace (device, 256-byte aligned, size
 * from gdn_hybrid_prefill_backward_workspace; its contents on entry do not
 * matter) holds the chunk preparation, the state entering every 64-token
 * chunk and the gradient of the state leaving it (bf16), and the softmax
 * row statistics.  fp32 gradients are accumulated from bf16 MFMA products
 * with fp32 accumulation.
 * Errors: as gdn_hybrid_prefill.
 */
int gdn_hybrid_prefill_backward_workspace(int B, int T, int H, int Hkv, int dk, int dv,
                                          int n_sink, int window, int dtype, int update,
                                          size_t* bytes);
int gdn_hybrid_prefill_backward(const void* q, const void* k, const void* v,
                                const float* a, const float* b,
                                const void* d_o, const float* d_state,
                                float* dq, float* dk, float* dv, float* da, float* db,
                                int B, int T, int H, int Hkv, int dk_, int dv_,
                                int n_sink, int window, int dtype, int update,
                                float w_lin, float w_swa,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fill the decode cache after a prefill of T tokens, so decoding resumes at
 * position T: sinks 0..min(n_sink,T)-1 and window tokens
 * max(n_sink, T-window)..T-1 go to their slots (layouts as in
 * gdn_hybrid_decode), their gates to their ring indices; every other slot is
 * zeroed.  k, v, a, b are the prefill inputs (layouts of gdn_hybrid_prefill).
 */
int gdn_hybrid_cache_from_prefill(const void* k, const void* v,
                                  const float* a, const float* b,
                                  void* k_cache, void* v_cache,
                                  float* a_cache, float* b_cache,
                                  int B, int T, int H, int Hkv, int dk, int dv,
                                  int n_sink, int window, int dtype, int update,
                                  void* stream);

/*
 * Q/K/V preparation ([P1] 实践建议 item 3; [P2] short convolutions):
 * RoPE (flags & GDN_ROPE; q and k; rotate-half pairs (j, j + d/2),
 * inv_freq_j = rope_theta^(-2j/d), positions pos0 + t), then a causal
 * depthwise convolution of kernel size `ksize` on q, k and v
 * (y[t, c] = sum_{j<ksize} w[c, ksize-1-j] x[t-j, c], zero history, no bias),
 * then (flags & GDN_L2NORM) x / sqrt(sum x^2 + 1e-6) over each head of q, k.
 *
 *   q, q_out   [B, T, H, d]    dtype      channel c = h * d + i
 *   k, v, k_out, v_out [B, T, Hkv, d] dtype
 *   wq [H*d, ksize], wk [Hkv*d, ksize], wv [Hkv*d, ksize] fp32
 * Supported: d in {64, 128}; 1 <= ksize <= 8; rope_theta > 0; pos0 >= 0;
 * B <= 65535 and T <= 65535 * 64 (grid dimensions), else GDN_EUNSUPPORTED.
 */
int shortconv_qkv(const void* q, const void* k, const void* v,
                  const float* wq, const float* wk, const float* wv,
                  void* q_out, void* k_out, void* v_out,
                  int B, int T, int H, int Hkv, int d, int ksize,
                  float rope_theta, int pos0, int flags, int dtype,
                  void* stream);

/*
 * Short-conv history for decoding after a prefill ([P1] 实践建议 item 3: the
 * short convolution of shortconv_qkv, continued one token at a time).  For
 * q, k and v it holds the inputs of the last ksize - 1 tokens after RoPE
 * (q and k, flags & GDN_ROPE) and before the convolution, in fp32; token i
 * sits at ring index i mod (ksize - 1).  This call writes the history after
 * a prefill of T tokens at positions pos0 .. pos0 + T - 1, so that decoding
 * continues with token T; ring slots of tokens before 0 are zeroed.
 *
 *   q [B, T, H, d], k, v [B, T, Hkv, d]   dtype: the raw projections that
 *              were given to shortconv_qkv (may be NULL when T = 0)
 *   hist_q [B, ksize-1, H*d], hist_k, hist_v [B, ksize-1, Hkv*d] fp32, out
 *              (caller-owned; channel c = h * d + i)
 * ksize = 1 keeps no history: nothing is written and the history pointers
 * may be NULL.  Supported: d in {64, 128}; 1 <= ksize <= 8; B <= 65535;
 * rope_theta > 0 when RoPE is on; pos0 >= 0.
 */
int shortconv_history_from_prefill(const void* q, const void* k, const void* v,
                                   float* hist_q, float* hist_k, float* hist_v,
                                   int B, int T, int H, int Hkv, int d, int ksize,
                                   float rope_theta, int pos0, int flags, int dtype,
                                   void* stream);

/*
 * One decode step of the Q/K/V preparation: shortconv_qkv evaluated at one
 * new token per sequence.  Sequence b's token has index t = pos[b] in its
 * sequence and RoPE position pos0 + t.  pos is only read: call this before
 * gdn_hybrid_decode of the same step (which advances pos) and feed it the
 * outputs.  The token's input after RoPE is convolved with the history of
 * its ksize - 1 predecessors (zero before the sequence start), q and k are
 * L2-normalised (flags & GDN_L2NORM), and the input replaces token
 * t - ksize + 1 at ring index t mod (ksize - 1) of the history.
 *
 *   q, q_out   [B, H, d]      dtype (raw projection in, prepared out)
 *   k, v, k_out, v_out [B, Hkv, d] dtype
 *   wq, wk, wv as in shortconv_qkv
 *   hist_q, hist_k, hist_v  as in shortconv_history_from_prefill, in/out
 *              (a fresh sequence starts from zeros; may be NULL for ksize 1)
 *   pos        [B] int32 >= 0, read only
 * Supported: d in {64, 128}; 1 <= ksize <= 8; B <= 65535; rope_theta > 0
 * when RoPE is on; 0 <= pos0 < 2^30.
 */
int shortconv_qkv_decode(const void* q, const void* k, const void* v,
                         const float* wq, const float* wk, const float* wv,
                         float* hist_q, float* hist_k, float* hist_v,
                         const int* pos,
                         void* q_out, void* k_out, void* v_out,
                         int B, int H, int Hkv, int d, int ksize,
                         float rope_theta, int pos0, int flags, int dtype,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_HYBRID_H */
