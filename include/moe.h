/*
 * moe.h -- C ABI of the MI355X (gfx950) sparsely-gated mixture-of-experts
 * layer forward.
 *
 * The layer (FastMoE announcement page, "§1 MoE 设计", Fig. 1; industry
 * overview page, "MoE的內涵"): a gate scores every token against E experts,
 * each token goes to its k best experts, each expert is a two-layer MLP, and
 * the token's output is the gate-weighted sum of its experts' outputs.  The
 * entry points below are its steps:
 *
 *   moe_route        gate GEMM -> [gating-logit normalisation] -> softmax -> top-k
 *   moe_permute      per-expert counts, capacity clip, stable counting-sort
 *                    permutation of the token rows by expert
 *   moe_expert_up    first expert linear layer + activation, per expert segment
 *   moe_expert_down  second expert linear layer, per expert segment
 *   moe_grouped_ffn  moe_expert_up then moe_expert_down
 *   moe_combine      gate-weighted un-permute back to token order
 *   moe_forward      all of the above
 *   moe_router_stats balancing statistics of a routed batch (aux / Z-loss
 *                    inputs, drop rate)
 *   moe_shared_expert, moe_combine_shared
 *                    an ungated shared expert over all tokens, added in the
 *                    combine
 *   moe_quantize_fp8, moe_expert_up_fp8, moe_expert_down_fp8, moe_forward_fp8
 *                    the layer with FP8 (E4M3) expert weights and activations
 *   moe_forward_train, moe_backward
 *                    training: the forward keeping its intermediates, and the
 *                    gradients of every input and weight
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory: every tensor argument is DEVICE memory owned by the caller (for
 *   example a torch tensor's data_ptr()).  The library never allocates, frees,
 *   copies to the host or synchronises; it only enqueues kernels on `stream`
 *   (a hipStream_t; NULL is the null stream).  Results are valid once the
 *   caller has synchronised with that stream.  Outputs must not alias inputs
 *   or each other.  The library keeps no state between calls except a cached
 *   per-device compute-unit count; calls are reentrant.
 * Layout: every tensor is dense row-major.  "dtype" tensors hold fp32 or bf16
 *   (bf16 as raw 16-bit patterns) according to problem->dtype.
 *     x       [T][d]      dtype   token activations
 *     Wg      [E][d]      dtype   gate weight (out x in, like nn.Linear.weight)
 *     bg      [E]         fp32    gate bias (nullable)
 *     logits  [T][E]      fp32
 *     W1      [E][n1][d]  dtype   n1 = F (ReLU) or 2F (SwiGLU: rows 0..F-1 are
 *                                 the gate projection, rows F..2F-1 the up
 *                                 projection, the fused order of the
 *                                 Megatron-Core page, "权重转换要点")
 *     W2      [E][d][F]   dtype
 *     topk_idx, slot [T][k] int32;  topk_w [T][k] fp32
 *     counts [E], offsets [E+1] int32;  src_token [T*k] int32
 *     x_perm, y_perm [T*k][d] dtype;  h [T*k][F] dtype
 *   Only the first offsets[E] rows of x_perm / y_perm / h / src_token are
 *   meaningful (P = offsets[E] = number of kept assignments).
 * Alignment: dtype tensors and the workspace must be 16-byte aligned, int32
 *   and fp32 tensors 4-byte aligned.
 * Errors: arguments are checked on the host before anything is enqueued; on
 *   any error nothing is enqueued, the call returns a non-zero moe_status and
 *   moe_last_error() (per thread) says why.  A failed kernel launch returns
 *   MOE_ERR_HIP.  Faults inside kernels surface at the caller's next
 *   synchronisation.  Non-finite logits or inputs violate a precondition and
 *   give unspecified (but in-bounds) results.
 * Limits: 1 <= k <= min(E, 8), E <= 1024, 0 <= T <= 2^24, d and F multiples
 *   of 64 with 64 <= d, F <= 65536.  T == 0 is a valid empty call.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad option */
    MOE_ERR_UNSUPPORTED = 2, /* outside the limits above */
    MOE_ERR_WORKSPACE = 3,   /* workspace too small */
    MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} moe_status;

enum { MOE_ACT_RELU = 0, MOE_ACT_SWIGLU = 1 };
enum { MOE_F32 = 0, MOE_BF16 = 1 };

typedef struct {
    int32_t T;                /* tokens */
    int32_t d;                /* model width */
    int32_t E;                /* experts */
    int32_t k;                /* experts per token */
    int32_t F;                /* expert hidden width */
    int32_t act;              /* MOE_ACT_RELU | MOE_ACT_SWIGLU */
    int32_t dtype;            /* MOE_F32 | MOE_BF16 */
    int32_t normalize;        /* 0: softmax(z); 1: softmax(lambda * standardise(z)) */
    float lambda;             /* finite and > 0 when normalize == 1 */
    float capacity_factor;    /* <= 0: dropless; > 0: capacity C = ceil(cf*T*k/E), see moe_capacity */
} moe_problem;

/* Optional outputs of moe_forward; each field may be NULL (the library then
 * keeps that tensor in the workspace). */
typedef struct {
    int32_t* topk_idx;  /* [T][k] */
    float* topk_w;      /* [T][k] */
    int32_t* counts;    /* [E] assignments per expert before the capacity clip */
    int32_t* offsets;   /* [E+1] */
    int32_t* slot;      /* [T][k] permuted row, -1 when dropped */
    int32_t* src_token; /* [T*k] */
} moe_route_info;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status s);

/* Message of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* Expert capacity of a problem: C = ceil(cf * T * k / E) (cf > 0), or -1
 * when dropless (cf <= 0).  cf is the fp32 value held in the problem, and C
 * is the exact ceiling for that value (the product and quotient are formed in
 * double, where they are exact or cannot cross an integer): a factor that is
 * not exact in binary rounds from its fp32 neighbour, so cf = 0.3f with
 * T*k/E = 100 gives C = 31 (0.3f is slightly above 0.3), while dyadic factors
 * such as 0.25 or 1.25 give the decimal result.  Tokens beyond C on one
 * expert are dropped and contribute zero; the caller's residual connection
 * carries them (Megatron-Core page, "MoE负载均衡的挑战与应对" and its Q&A).
 * Host only. */
moe_status moe_capacity(const moe_problem* p, int32_t* C);

/* Bytes of workspace that suffice for every entry point of this problem
 * (moe_forward needs the most: routing, permutation, h, y_perm and the
 * partial tiles of the grouped GEMM's K-split last round).  Host only. */
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);

/* Gate and routing (FastMoE page, "特色二": one fully connected layer as
 * gate; Skywork-MoE news item, "技术创新 1", and Skywork slides, slide 6:
 * gating-logit normalisation; Megatron-Core page, "关键特性": Top-K router).
 *   If x and Wg are both non-NULL: logits[t,e] = sum_i x[t,i] Wg[e,i] + bg[e]
 *   (products and sums in fp64, rounded once to fp32) is WRITTEN.
 *   If x and Wg are both NULL: logits is an INPUT.
 *   Then per token: s = z, or lambda*(z - mean_e z)/std_e z (population std;
 *   a token with std 0 gets s = 0); p = softmax(s) over all E experts;
 *   topk_idx[t,0..k-1] = the k largest fp32 logits in descending order, equal
 *   logits to the lower expert index, -0 == +0; topk_w[t,j] = p[topk_idx[t,j]]
 *   (not renormalised). */
moe_status moe_route(const moe_problem* p, const void* x, const void* Wg, const float* bg,
                     float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/* Counting, capacity and permutation (Megatron-Core page, "关键特性": token
 * permutation; "MoE负载均衡的挑战与应对": capacity / dropless).
 *   counts[e] = number of (t,j) with topk_idx[t,j] == e;
 *   kept_e = min(counts[e], C) (C from moe_capacity; no clip when dropless);
 *   offsets = exclusive prefix sum of kept (E+1 entries);
 *   the rank of (t,j) on its expert e is the number of earlier tokens t' < t
 *   that chose e; it is kept iff rank < C, at row offsets[e] + rank:
 *   slot[t,j] = that row (else -1), src_token[row] = t, x_perm[row] = x[t].
 * topk_idx entries must lie in [0,E) and be distinct within a token (entries
 * outside [0,E) are skipped; duplicates give unspecified rows, never writes
 * out of bounds).  x_perm == NULL (then x may be NULL too) skips the row
 * copy, for callers that read x through src_token (moe_expert_up does).
 * Needs ws_bytes >= moe_workspace_size. */
moe_status moe_permute(const moe_problem* p, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* slot, int32_t* src_token, void* x_perm, void* ws,
                       size_t ws_bytes, void* stream);

/* First expert layer over the expert segments (FastMoE page, "特色三": ReLU
 * two-layer MLP experts, many experts on one GPU; Megatron-Core page,
 * "关键特性": GroupedGEMM): for every expert e and row r in
 * [offsets[e], offsets[e+1]):  u = W1[e] a_r, where a_r = a[r] when
 * src_token is NULL (a = x_perm, T*k rows) and a_r = a[src_token[r]] when it
 * is given (a = x, T rows: the permuted rows are gathered on the fly; x
 * must then be below 0xF0000000 bytes, else MOE_ERR_UNSUPPORTED);
 *   ReLU:   h[r,f] = max(u_f, 0)
 *   SwiGLU: h[r,f] = silu(u_f) * u_{F+f},  silu(g) = g / (1 + exp(-g))
 * fp32 accumulation, h stored in dtype.  offsets is read on the device (no
 * host synchronisation) and must be non-decreasing with offsets[E] <= T*k;
 * h holds T*k rows.  Offsets outside [0, T*k] or decreasing are
 * clamped into range (unspecified results, never an out-of-bounds access).
 * ws (nullable; if given, ws_bytes >= moe_workspace_size) lets the last,
 * partly filled round of output tiles be split along K, with the parts
 * summed in a fixed order: results stay deterministic, but may differ from
 * the unsplit ones in the last bits (another fp32 summation order). */
moe_status moe_expert_up(const moe_problem* p, const void* a, const int32_t* src_token, const int32_t* offsets,
                         const void* W1, void* h, void* ws, size_t ws_bytes, void* stream);

/* Second expert layer: y_perm[r] = W2[e] h[r] for r in expert e's segment
 * (same offsets and workspace rules as moe_expert_up). */
moe_status moe_expert_down(const moe_problem* p, const void* h, const int32_t* offsets, const void* W2,
                           void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* moe_expert_up then moe_expert_down, with h in the workspace. */
moe_status moe_grouped_ffn(const moe_problem* p, const void* x_perm, const int32_t* offsets, const void* W1,
                           const void* W2, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine (industry overview page, "MoE的內涵": the gate weights the
 * experts' mix): y[t] = sum over j = 0..k-1 with slot[t,j] >= 0, in that
 * order, of topk_w[t,j] * y_perm[slot[t,j]] (fp32 accumulation, stored in
 * dtype).  A token with every choice dropped gets y[t] = 0.  y_perm holds
 * T*k rows; a slot >= T*k counts as dropped. */
moe_status moe_combine(const moe_problem* p, const void* y_perm, const int32_t* slot, const float* topk_w,
                       void* y, void* stream);

/* The whole layer.  Wg == NULL means logits is a given INPUT (x is still the
 * token activations); otherwise logits (nullable) receives the gate logits.
 * info (nullable) receives the routing and permutation.  Needs
 * ws_bytes >= moe_workspace_size. */
moe_status moe_forward(const moe_problem* p, const void* x, const void* Wg, const float* bg, const void* W1,
                       const void* W2, void* y, float* logits, const moe_route_info* info, void* ws,
                       size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same steps and kernels, with the workspace in the library's own device
 * scratch, a fixed 32 MiB array per GPU (held from the library's load until
 * the process ends; its address is looked up once per device on that
 * device's first call).  The caller passes inputs and outputs as in
 * moe_forward and no workspace; nothing is allocated or freed.  The grouped
 * GEMMs run without the K split of their last round (the split needs room for
 * partial tiles), so y may differ from moe_forward's in the last bits (fp32
 * summation order); routing and permutation are identical.  Problems whose
 * workspace without those partial tiles exceeds 32 MiB (about 450 tokens at
 * the Mixtral shape) return MOE_ERR_WORKSPACE.  Every call on a GPU uses that
 * GPU's one scratch: calls that overlap on one GPU (other streams, other
 * threads) race and give undefined results; no step relies on the scratch's
 * previous contents. */
moe_status moe_forward_noalloc(const moe_problem* p, const void* x, const void* Wg, const float* bg,
                               const void* W1, const void* W2, void* y, float* logits,
                               const moe_route_info* info, void* stream);

/* Router by-products (Megatron-Core page, "MoE负载均衡的挑战与应对": an
 * auxiliary loss pushes experts towards equal token counts, "关键特性":
 * Z-Loss; Skywork-MoE news item, "技术创新 2. 自适应的Aux Loss", and slides,
 * slide 7: the loss coefficient follows the token drop rate).  The pages give
 * no formulas; these are the plainest readings:
 *   frac[e]      = counts[e] / (T k)          (share of the assignments)
 *   mean_prob[e] = (1/T) sum_t p[t,e]         (p as in moe_route, after the
 *                                              optional normalisation)
 *   scalars[0]   = E * sum_e frac[e] mean_prob[e]   (auxiliary loss, without
 *                                                    its coefficient)
 *   scalars[1]   = (1/T) sum_t (log sum_e exp logits[t,e])^2   (Z-loss)
 *   scalars[2]   = (T k - offsets[E]) / (T k)                   (drop rate)
 * logits [T][E] fp32 are the ones the routing used; counts [E] and offsets
 * [E+1] come from moe_permute.  Sums in fp64 in a fixed order (the same bits
 * on every run), outputs fp32: frac [E], mean_prob [E], scalars [3].  Needs
 * ws_bytes >= moe_workspace_size. */
moe_status moe_router_stats(const moe_problem* p, const float* logits, const int32_t* counts,
                            const int32_t* offsets, float* frac, float* mean_prob, float* scalars, void* ws,
                            size_t ws_bytes, void* stream);

/* Shared expert (industry overview page, "MoE未來重點研究方向" item 4:
 * DeepSeekMoE's shared experts): one more two-layer MLP that every token
 * passes through, ungated, with hidden width Fs (a multiple of 64 in
 * [64, 65536]) and the problem's activation:
 *   y_shared[t] = Ws2 act(Ws1 x[t])
 * Ws1 [n1s][d] (n1s = Fs, or 2Fs for SwiGLU, gate rows first), Ws2 [d][Fs],
 * x and y_shared [T][d], all dtype.  The hidden rows live in the workspace:
 * ws_bytes >= moe_shared_workspace_size(p, Fs). */
moe_status moe_shared_workspace_size(const moe_problem* p, int32_t Fs, size_t* bytes);
moe_status moe_shared_expert(const moe_problem* p, int32_t Fs, const void* x, const void* Ws1, const void* Ws2,
                             void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* moe_combine with the shared expert's output added with weight one:
 * y[t] = y_shared[t] + sum over kept j of topk_w[t,j] * y_perm[slot[t,j]]
 * (fp32 accumulation starting from y_shared[t], j in order).  A token whose
 * choices were all dropped gets y_shared[t]. */
moe_status moe_combine_shared(const moe_problem* p, const void* y_perm, const int32_t* slot, const float* topk_w,
                              const void* y_shared, void* y, void* stream);

/* ---------------------------------------------------------------- training
 * Backward of the layer (every throughput figure on the pages is for
 * training: Skywork news item "训练Infra", FastMoE page "特色三", Megatron-Core
 * page "训练效果与性能实测").  The chain rule through the combine, both expert
 * layers, the softmax, the normalisation and the gate; the top-k choice and
 * the capacity drops pass no gradient (a dropped choice does not touch y).
 * moe_forward_train is moe_forward keeping what the backward needs: logits,
 * every info field, and the saved tensors below ([T*k] rows each, dtype).
 * A shared expert (moe_shared_expert) trains through the same two calls as a
 * layer with E = 1, k = 1 and given logits: the softmax of a single logit is
 * exactly 1, so that layer's output is the shared expert's. */
typedef struct {
    void* u;      /* [T*k][n1] pre-activation x W1[e]^T (gate then up columns for SwiGLU) */
    void* h;      /* [T*k][F] activation output */
    void* y_perm; /* [T*k][d] expert outputs */
} moe_saved;

/* The forward with logits (required, written or given as in moe_forward),
 * info (required, every field) and saved filled in.  Needs ws_bytes >=
 * moe_workspace_size. */
moe_status moe_forward_train(const moe_problem* p, const void* x, const void* Wg, const float* bg, const void* W1,
                             const void* W2, void* y, float* logits, const moe_route_info* info,
                             const moe_saved* saved, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace for moe_backward (gradients of the permuted rows,
 * transposed row operands of the weight gradients, and for fp32 layers
 * transposed copies of W1 and W2; bf16 layers read them as stored).  Host
 * only.  MOE_ERR_UNSUPPORTED when an operand [max(d,F,n1)][T*k + 64E] exceeds
 * 32-bit offsets. */
moe_status moe_backward_workspace_size(const moe_problem* p, size_t* bytes);

/* Balancing losses added to the training loss (their values are
 * moe_router_stats' aux and Z-loss; the auxiliary loss keeps experts
 * balanced: Megatron-Core page, "MoE负载均衡的挑战与应对" and "关键特性";
 * Skywork news, 技术创新 2, with a coefficient that follows the drop rate).
 * moe_backward adds their gradients:
 *   aux_coef * aux, aux = E sum_e f_e P_e (f_e = counts_e / (T k), constant):
 *     dp[t,e] += aux_coef E f_e / T before the softmax backward;
 *   z_coef * Z-loss, Z-loss = (1/T) sum_t lse(z_t)^2 on the raw logits:
 *     dz[t,e] += z_coef (2/T) lse(z_t) softmax(z_t)[e]. */
typedef struct {
    float aux_coef;
    float z_coef;
} moe_router_losses;

/* Gradients given dy = dL/dy [T][d] (dtype) and the forward's logits, info and
 * saved tensors (from moe_forward_train on the same inputs), and optionally
 * the balancing losses (losses == NULL: none; info->counts is read when
 * aux_coef != 0):
 *   dx [T][d] dtype; dW1 [E][n1][d], dW2 [E][d][F] fp32;
 *   dWg [E][d], dbg [E] fp32 (required when Wg != NULL; Wg == NULL means the
 *   logits were given and there is no gate gradient).
 * Per kept choice (t, j, e, w): d_w = <dy_t, y_perm row>, do = w dy_t;
 * dW2[e] += do h^T; dh = W2[e]^T do; du = act'(u) dh (ReLU: [u > 0]; SwiGLU:
 * dg = dh v silu'(g), dv = dh silu(g)); dW1[e] += du x_t^T; dx_t += W1[e]^T du.
 * Router: dp[e] = d_w of the kept choice on e; ds = p (dp - <p,dp>); with the
 * normalisation dz = (lambda/sigma)(ds - mean ds - zh mean(ds zh)) (0 when
 * sigma == 0), else dz = ds.  Gate: dWg = dz^T x, dbg = sum_t dz,
 * dx += dz Wg.  fp32 accumulation; sums in fixed orders (the same bits on
 * every run).  Needs ws_bytes >= moe_backward_workspace_size. */
moe_status moe_backward(const moe_problem* p, const void* dy, const void* x, const void* Wg, const void* W1,
                        const void* W2, const float* logits, const moe_route_info* info, const moe_saved* saved,
                        const moe_router_losses* losses, void* dx, float* dWg, float* dbg, float* dW1, float* dW2,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- FP8 experts
 * Expert weights as OCP FP8 E4M3 codes (Skywork-MoE model card: an FP8
 * checkpoint; Skywork news item, "4090推理": FP8-quantised inference;
 * Megatron-Core page, "关键特性": FP8 among the coming features).  The pages
 * fix no scheme; this one: every row of a weight matrix, every token row of x
 * and every row of h carries a power-of-two scale s, the smallest with
 * max|row| <= 448 s, and holds the E4M3 codes nearest to v / s (ties to even,
 * saturating at 448).  The expert GEMMs multiply codes on gfx950's FP8 MFMA
 * (fp32 accumulation) and apply row scale x weight-row scale to each output
 * before the activation; h, y_perm and y are bf16.  Routing is the bf16
 * layer's (gate on the bf16 x).  Requirements beyond the common limits:
 * problem->dtype == MOE_BF16 (the activation type), d and F multiples of 128.
 *   W1q [E][n1][d] codes, w1s [E][n1] fp32 scales (gate rows first for SwiGLU)
 *   W2q [E][d][F] codes,  w2s [E][d] fp32 scales
 *   xq [T][d] codes, xs [T];  hq [T*k][F] codes, hs [T*k]
 * Codes must be 16-byte aligned. */

/* Quantise rows rows of K values (src_dtype MOE_F32 or MOE_BF16; K a multiple
 * of 64): codes [rows][K], scales [rows] = 2^e as above.  Usable for weights
 * (one expert's matrix is E*n1 rows) and activations.  No workspace. */
moe_status moe_quantize_fp8(const void* src, int32_t src_dtype, int64_t rows, int32_t K, uint8_t* codes,
                            float* scales, void* stream);

/* Bytes of workspace for moe_forward_fp8 (the bf16 workspace plus the codes
 * and scales of x and h).  Host only. */
moe_status moe_fp8_workspace_size(const moe_problem* p, size_t* bytes);

/* FP8 first expert layer: as moe_expert_up, with aq the codes of x
 * (src_token given, rows gathered on the fly) or of x_perm (src_token NULL)
 * and as their row scales (indexed like aq's rows).  The gather addresses
 * the codes with 32-bit byte offsets: with src_token, T*d must stay below
 * 0xF0000000 bytes, else MOE_ERR_UNSUPPORTED (pass permuted codes). */
moe_status moe_expert_up_fp8(const moe_problem* p, const uint8_t* aq, const float* as, const int32_t* src_token,
                             const int32_t* offsets, const uint8_t* W1q, const float* w1s, void* h, void* ws,
                             size_t ws_bytes, void* stream);

/* FP8 second expert layer: y_perm[r] = (W2q[e] w2s[e]) (hq[r] hs[r]), bf16 out.
 * ws as in moe_expert_down. */
moe_status moe_expert_down_fp8(const moe_problem* p, const uint8_t* hq, const float* hs, const int32_t* offsets,
                               const uint8_t* W2q, const float* w2s, void* y_perm, void* ws, size_t ws_bytes,
                               void* stream);

/* The whole layer with FP8 experts: route and permute as moe_forward, then
 * quantise x per token, FP8 up-projection, quantise h per row, FP8
 * down-projection, combine.  Needs ws_bytes >= moe_fp8_workspace_size.  The
 * up-projection gathers the token codes (T*d bytes) with 32-bit offsets:
 * T*d >= 0xF0000000 returns MOE_ERR_UNSUPPORTED. */
moe_status moe_forward_fp8(const moe_problem* p, const void* x, const void* Wg, const float* bg, const uint8_t* W1q,
                           const float* w1s, const uint8_t* W2q, const float* w2s, void* y, float* logits,
                           const moe_route_info* info, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
