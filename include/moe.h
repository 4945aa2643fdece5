/*
 * moe.h: C ABI of the MI355X (gfx950) top-k Mixture-of-Experts layer forward.
 *
 * The library computes, on one GPU with every expert resident, the forward pass of a
 * top-k MoE FFN layer: fp32 router logits, softmax, top-k selection with gate
 * renormalisation modes, the per-expert load histogram and capacity slots, the
 * permutation of tokens into expert-contiguous buffers, the gated expert FFN as two
 * grouped GEMMs, and the gate-weighted combine back to token order.
 *
 * Sources (the pages the method is taken from; cited below by their short key):
 *   [GROK5]  "第 5 章 model.py 精读·中：MoE 路由与专家" (Grok-1 中文精读, chapter 5),
 *            https://yingwang.github.io/grok-1/05-model-2/
 *   [BOOK12] "第 12 章 MoE：路由、专家与负载" (LLMs from scratch, chapter 12),
 *            https://book.ozine.me/llm/llms-from-scratch/chapters/12_moe.html
 *   [SERIES] "8.1 MoE 系列：从 GShard 到 Mixtral，再到 Switch Transformer",
 *            https://gitcode.csdn.net/69b8cfc40a2f6a37c5980bb1.html
 *   [GROKIX] "Grok-1 中文精读" (book index page), https://yingwang.github.io/grok-1/
 *   [F2C]    "MoE 公式到源码对照",
 *            https://jerryiiii.gitbook.io/llm-review/notes/distributed/moe-formula-to-code-walkthrough
 *
 * Conventions shared by every entry point
 *  - Tensor arguments are DEVICE pointers to caller-owned memory, row-major, densely
 *    packed, 16-byte aligned. The library never frees, retains or allocates them.
 *  - `desc` is a HOST pointer; it is read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every compute
 *    entry point only enqueues work on that stream and returns; none allocates memory
 *    or synchronises, except moe_read_stats, which synchronises the stream.
 *  - Every call validates all sizes and pointers on the host BEFORE enqueuing anything;
 *    on an error nothing is launched and the outputs are untouched.
 *  - Index work (selection, histogram, slots, drop mask) is deterministic and exact.
 *    Floating-point reductions run in a fixed order, so results are bit-identical
 *    from run to run. No kernel uses global atomics.
 *  - Inputs must be finite; behaviour on NaN/Inf inputs is unspecified.
 *  - The layer returns the FFN increment only; the residual add belongs to the caller
 *    ([SERIES] §2.2 case B: a token that overflows every expert gets increment 0).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point below is exported from the shared library. */
#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

/* ---- status codes --------------------------------------------------------------- */
enum {
  MOE_OK = 0,
  MOE_E_INVAL = -1,       /* invalid size, enum, or NULL/misaligned required pointer   */
  MOE_E_UNSUPPORTED = -2, /* valid but outside what the kernels implement (see below)  */
  MOE_E_WORKSPACE = -3,   /* workspace/scratch pointer NULL or smaller than required   */
  MOE_E_HIP = -4          /* a HIP runtime call failed (launch error, no device, ...)  */
};

/* ---- enums carried in moe_desc ------------------------------------------------- */
/* Element type of x, W1, W2, W3, h, y_perm and y. W_r, logits, probs and gates are always fp32. */
enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 };

/* Gate rule ([GROK5] §5.2.3 "softmax 在 top-k 之前还是之后"):
 *  SOFTMAX_TOPK: softmax over all E experts, the k selected probabilities are the gates
 *                unnormalised (sum < 1), the Grok-1 rule.
 *  TOPK_SOFTMAX: softmax over the k selected logits only (sum = 1), the Mixtral rule;
 *                equal to renormalising the selected probabilities ([F2C] §1.2,
 *                [BOOK12] §12.1). */
enum { MOE_ROUTE_SOFTMAX_TOPK = 0, MOE_ROUTE_TOPK_SOFTMAX = 1 };

/* Noise in the selection (noise[N,E] fp32 is supplied by the caller):
 *  TOPK     : no noise; all k slots are the k largest logits.
 *  NOISY    : GShard random routing ([SERIES] §3): slot 0 is the clean argmax; slot
 *             j>=1 is the argmax, over experts not yet chosen, of fl32(logit + noise).
 *             Gates, probabilities and statistics use the clean logits.
 *  NOISY_ALL: noisy top-k gating ([GROK5] §5.2.2, logit' = logit + N(0, sigma)): the
 *             logits are replaced by logit' = fl32(logit + noise) before softmax,
 *             selection and gates; logits_out and probs_out report logit' and its
 *             softmax, and the balance statistic uses that softmax. */
enum { MOE_SECOND_TOPK = 0, MOE_SECOND_NOISY = 1, MOE_SECOND_NOISY_ALL = 2 };

/* Activation of the W1 branch: f_e(x) = [act(x W1_e) * (x W2_e)] W3_e
 * ([BOOK12] §12.1 gated FFN with SiLU; [GROK5] §5.3.5 GELU(x W_g) * (x W_v), exact erf
 * GELU, tanh form in §5.3.5.1). */
enum { MOE_ACT_SILU = 0, MOE_ACT_GELU_ERF = 1, MOE_ACT_GELU_TANH = 2 };

/* Expert buffer layout and capacity:
 *  NONE  : ragged expert-sorted rows, no capacity limit, nothing dropped; rows = N*k.
 *  PADDED: zero-padded [E, C, D] buffers with capacity C ([SERIES] §2.1, §2.3);
 *          rows = E*C; records beyond C are dropped ([F2C] §3.2). */
enum { MOE_CAP_NONE = 0, MOE_CAP_PADDED = 1 };

/* Order in which records claim capacity positions (PADDED; with NONE it only orders the
 * rows inside each expert):
 *  SLOT_MAJOR : every slot-0 record (tokens ascending) before every slot-1 record, and
 *               so on, so first choices are served before second choices.
 *  TOKEN_MAJOR: token by token, slots ascending inside a token, the loop of
 *               dispatch_to_experts ([F2C] §3.2). */
enum { MOE_PRIO_SLOT_MAJOR = 0, MOE_PRIO_TOKEN_MAJOR = 1 };

/* Capacity formula (PADDED):
 *  TOKENS_K: C = ceil(CF * N * k / E)     ([F2C] §3.1; [SERIES] §2.1)
 *  TOKENS  : C = ceil((N / E) * CF)       (Switch, no k: [SERIES] §7.2)
 * then C = max(C, min_capacity). */
enum { MOE_CAPF_TOKENS_K = 0, MOE_CAPF_TOKENS = 1 };

typedef struct moe_desc {
  int64_t N;              /* tokens (B*T flattened, [BOOK12] §12.2)                      */
  int64_t D;              /* model width                                                 */
  int64_t F;              /* expert FFN width                                            */
  int32_t E;              /* experts                                                     */
  int32_t k;              /* experts selected per token                                  */
  int32_t dtype;          /* MOE_DT_*                                                    */
  int32_t routing_mode;   /* MOE_ROUTE_*                                                 */
  int32_t second_choice;  /* MOE_SECOND_*                                                */
  int32_t activation;     /* MOE_ACT_*                                                   */
  int32_t capacity_mode;  /* MOE_CAP_*                                                   */
  int32_t min_capacity;   /* PADDED: lower bound on C (>= 0)                             */
  double capacity_factor; /* PADDED: CF > 0                                              */
  int32_t capacity_priority; /* MOE_PRIO_*                                               */
  int32_t capacity_formula;  /* MOE_CAPF_* (PADDED)                                      */
} moe_desc;

/* Limits of this implementation (MOE_E_UNSUPPORTED beyond them, MOE_E_INVAL below 1):
 *   1 <= E <= 64, 1 <= k <= min(E, 8), D and F multiples of 128,
 *   N*k, E*C and every row index fit in int32. */

/* Statistics of the last route+dispatch that used a given scratch buffer. */
typedef struct moe_stats {
  int64_t routed_slots;    /* N*k dispatch records ([BOOK12] §12.2)                      */
  int64_t dropped_slots;   /* records over capacity ([F2C] §3.3 numerator)               */
  int64_t dropped_tokens;  /* tokens with every slot dropped ([SERIES] §2.2 case B)      */
  int64_t capacity;        /* C used by the dispatch (N when capacity_mode is NONE)      */
  double drop_rate;        /* dropped_slots / (N*k), slot level ([F2C] §3.3)              */
  double token_drop_rate;  /* dropped_tokens / N                                         */
  double balance_loss;     /* E * sum_e f_e P_e, f_e = load_e/(N*k), P_e = mean_t p_te    */
  double balance_loss_div_n; /* E * sum_e (load_e/N) P_e, the ÷N form of [F2C] §2.3       */
} moe_stats;

/* Human-readable name of a status code (static string, never NULL). */
MOE_API const char* moe_status_string(int status);

/* ---- host-only queries (no GPU work; safe without a device) ---------------------- */

/* Expert capacity ([F2C] §3.1; [SERIES] §2.1 with min_capacity, §7.2 Switch form):
 *   PADDED, TOKENS_K: C = max(ceil(CF * N * k / E), min_capacity), evaluated in double
 *           as ceil(((CF*N)*k)/E). Worked example [SERIES] §2.1: N=8, E=4, k=2, CF=1 -> 4.
 *   PADDED, TOKENS  : C = max(ceil((N / E) * CF), min_capacity), evaluated in double as
 *           ceil((N/E)*CF).
 *   NONE  : C = N (no expert can receive more than N records, so nothing drops).
 * Errors: MOE_E_INVAL for NULL pointers, N<1, E<1, k<1, k>E, or CF<=0 in PADDED mode
 * (the invalid-input rule of [F2C] §3.1). */
MOE_API int moe_capacity(const moe_desc* desc, int64_t* capacity);

/* Number of rows of the expert buffers x_perm/h/y_perm: N*k (NONE) or E*C (PADDED). */
MOE_API int moe_rows(const moe_desc* desc, int64_t* rows);

/* Bytes of scratch used by moe_route, moe_dispatch, moe_expert_ffn and moe_read_stats
 * (per-block partial counts and sums; O(N*k/256*E) bytes). */
MOE_API int moe_scratch_size(const moe_desc* desc, size_t* bytes);

/* Bytes of workspace for moe_forward: the scratch region followed by every
 * intermediate (topk ids/gates, slots, x_perm, h, y_perm). */
MOE_API int moe_workspace_size(const moe_desc* desc, size_t* bytes);

/* Byte offsets of the intermediates inside a moe_forward workspace, so that a caller
 * can inspect them after moe_forward returns (the workspace keeps the last call's
 * contents). Layout of each is as in the step functions below. Exception: for bf16
 * layers with bf16 expert weights, N > 256 (or more than 4096 expert-buffer rows) and
 * experts that can hold more than 64 rows (N, or C when padded), moe_forward's
 * up-projection reads the token rows of x directly through token_of_row, so x_perm is
 * not written and the padding entries of token_of_row (PADDED) are unspecified. */
typedef struct moe_ws_layout {
  size_t scratch;        /* moe_scratch_size bytes                                      */
  size_t topk_idx;       /* int32 [N,k]                                                 */
  size_t topk_gate;      /* fp32  [N,k]                                                 */
  size_t load;           /* int32 [E]                                                   */
  size_t counts;         /* int32 [E]                                                   */
  size_t offsets;        /* int32 [E+1]                                                 */
  size_t row_of;         /* int32 [N,k]                                                 */
  size_t dropped;        /* uint8 [N,k]                                                 */
  size_t gate_eff;       /* fp32  [N,k]                                                 */
  size_t token_of_row;   /* int32 [rows]                                                */
  size_t x_perm;         /* dtype [rows,D]                                              */
  size_t h;              /* dtype [rows,F]                                              */
  size_t y_perm;         /* dtype [rows,D]                                              */
  size_t total;          /* == moe_workspace_size                                       */
} moe_ws_layout;
MOE_API int moe_workspace_layout(const moe_desc* desc, moe_ws_layout* layout);

/* ---- compute entry points (asynchronous on `stream`) ----------------------------- */

/* Router: steps "router linear in fp32 -> softmax -> top-k -> gates"
 * ([GROK5] §5.2, §5.2.1, §5.2.3; [F2C] §1.1-1.2; [SERIES] §1.1, §3).
 *   logits[t,e] = sum_d fp32(x[t,d]) * w_r[d,e] (+ logit_bias[e]), fp32 accumulation.
 *   Selection compares fp32 logits (equal to comparing probabilities, softmax being
 *   monotone per token); ties go to the LOWER expert index; slot 0 holds the largest.
 *   Gates per routing_mode / second_choice (see the enums).
 * Arguments:
 *   x          [N,D] dtype       required unless logits_in is given (then ignored)
 *   w_r        [D,E] fp32        required unless logits_in is given (then ignored)
 *   logit_bias [E]   fp32        optional additive per-expert logit bias (NULL = none)
 *   noise      [N,E] fp32        required iff second_choice is NOISY or NOISY_ALL, else ignored
 *   logits_in  [N,E] fp32        optional: route these logits and skip the GEMM
 *   logits_out [N,E] fp32        optional output of the logits
 *   probs_out  [N,E] fp32        optional output of softmax over all E
 *   topk_idx   [N,k] int32       required output, expert of each slot
 *   topk_gate  [N,k] fp32        required output, gate of each slot
 *   scratch    moe_scratch_size  optional (NULL = skip); receives the probabilities'
 *                                sums per 32-token block for the balance statistic (for
 *                                bf16 x and at most 64 tokens and 16 experts, the
 *                                probabilities themselves, which moe_read_stats adds up
 *                                in the same blocks), and with bf16 x the working data of
 *                                the logit GEMM. */
MOE_API int moe_route(const moe_desc* desc, const void* x, const float* w_r, const float* logit_bias,
              const float* noise, const float* logits_in, float* logits_out, float* probs_out,
              int32_t* topk_idx, float* topk_gate, void* scratch, size_t scratch_bytes,
              void* stream);

/* Dispatch: load histogram, capacity slots, drop rule and gather
 * ([F2C] §1.3 load, §3.1-3.2 capacity and dropped mask; [SERIES] §2.2 overflow cases,
 *  §2.3 zero padding; [BOOK12] §12.2 expert-grouped buffers).
 *   load[e]   = #{(t,j): topk_idx[t,j] = e}   (before capacity)
 *   Positions inside an expert are assigned in the order of capacity_priority
 *   (MOE_PRIO_*: slot-major by default, or token-major); a record is kept iff its
 *   position < C.
 *   counts[e] = min(load[e], C) rows filled; offsets[e] = first row of expert e
 *   (NONE: exclusive scan of counts; PADDED: e*C); offsets[E] = rows.
 *   row_of[t,j] = row of the record, or -1 if dropped; dropped[t,j] = 1 if dropped.
 *   gate_eff: all slots kept -> the gates; none kept -> 0; otherwise each kept slot
 *   gets g_j * (sum of all gates) / (sum of kept gates) and dropped slots 0 (for two
 *   renormalised gates with the 2nd dropped this is (1,0), [SERIES] §2.2 case A).
 *   token_of_row[r] = token of row r, -1 for padding rows.
 *   x_perm[r,:] = x[token_of_row[r],:], zero for padding rows.
 * Arguments: x [N,D] dtype; topk_idx, topk_gate as produced by moe_route; outputs
 *   load [E], counts [E], offsets [E+1] int32; row_of [N,k] int32; dropped [N,k] uint8;
 *   gate_eff [N,k] fp32; token_of_row [rows] int32; x_perm [rows,D] dtype.
 *   scratch (moe_scratch_size bytes) is required. Every pointer is required.
 *   topk_idx entries must lie in [0,E) and be distinct per token (as moe_route makes). */
MOE_API int moe_dispatch(const moe_desc* desc, const void* x, const int32_t* topk_idx,
                 const float* topk_gate, int32_t* load, int32_t* counts, int32_t* offsets,
                 int32_t* row_of, uint8_t* dropped, float* gate_eff, int32_t* token_of_row,
                 void* x_perm, void* scratch, size_t scratch_bytes, void* stream);

/* Expert FFN as two grouped GEMMs over the expert buffers ([BOOK12] §12.1 gated FFN;
 * [GROK5] §5.3.5):
 *   h[r,:]      = act(x_perm[r,:] W1_e) * (x_perm[r,:] W2_e)      (stored in dtype)
 *   y_perm[r,:] = h[r,:] W3_e
 * for every row r in [offsets[e], offsets[e] + counts[e]). Rows outside those ranges
 * (padding rows of the PADDED layout) are left unspecified.
 * Arguments: x_perm [rows,D], w1 and w2 [E,D,F], w3 [E,F,D], h [rows,F], y_perm [rows,D],
 *   all dtype; offsets [E+1], counts [E] int32 as produced by moe_dispatch.
 *   scratch (moe_scratch_size bytes) is required. Accumulation is fp32. */
MOE_API int moe_expert_ffn(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                   const int32_t* counts, const void* w1, const void* w2, const void* w3,
                   void* h, void* y_perm, void* scratch, size_t scratch_bytes, void* stream);

/* The two halves of moe_expert_ffn, for callers that schedule or time them apart:
 *   moe_expert_up  : h = act(x_perm W1_e) * (x_perm W2_e)   (the gated up-projection)
 *   moe_expert_down: y_perm = h W3_e                          (the down-projection)
 * Arguments, row ranges and errors as for moe_expert_ffn. */
MOE_API int moe_expert_up(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                  const int32_t* counts, const void* w1, const void* w2, void* h, void* scratch,
                  size_t scratch_bytes, void* stream);
MOE_API int moe_expert_down(const moe_desc* desc, const void* h, const int32_t* offsets,
                    const int32_t* counts, const void* w3, void* y_perm, void* scratch,
                    size_t scratch_bytes, void* stream);

/* The gated up-projection with its rows taken from x instead of x_perm: buffer row r of
 * expert e reads x[token_of_row[r],:] (token_of_row as written by moe_dispatch), so the
 * gather of moe_dispatch is not needed. h equals moe_expert_up's result on the gathered
 * x_perm bit for bit. This is the form moe_forward runs for bf16 layers whose experts may
 * hold more than 64 rows (the skinny decode regime and fp32 layers keep x_perm); for
 * other layers it returns MOE_E_UNSUPPORTED. Arguments: x [N,D] and h [rows,F] bf16;
 * token_of_row [rows] int32; the rest as for moe_expert_up. */
MOE_API int moe_expert_up_gathered(const moe_desc* desc, const void* x, const int32_t* token_of_row,
                           const int32_t* offsets, const int32_t* counts, const void* w1, const void* w2,
                           void* h, void* scratch, size_t scratch_bytes, void* stream);

/* Combine ([GROK5] §5.3.5 gate-weighted sum, §5.8; [BOOK12] §12.2 accumulate, not
 * overwrite): y[t,:] = sum over kept slots j, in slot order, of
 * gate_eff[t,j] * y_perm[row_of[t,j],:], accumulated in fp32 and rounded once to dtype;
 * exactly 0 for a token with every slot dropped.
 * Arguments: y_perm [rows,D] dtype; row_of [N,k] int32; gate_eff [N,k] fp32; y [N,D]. */
MOE_API int moe_combine(const moe_desc* desc, const void* y_perm, const int32_t* row_of,
                const float* gate_eff, void* y, void* stream);

/* The whole layer: moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine with every
 * intermediate in `workspace` (moe_workspace_size bytes, laid out as
 * moe_workspace_layout reports; see there for when x_perm is not materialised).
 * Arguments as in the step functions; y [N,D] dtype, equal bit for bit to the step
 * functions' result. */
MOE_API int moe_forward(const moe_desc* desc, const void* x, const float* w_r, const float* logit_bias,
                const float* noise, const void* w1, const void* w2, const void* w3, void* y,
                void* workspace, size_t workspace_bytes, void* stream);

/* The layer forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward with its
 * workspace in a static device array of MOE_NOALLOC_WORKSPACE_BYTES that the library
 * holds on each GPU it runs on until the process ends. Calls no allocating routine.
 * Arguments, results and errors as for moe_forward (y equal to its result bit for bit),
 * except: no workspace argument; MOE_E_WORKSPACE if moe_workspace_size(desc) exceeds
 * MOE_NOALLOC_WORKSPACE_BYTES (e.g. Mixtral-shaped decode batches fit, prefill batches do
 * not); MOE_E_INVAL if `stream` belongs to another device than the current one.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different host threads) race and must be serialised by the
 * caller. The array keeps the previous call's intermediates; nothing in the forward
 * depends on their initial contents. */
#define MOE_NOALLOC_WORKSPACE_BYTES (128u << 20)
MOE_API int moe_forward_noalloc(const moe_desc* desc, const void* x, const float* w_r, const float* logit_bias,
                        const float* noise, const void* w1, const void* w2, const void* w3, void* y,
                        void* stream);

/* ---- weight-only 8-bit experts ------------------------------------------------------
 * Grok-1 keeps its expert weights 8-bit and dequantises them right before the expert
 * matmul, weight = weight * scales ([GROK5] §5.3.3 moe_slow_matmul1 and §5.3.4 moe_slow_matmul2). Here:
 *   W1q, W2q [E,D,F] int8, W3q [E,F,D] int8, with fp32 scales s1, s2 [E,F] and s3 [E,D]:
 *   the dequantised weight is W[e,k,n] = q[e,k,n] * s[e,n], one scale per expert and
 *   output column, broadcast over the input dimension (the pages print the scales as
 *   having the weight's shape; a per-column scale is that array broadcast along K).
 * The expert FFN then equals moe_expert_ffn on the dequantised weights, up to rounding:
 * the int8 values are widened exactly to bf16 for the matrix cores, products accumulate
 * in fp32 and the column scale multiplies the fp32 sum before the activation / store.
 * desc->dtype must be MOE_DT_BF16 (MOE_E_UNSUPPORTED otherwise); every scale pointer is
 * required and 16-byte aligned (MOE_E_INVAL). Everything else as for the bf16 entry
 * points above: arguments, scratch, row ranges, errors. */
MOE_API int moe_expert_up_q8(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                     const int32_t* counts, const int8_t* w1, const float* s1, const int8_t* w2,
                     const float* s2, void* h, void* scratch, size_t scratch_bytes, void* stream);
MOE_API int moe_expert_down_q8(const moe_desc* desc, const void* h, const int32_t* offsets,
                       const int32_t* counts, const int8_t* w3, const float* s3, void* y_perm,
                       void* scratch, size_t scratch_bytes, void* stream);
MOE_API int moe_expert_ffn_q8(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                      const int32_t* counts, const int8_t* w1, const float* s1, const int8_t* w2,
                      const float* s2, const int8_t* w3, const float* s3, void* h, void* y_perm,
                      void* scratch, size_t scratch_bytes, void* stream);
MOE_API int moe_forward_q8(const moe_desc* desc, const void* x, const float* w_r, const float* logit_bias,
                   const float* noise, const int8_t* w1, const float* s1, const int8_t* w2,
                   const float* s2, const int8_t* w3, const float* s3, void* y, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Reduces the statistics left in `scratch` (or in a moe_forward workspace, whose first
 * moe_scratch_size bytes are the scratch) by the last moe_route + moe_dispatch on it,
 * copies them to *out and SYNCHRONISES `stream`. balance_loss fields are 0 if moe_route
 * ran without scratch. */
MOE_API int moe_read_stats(const moe_desc* desc, const void* scratch, size_t scratch_bytes,
                   moe_stats* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
