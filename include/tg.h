/*
 * tg.h -- C ABI of the TokenGate gated-prefill library (libtokengate.so).
 *
 * TokenGate ("Researchers from Stanford and UC Berkeley Introduce TokenGate:
 * Token-Gated Attention Makes Long-Context Prefill Up to 11.3x Faster",
 * MarkTechPost) splits prefill into three phases (section "How does TokenGate
 * learned token pruning work?"): a standard forward below the gate layer, a
 * gate module (an MLP scores every token, a top-K selector keeps the best
 * document tokens, the question is never pruned), and a pruned forward that
 * sees only the kept tokens.  Section "What is token-gated attention?" turns
 * each kept token's score into an additive bias on the attention logits, with
 * a per-head gain and a temperature.  The calls below are the device side of
 * phases two and three:
 *
 *   tg_plan            host-only sizes of the kept set (no device work)
 *   tg_sample_budgets  host-only random document budgets (training's
 *                      random-budget loss)
 *   tg_gate_score      gate MLP score of every token
 *   tg_select_topk     per-prompt top-K over the document span -> keep flags
 *   tg_compact         stable gather of kept rows, positions and biases
 *   tg_gated_attn_fwd  causal GQA attention over the kept tokens with the
 *                      score bias: logit = tau * q.k / sqrt(d) + g_h * s_j
 *   tg_gated_attn_bwd  its backward: dq, dk, dv and the gradients of the
 *                      bias, the gains and the temperature
 *   tg_gate_bwd        backward of the gate MLP from the kept rows' bias
 *                      gradient (the scorer's gradient path)
 *   tg_kv_scatter      the prefill's kept k, v and bias into a decode cache
 *   tg_kv_append       a decode step's new k, v into the cache (bias 0)
 *   tg_decode_attn     one decode step of token-gated attention over the
 *                      kept-only cache
 *   tg_rope_table      cos / sin of the rotary embedding at the kept rows'
 *                      original positions
 *   tg_qkv_rope        fused q/k/v projection of the kept rows, rotated at
 *                      their original positions (the pruned layers' input)
 *   tg_rms_norm        RMSNorm of the kept rows (before attention and MLP)
 *   tg_linear_residual projection added to the residual stream (attention
 *                      output projection, MLP down projection)
 *   tg_swiglu          the MLP's gate and up projections with SiLU(gate) * up
 *
 * Conventions (every call):
 *   - Pointers are device pointers unless the parameter name ends in _h
 *     (host).  The caller owns every buffer; the library allocates nothing
 *     and keeps no state between calls.
 *   - A call checks its arguments on the host first.  An invalid call
 *     returns a negative tg_status before any device work and has no side
 *     effect.  A valid call enqueues its kernels on `stream` (a hipStream_t;
 *     NULL means the default stream) and returns TG_OK without waiting.  A
 *     failed launch returns TG_ERR_HIP.
 *   - Outputs never alias inputs.  Token indices are int32, sizes int64.
 *   - Packed prompts: prompt b owns tokens [cu_seqlens[b], cu_seqlens[b+1]);
 *     cu_seqlens[0] == 0, non-decreasing, cu_seqlens[B] == T.  Its document
 *     is the prompt-relative span [doc_begin[b], doc_end[b]).
 *   - Every output is bit-reproducible from run to run (no float atomics).
 */
#ifndef TOKENGATE_TG_H
#define TOKENGATE_TG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_ABI_VERSION 1

typedef enum {
  TG_OK = 0,
  TG_ERR_NULL = -1,        /* a required pointer is NULL */
  TG_ERR_SHAPE = -2,       /* a size or stride is negative or inconsistent */
  TG_ERR_DTYPE = -3,       /* unknown dtype code */
  TG_ERR_RANGE = -4,       /* a scalar argument is out of range (e.g. tau not finite) */
  TG_ERR_ALIGN = -5,       /* a pointer or stride breaks the 16-byte rule */
  TG_ERR_UNSUPPORTED = -6, /* valid, but a shape the library has no kernel for */
  TG_ERR_WORKSPACE = -7,   /* workspace NULL or smaller than the *_workspace size */
  TG_ERR_HIP = -8          /* the HIP runtime reported an error at launch */
} tg_status;

typedef enum { TG_F32 = 0, TG_BF16 = 1 } tg_dtype;

/* TG_ABI_VERSION of the built library. */
int tg_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* tg_status_string(int status);

/*
 * Kept-set sizes, on the host (article, "How does TokenGate learned token
 * pruning work?": only the document is prunable; "How do you deploy
 * TokenGate?": generation takes a budget on kept prefill tokens).  The budget
 * counts document tokens: prompt b keeps min(budget_h[b], doc length) document
 * tokens plus all its other tokens.
 *
 * In (host, [B] or [B+1]): cu_seqlens_h, doc_begin_h, doc_end_h, budget_h.
 * Out (host): cu_kept_h[B+1] exclusive prefix of kept counts (cu_kept_h[B] is
 * the total Kt), *max_kept_len_h the longest kept prompt.
 * Errors: TG_ERR_NULL, TG_ERR_SHAPE (B < 0, cu_seqlens not a prefix, a doc span
 * outside its prompt, a negative budget, Kt > INT32_MAX).
 */
int tg_plan(int B, const int32_t* cu_seqlens_h, const int32_t* doc_begin_h,
            const int32_t* doc_end_h, const int32_t* budget_h,
            int32_t* cu_kept_h, int32_t* max_kept_len_h);

/*
 * Random document budgets (host only; section "What is token-gated
 * attention?": each training step averages a full-context loss and a
 * random-budget loss).  Prompt b keeps the fraction
 *     f_b = min_frac + (max_frac - min_frac) * u_h[b]
 * of its document: budget_h[b] = floor(f_b * (doc_end_h[b] - doc_begin_h[b]))
 * in double precision.  u_h [B]: the caller's uniform draws in [0, 1).
 * 0 <= min_frac <= max_frac <= 1, else TG_ERR_RANGE.  Random-K selection
 * (the ablation that keeps K random document tokens) needs no call of its
 * own: tg_select_topk over i.i.d. uniform keys keeps a uniformly random
 * K-subset of each document; the compaction still takes the gate scores.
 */
int tg_sample_budgets(int B, const int32_t* doc_begin_h, const int32_t* doc_end_h,
                      const float* u_h, float min_frac, float max_frac, int32_t* budget_h);

/*
 * Gate score of every token (article, "How does TokenGate learned token
 * pruning work?": an MLP scores each token from its post-attention residual):
 *     s_t = b2 + sum_f w2[f] * SiLU(b1[f] + sum_k W1[f,k] * hidden[t,k])
 * with SiLU(a) = a / (1 + exp(-a)), fp32 accumulation and an fp32 epilogue.
 *
 * hidden  [T, D] row-major, row stride ld_hidden elements (>= D), dtype.
 * W1      [F, D] row-major, dtype.   b1 [F] fp32 or NULL (zero).
 * w2      [F] fp32.  b2 scalar.      scores [T] fp32 out.
 * Supported: TG_BF16 with D % 8 == 0, F in {64, 128, 256} and a row stride
 * below 2^22 elements, or
 * TG_F32 with any D >= 1 and 1 <= F <= 1024.  bf16 needs hidden, W1 and the
 * row stride aligned to 16 bytes.  T == 0 is a no-op.
 */
int tg_gate_score(const void* hidden, int64_t ld_hidden, int64_t T, int D,
                  const void* W1, const float* b1, const float* w2, float b2,
                  int F, int dtype, float* scores, void* stream);

/* Workspace bytes that tg_select_topk needs for B prompts over T tokens. */
int tg_select_topk_workspace(int B, int64_t T, size_t* bytes);

/*
 * Document-only top-K (article, "How does TokenGate learned token pruning
 * work?": a top-K selector keeps the highest-scoring tokens; only the
 * document part is prunable).  For each prompt b keeps the k = min(budget[b],
 * doc length) document tokens ranked first by (score descending, token index
 * ascending) and every token outside the document.  -0.0 ranks equal to
 * +0.0; NaN ranks below every number, NaNs tied by index.
 *
 * scores [T] fp32; cu_seqlens [B+1], doc_begin/doc_end/budget [B] int32 (all
 * device, same values as given to tg_plan); keep [T] uint8 out (1 = kept).
 * workspace: device memory of at least tg_select_topk_workspace() bytes, any
 * contents on entry, clobbered.  Device arguments are trusted to satisfy the
 * rules tg_plan checks; T must equal cu_seqlens[B].  Supported: B <= 65535.
 */
int tg_select_topk(const float* scores, const int32_t* cu_seqlens,
                   const int32_t* doc_begin, const int32_t* doc_end,
                   const int32_t* budget, int B, int64_t T, uint8_t* keep,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * tg_select_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and checks as
 * tg_select_topk; the workspace is a static device array inside the library
 * (4 MiB, one copy per GPU, held until the process ends).  The call itself
 * allocates nothing: on its first use on a device it only looks up that
 * array's address (the array of the stream's device; of the current device
 * for the null stream).
 * Limit: the tg_select_topk_workspace size of (B, T) must fit in 4 MiB when
 * T > 32768 (about B <= 190 prompts at any T; T <= 32768 needs no scratch),
 * else TG_ERR_WORKSPACE before any device work.
 * Every call on a GPU shares that GPU's array: calls that can overlap on one
 * GPU (other streams, other host threads) race and must be serialized by the
 * caller.  Nothing in the array needs clearing between calls.
 */
int tg_select_topk_noalloc(const float* scores, const int32_t* cu_seqlens,
                           const int32_t* doc_begin, const int32_t* doc_end,
                           const int32_t* budget, int B, int64_t T, uint8_t* keep,
                           void* stream);

/* Workspace bytes that tg_compact needs for B prompts over T tokens. */
int tg_compact_workspace(int B, int64_t T, size_t* bytes);

/*
 * Stable compaction of the kept tokens (article, "How does TokenGate learned
 * token pruning work?": layers above the gate process only the kept tokens;
 * "What is token-gated attention?": the kept token's score becomes its bias).
 * Kept token t (ascending t, so prompt by prompt) goes to row r = number of
 * kept tokens before t:
 *     hidden_out[r, :] = hidden[t, :]            (bytes copied exactly)
 *     pos_out[r]       = pos[t], or t - cu_seqlens[b] when pos == NULL
 *     bias_out[r]      = scores[t] inside the document, +0.0 outside
 *     kept_idx_out[r]  = t                       (optional, may be NULL)
 *
 * hidden [T, D] row stride ld_hidden; hidden_out [Kt, D] packed; dtype gives
 * the element size (the copy is a byte copy).  Kt must equal the number of
 * kept flags (tg_plan's total).  hidden and hidden_out need element
 * alignment only; rows move in 16-byte units when the row size, the row
 * stride and both base pointers are multiples of 16 bytes, else element by
 * element.  workspace as for tg_select_topk.
 */
int tg_compact(const void* hidden, int64_t ld_hidden, int D, int dtype,
               const int32_t* pos, const float* scores, const uint8_t* keep,
               const int32_t* cu_seqlens, const int32_t* doc_begin,
               const int32_t* doc_end, int B, int64_t T, int64_t Kt,
               void* hidden_out, int32_t* pos_out, float* bias_out,
               int32_t* kept_idx_out, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * Token-gated causal GQA attention over the kept tokens (article, "What is
 * token-gated attention?": the kept token's score is an additive logit bias,
 * refined by a per-head gain and a temperature).  For prompt b (kept rows
 * [cu_kept[b], cu_kept[b+1])), query head h, KV head h / (Hq / Hkv), and
 * kept row i:
 *     x_j  = tau * (q_i . k_j) / sqrt(d) + gain[h] * bias_s[j],  j <= i in b
 *     o_i  = sum_j softmax(x)_j * v_j
 *     lse_i = ln sum_j exp(x_j)
 * gain == NULL drops the bias term (plain causal attention with temperature).
 * tau must be finite and positive (a temperature), else TG_ERR_RANGE.
 *
 * q [Kt, Hq, d], k and v [Kt, Hkv, d]: heads contiguous inside a token, token
 * strides in elements (>= heads * d).  bias_s [Kt] fp32 (may be NULL only when
 * gain is NULL), gain [Hq] fp32, cu_kept [B+1] int32 (device copy of
 * tg_plan's output), max_kept_len its longest prompt.  out [Kt, Hq, d]
 * packed, same dtype as q.  lse [Hq, Kt] fp32, or NULL.
 * Supported: d in {64, 128}, Hq % Hkv == 0, k and v token strides up to
 * 2^23 elements, B <= 65535, max_kept_len <= 65535 * 256 (bf16) and
 * Hq <= 65535 (fp32).  bf16 runs on MFMA with fp32
 * accumulation and rounds the softmax weights to bf16 before the value
 * product; fp32 runs on vector ALUs throughout.  bf16 needs q, k, v, out and
 * the token strides aligned to 16 bytes.
 */
int tg_gated_attn_fwd(const void* q, const void* k, const void* v,
                      int64_t q_tok_stride, int64_t k_tok_stride,
                      int64_t v_tok_stride, const float* bias_s,
                      const float* gain, float tau, const int32_t* cu_kept,
                      int B, int max_kept_len, int64_t Kt, int Hq, int Hkv,
                      int d, int dtype, void* out, float* lse, void* stream);

/* Workspace bytes that tg_gated_attn_bwd needs for these shapes and dtype
 * (bf16 with Hq > Hkv adds 2 Hq Kt d fp32 per-head dK and dV sums). */
int tg_gated_attn_bwd_workspace(int B, int64_t Kt, int Hq, int Hkv, int d, int dtype,
                                int max_kept_len, size_t* bytes);

/*
 * Backward of tg_gated_attn_fwd (section "What is token-gated attention?":
 * top-K is not differentiable, so the kept token's score enters the
 * attention as a logit bias, which gives the loss a gradient path back to
 * the scorer; the per-head gain and the temperature are learned too).
 * Gradients of sum(dout * out) with, over visible keys j <= i of a prompt,
 *     x_ij = tau q_i.k_j / sqrt(d) + g_h s_j,  P = softmax_j(x),
 *     dx_ij = P_ij (dout_i.v_j - dout_i.out_i):
 *     dq_i = tau/sqrt(d) sum_j dx_ij k_j
 *     dk_j = tau/sqrt(d) sum_(h in group, i) dx_ij q_i
 *     dv_j = sum_(h in group, i) P_ij dout_i
 *     dbias_j = sum_h g_h sum_i dx_ij      dgain_h = sum_ij dx_ij s_j
 *     dtau = sum_(h, ij) dx_ij q_i.k_j / sqrt(d)
 * P is recomputed from lse, which must be the forward's (tg_gated_attn_fwd
 * with the same inputs and lse != NULL); out is the forward's output.
 * Inputs as tg_gated_attn_fwd (q, k, v with token strides); out, dout and dq
 * packed [Kt, Hq, d], dk and dv packed [Kt, Hkv, d], all in dtype; dbias
 * [Kt], dgain [Hq] and dtau [1] fp32, each may be NULL (not computed);
 * with gain == NULL they are zero.  The gradient of a kept token's gate
 * score is dbias_j inside the document (the bias there is the score) and
 * nothing outside it (the bias there is a constant 0).
 * bf16: the MFMA products take bf16 operands (P and dx rounded to bf16
 * before the second products) with fp32 accumulation; dx, the column sums
 * and the reductions are fp32.  Every sum runs in a fixed order.
 * Supported: as tg_gated_attn_fwd, with token strides and Hq*d up to 2^23
 * elements, max_kept_len <= 65535 * 128.  workspace >= the size from
 * tg_gated_attn_bwd_workspace, 16-byte aligned.
 */
int tg_gated_attn_bwd(const void* q, const void* k, const void* v, int64_t q_tok_stride,
                      int64_t k_tok_stride, int64_t v_tok_stride, const float* bias_s,
                      const float* gain, float tau, const int32_t* cu_kept, int B,
                      int max_kept_len, int64_t Kt, int Hq, int Hkv, int d, int dtype,
                      const void* out, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, float* dbias, float* dgain, float* dtau, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes that tg_gate_bwd needs. */
int tg_gate_bwd_workspace(int64_t Kt, int D, int F, int dtype, size_t* bytes);

/*
 * Backward of the gate MLP (section "What is token-gated attention?": the
 * kept token's score is its attention bias above the gate, the scorer's
 * gradient path; top-K passes none).  dbias [Kt] fp32 is the bias gradient
 * of the kept rows (tg_gated_attn_bwd's dbias summed over the pruned
 * layers).  Row r's token t = kept_idx[r] gets ds_t = dbias[r] when t lies
 * in its prompt's document (the bias there is the score) and 0 otherwise;
 * every other token gets nothing.  With a_r = W1 h_r + b1 (h_r = hidden_k
 * row r, the gate input of token t):
 *     da_r = ds_r w2 * silu'(a_r)    dhidden_k[r] = W1^T da_r
 *     dW1 = sum_r da_r h_r^T   db1 = sum_r da_r   dw2 = sum_r ds_r silu(a_r)
 *     db2 = sum_r ds_r
 * hidden_k [Kt, D] row stride ld_hidden (tg_compact's hidden_out), W1
 * [F, D] in its dtype; b1 [F] (may be NULL), w2 [F] fp32, 16-byte aligned;
 * kept_idx [Kt] int32 (tg_compact's kept_idx_out); cu_seqlens [B+1],
 * doc_begin / doc_end [B] as for tg_select_topk (device).  Outputs:
 * dhidden_k [Kt, D] packed in the dtype; dW1 [F, D], db1 [F] (may be NULL),
 * dw2 [F], db2 [1] fp32.  bf16: MFMA for the three products (da rounded to
 * bf16 for dhidden_k and dW1), fp32 sums in fixed order.  Supported:
 * F in {64, 128, 256}; bf16 needs D % 64 == 0, ld_hidden and D below 2^22,
 * aligned pointers and row stride.  workspace >= tg_gate_bwd_workspace.
 */
int tg_gate_bwd(const void* hidden_k, int64_t ld_hidden, int64_t Kt, int D, const void* W1,
                const float* b1, const float* w2, int F, const float* dbias,
                const int32_t* kept_idx, const int32_t* cu_seqlens, const int32_t* doc_begin,
                const int32_t* doc_end, int B, int dtype, void* dhidden_k, float* dW1, float* db1,
                float* dw2, float* db2, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over the kept-only KV cache (section "How does TokenGate learned
 * token pruning work?": the layers above the gate never create KV entries
 * for pruned tokens, so generation reads only the kept ones; "What is
 * token-gated attention?": a kept token's score is its bias).  The bias is
 * persistent: a document key keeps its gate score, question and generated
 * keys carry 0.
 *
 * Cache of one pruned layer: k_cache, v_cache [rows, Hkv, d] with token
 * strides cache_k_stride / cache_v_stride (elements, >= Hkv*d, multiples of
 * 16 bytes), bias_cache [rows] fp32.  Sequence b owns rows start[b] ..
 * start[b] + len - 1 (start [B] int32, device), with room after them for
 * its generated tokens; the caller tracks the lengths.
 *
 * tg_kv_scatter: kept row r of prompt b (rows [cu_kept[b], cu_kept[b+1]) of
 * k, v [Kt, Hkv, d] with token strides, bias_s [Kt] or NULL for 0) goes to
 * cache row start[b] + r - cu_kept[b].
 */
int tg_kv_scatter(const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
                  const float* bias_s, const int32_t* cu_kept, int B, int64_t Kt, int Hkv, int d,
                  int dtype, void* k_cache, void* v_cache, int64_t cache_k_stride,
                  int64_t cache_v_stride, float* bias_cache, const int32_t* start, void* stream);

/* tg_kv_append: k_new, v_new packed [B, Hkv, d] go to cache row
 * start[b] + pos[b] (pos [B] int32, device: the length before the step);
 * their bias is 0. */
int tg_kv_append(const void* k_new, const void* v_new, int B, int Hkv, int d, int dtype,
                 void* k_cache, void* v_cache, int64_t cache_k_stride, int64_t cache_v_stride,
                 float* bias_cache, const int32_t* start, const int32_t* pos, void* stream);

/* Workspace bytes that tg_decode_attn needs. */
int tg_decode_attn_workspace(int B, int Hq, int d, int max_len, size_t* bytes);

/* One decode step: for sequence b (lens[b] cached keys, the new token's own
 * included; lens [B] int32, device, each <= max_len), query head h (KV head
 * h / (Hq / Hkv)):
 *     x_j = tau * q_bh . k_j / sqrt(d) + gain[h] * bias_cache[j]
 *     out[b, h] = softmax(x) v,   lse[b, h] = ln sum_j exp(x_j)
 * q and out packed [B, Hq, d] in dtype; lse [B, Hq] fp32 or NULL; gain
 * NULL drops the bias term.  A sequence of length 0 gives NaN.  Vector-ALU
 * kernel (a step reads each cached key once: HBM-bound), fp32 arithmetic.
 * Each sequence's keys are cut into splits merged in a fixed order: splits
 * of 128 keys, or of 256 keys when B * Hkv * ceil(max_len / 256) >= 2048
 * (enough workgroups to fill the chip).  The split size sets the order of
 * the sums, so a sequence's output can differ in its last bits between
 * calls whose B or max_len put them on different sides of that rule; calls
 * with the same arguments give identical bits.  Supported: d in {64, 128},
 * Hq / Hkv <= 8, max_len <= 65535 * 128; q, caches and workspace 16-byte
 * aligned.
 */
int tg_decode_attn(const void* q, const void* k_cache, const void* v_cache, int64_t cache_k_stride,
                   int64_t cache_v_stride, const float* bias_cache, const float* gain, float tau,
                   const int32_t* start, const int32_t* lens, int B, int max_len, int Hq, int Hkv,
                   int d, int dtype, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Rotary table of the kept rows (section "How does TokenGate learned token
 * pruning work?": the pruned forward keeps each kept token's original
 * position id).  For row t and frequency index i < d/2:
 *     a = pos[t] * rope_theta^(-2 i / d)
 *     table[t, i] = (cos a, sin a)
 * evaluated in fp64 and stored as an fp32 pair.  pos [Kt] int32 (device,
 * e.g. tg_compact's pos_out); table [Kt, d/2, 2] fp32, 16-byte aligned.
 * rope_theta is the rotary base (1e6 for the Qwen3 family), finite and > 1,
 * else TG_ERR_RANGE.  d in {64, 128}.  The table depends on the positions
 * only: a pruned forward builds it once and every layer reuses it.
 */
int tg_rope_table(const int32_t* pos, int64_t Kt, int d, double rope_theta, float* table,
                  void* stream);

/* Attention inputs of a pruned layer (section "How does TokenGate learned
 * token pruning work?": the layers above the gate process the kept tokens
 * only, at their original positions).  For kept row t:
 *     y_t = W_qkv . x_t          W_qkv [(Hq + 2 Hkv) d, D], rows: the Hq q
 *                                heads, then the Hkv k heads, then the Hkv
 *                                v heads, d rows each
 * then every q and k head is rotated in the rotate-half form with row t of
 * rope_table (tg_rope_table, same d): for i < d/2, (c, s) = table[t, i],
 *     y_i       <- y_i c - y_{i+d/2} s
 *     y_{i+d/2} <- y_{i+d/2} c + y_i s
 * and the v heads are stored as projected.  No bias, no per-head norm.
 *
 * x [Kt, D] with token stride ld_x (>= D) elements, e.g. tg_compact's
 * hidden_out; w_qkv packed [(Hq + 2 Hkv) d, D]; qkv [Kt, (Hq + 2 Hkv) d]
 * with token stride ld_qkv (>= (Hq + 2 Hkv) d): q at column 0, k at Hq d,
 * v at (Hq + Hkv) d, so that tg_gated_attn_fwd reads q, k and v in place
 * with token strides ld_qkv.  x, w_qkv and qkv share the dtype.
 * Supported: d in {64, 128}; bf16 needs D % 64 == 0, ld_x and D below 2^22,
 * x, w_qkv, qkv and rope_table 16-byte aligned and ld_x, ld_qkv multiples
 * of 8; fp32 needs Kt * (Hq + 2 Hkv) d < 2^31 and an aligned rope_table.
 * bf16 runs on MFMA with fp32 accumulation, rotates in fp32 and rounds to
 * bf16 once; fp32 runs on vector ALUs.
 */
int tg_qkv_rope(const void* x, int64_t ld_x, int64_t Kt, int D, const void* w_qkv,
                const float* rope_table, int Hq, int Hkv, int d, int dtype, void* qkv,
                int64_t ld_qkv, void* stream);

/* The rest of a pruned layer (section "How does TokenGate learned token
 * pruning work?": the layers above the gate process the kept tokens only).
 * Reading: a pre-norm layer of the Qwen3 family, the model the article
 * names,
 *     a = x + W_o . attention(tg_qkv_rope(tg_rms_norm(x)))
 *     y = a + W_down . tg_swiglu(tg_rms_norm(a))
 * with the attention of tg_gated_attn_fwd.  No biases.
 *
 * RMSNorm of every row: out[t, c] = weight[c] * x[t, c] / sqrt(mean_c(x[t, :]^2) + eps),
 * computed in fp32 (sum of squares in a fixed order), rounded once to the
 * output dtype.  x [n, D] row stride ld_x, out [n, D] row stride ld_out,
 * same dtype; weight [D] fp32.  out may be x itself (same pointer and
 * stride), no other overlap.  eps finite and >= 0 (1e-6 in the Qwen3
 * family), else TG_ERR_RANGE.  Supported: D % 8 == 0; x, out, weight
 * 16-byte aligned, row strides multiples of 16 bytes.
 */
int tg_rms_norm(const void* x, int64_t ld_x, int64_t n, int D, const float* weight, float eps,
                int dtype, void* out, int64_t ld_out, void* stream);

/* out[t, :] = residual[t, :] + W . a[t, :]: a [n, K] row stride ld_a,
 * W [N, K] packed, residual and out [n, N] with row strides ld_res and
 * ld_out, one dtype.  The attention output projection (a = the attention
 * output [Kt, Hq d], W = W_o [D, Hq d]) and the MLP's down projection
 * (a = the SwiGLU activation [Kt, I], W = W_down [D, I]).  out may be the
 * residual itself (same pointer and stride), no other overlap.
 * bf16: MFMA with fp32 accumulation, the residual added in fp32, one
 * rounding; needs K % 64 == 0, N % 64 == 0, ld_a and K below 2^22, 16-byte
 * aligned pointers and row strides.  fp32: vector ALUs, n * N < 2^31,
 * element alignment.
 */
int tg_linear_residual(const void* a, int64_t ld_a, int64_t n, int K, const void* W, int N,
                       const void* residual, int64_t ld_res, int dtype, void* out, int64_t ld_out,
                       void* stream);

/* The MLP's activation: out[t, j] = silu(W_gate[j] . h[t]) * (W_up[j] . h[t]),
 * silu(z) = z / (1 + exp(-z)).  h [n, D] row stride ld_h; W_gate and W_up
 * [I, D] packed; out [n, I] row stride ld_out; one dtype.  bf16: both
 * products on MFMA in one pass (a tile stages 128 rows of W_gate and the
 * same rows of W_up), fp32 accumulation, one rounding; needs D % 64 == 0,
 * I % 32 == 0, ld_h and D below 2^22, 16-byte aligned pointers and row
 * strides.  fp32: vector ALUs, n * I < 2^31, element alignment.
 */
int tg_swiglu(const void* h, int64_t ld_h, int64_t n, int D, const void* w_gate, const void* w_up,
              int I, int dtype, void* out, int64_t ld_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_TG_H */
