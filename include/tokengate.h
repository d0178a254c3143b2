/*
 * tokengate.h - C ABI of the TokenGate pruned-prefill layer for MI355X (gfx950).
 *
 * The layer runs in four steps:
 *
 *   1. tg_gate_score       a small MLP scores every token from its residual at
 *                          the gate layer;
 *   2. tg_select_topk      per prompt, keep the best-scored document rows and
 *                          every row outside the document (the question);
 *   3. tg_compact          gather the kept rows of any number of row-major
 *                          tensors (hidden states, Q, K, V), their original
 *                          positions and their attention bias;
 *   4. tg_gated_attention  causal attention over the kept rows only, with the
 *                          bias of every kept key added to its logits.
 *
 * Beyond the forward pass: tg_gated_attention_backward, tg_score_grad and
 * tg_gate_backward carry a gradient from the attention output through the
 * bias back to the gate's weights (training); tg_dense_layer runs a whole
 * above-gate decoder layer over the kept rows and tg_gated_delta_scan the token
 * mixer of a Gated-DeltaNet layer; tg_decode_attention attends new tokens over
 * the kept rows' cache (generation).
 *
 * Sources: the pages about "TokenGate: Adapting LLMs for Fast and
 * Memory-Efficient Prefill with Learned Token Pruning". The spke.com article
 * (German) defines the steps in its section "Wie hat TokenGate das Pruning von
 * Tokens verstanden?" (gate MLP on the post-attention residual of gate layer
 * L, top-K selector, only the kept tokens go up, no KV for the pruned ones,
 * only the document is prunable) and the bias in "Was ist token-gated
 * Attention?" (kept score -> logit bias, per-head gain, temperature); its
 * section "Wie wird TokenGate implementiert?" describes the budget given per
 * call and the placeholder that marks the document. The pages fix the bias
 * only qualitatively; this library computes, for kept rows i, j of a prompt
 * and query head h,
 *
 *     logit_ij = q_i . k_j / (sqrt(head_dim) * tau) + gain[h] * b_j,
 *     b_j      = logsigmoid(s_j) for document keys, 0 for the rest,
 *
 * over the keys j with pos_j <= pos_i.
 *
 * Conventions shared by every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller. tg_seq and
 *    tg_gather arrays are HOST memory, read during the call only.
 *  - The library allocates nothing and keeps no state other than a
 *    thread-local error string. Scratch memory, where a call needs any, is a
 *    caller-provided device workspace whose size the matching
 *    *_workspace_bytes function returns. The one exception is
 *    tg_decode_attention_noalloc, whose scratch is a static device array
 *    (see there).
 *  - Every call validates its arguments on the host first. A status other
 *    than TG_OK means nothing was enqueued; tg_last_error() gives details.
 *    A failed launch returns TG_ERR_HIP. Faults inside a kernel surface at the
 *    caller's next synchronisation, as with any HIP library.
 *  - Calls are asynchronous on `stream` and never synchronise. Every output
 *    size is known on the host (tg_kept_rows), so no call reads device memory
 *    back.
 *  - Outputs are bitwise deterministic for identical inputs.
 *  - Prompts are packed back to back ("varlen"): prompt b owns packed rows
 *    [start_b, start_b + len_b); kept rows are packed in the same prompt
 *    order, prompt b's kept rows at [off_b, off_b + M_b) with
 *    M_b = k_doc_b + len_b - (doc_end_b - doc_begin_b) and off_b the sum of
 *    the earlier M's.
 *  - bf16 is stored as the upper 16 bits of an IEEE binary32 (torch.bfloat16).
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TG_OK = 0,
    TG_ERR_INVALID_ARGUMENT = 1, /* a pointer, size or descriptor is wrong      */
    TG_ERR_UNSUPPORTED = 2,      /* valid, but a shape/alignment not built here */
    TG_ERR_WORKSPACE = 3,        /* workspace missing or too small              */
    TG_ERR_HIP = 4               /* the HIP runtime refused a launch            */
} tg_status;

typedef enum { TG_F32 = 0, TG_BF16 = 1 } tg_dtype;

/* Largest number of prompts one prefill call accepts (descriptors travel as
 * kernel arguments). Decode calls take up to 2^20 sequences, run in launches
 * of TG_MAX_SEQS sequences each. */
#define TG_MAX_SEQS 64
/* Largest number of tensors one tg_compact call gathers. */
#define TG_MAX_GATHERS 16

/* One packed prompt (host memory). The prunable document is rows
 * [start + doc_begin, start + doc_end); every other row of the prompt (the
 * question) is always kept. k_doc = document rows to keep, 0 <= k_doc <=
 * doc_end - doc_begin. Prompts must be given in increasing, non-overlapping
 * row order. */
typedef struct {
    int64_t start;
    int32_t len;
    int32_t doc_begin;
    int32_t doc_end;
    int32_t k_doc;
} tg_seq;

/* One tensor to gather (host memory describing device buffers): kept row m
 * is copied from src + kept_idx[m] * src_stride to dst + m * dst_stride,
 * row_bytes bytes. All three sizes and both pointers must be multiples of
 * 16 bytes. */
typedef struct {
    const void* src;
    void* dst;
    int64_t row_bytes;
    int64_t src_stride;
    int64_t dst_stride;
} tg_gather;

/* Rows kept by the given prompts: sum of k_doc + len - (doc_end - doc_begin).
 * Host only. Returns -1 (and sets the error text) if a descriptor is invalid. */
int64_t tg_kept_rows(const tg_seq* seqs, int32_t n_seqs);

/* Step 1 - gate score. For each of the n_rows rows x_r of x (row-major
 * [n_rows, d_model], dtype dt):
 *     h = W1 x_r + b1,   scores[r] = w2 . SiLU(h) + b2,
 * with W1 row-major [d_hidden, d_model] (nn.Linear layout), b1 [d_hidden]
 * (nullable: zero), w2 [d_hidden], all of dtype dt; scores is fp32 [n_rows].
 * Accumulation is fp32. bf16 inputs with d_model % 64 == 0, d_hidden in
 * {64, 128, 192, 256} and 16-byte-aligned x and w1 take the MFMA path;
 * every other shape takes a plain fp32-FMA path. Source: section "Wie hat
 * TokenGate das Pruning von Tokens verstanden?" (the MLP gate scores every
 * token from its post-attention residual at gate layer L). */
tg_status tg_gate_score(tg_dtype dt, const void* x, int64_t n_rows, int32_t d_model,
                        const void* w1, const void* b1, int32_t d_hidden, const void* w2,
                        float b2, float* scores, hipStream_t stream);

/* Device workspace tg_select_topk needs, in bytes: 0 (pass NULL) when every
 * prompt has at most 32768 rows, else about 24.6 KB per longer prompt plus
 * 65552 bytes per 16384 of its rows, rounded up to whole chunks (about 4
 * bytes per row: histograms, per-pass bin state, per-chunk counts and the
 * per-chunk lists of candidate keys of the multi-workgroup select). Also 0
 * for an invalid table (tg_select_topk then reports the error). The caller
 * owns the buffer; its contents need no initialisation and are scratch
 * after the call. */
size_t tg_select_workspace_bytes(const tg_seq* seqs, int32_t n_seqs);

/* Step 2 - top-K select. For each prompt, ranks its document rows by
 * scores (fp32 [total rows]), highest first, ties to the lower row id, NaN
 * below every number, -0 equal to +0; keeps the first k_doc of them and every
 * row outside the document; writes the kept packed row ids (int32) in
 * ascending order to kept_idx[off_b .. off_b + M_b). kept_idx must hold
 * tg_kept_rows(seqs) entries. workspace: device memory, 4-byte aligned, of at
 * least tg_select_workspace_bytes(seqs) bytes (TG_ERR_WORKSPACE otherwise);
 * two calls in flight at once need two workspaces. Bit-exact and
 * deterministic. Sources: section
 * "Wie hat TokenGate das Pruning von Tokens verstanden?" (top-K keeps the
 * best-scored tokens; the question is never removed). */
tg_status tg_select_topk(const float* scores, const tg_seq* seqs, int32_t n_seqs,
                         int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Step 3 - compaction of the m_rows = tg_kept_rows(seqs) kept rows.
 *  - gathers[0 .. n_gathers): row gathers, bit-exact (see tg_gather);
 *  - pos_kept (nullable) int32 [m_rows]: pos[kept_idx[m]], or, with pos NULL,
 *    kept_idx[m] - start of its prompt (original position in the prompt);
 *  - bias_kept (nullable, needs scores) fp32 [m_rows]:
 *    logsigmoid(scores[kept_idx[m]]) for document rows, 0 for the others.
 * kept_idx rows must belong to the prompts and be ordered by prompt.
 * Sources: section "Wie hat TokenGate das Pruning von Tokens verstanden?"
 * (layers above the gate process only the K kept tokens and create no KV for
 * the pruned), section "Was ist token-gated Attention?" (the kept score
 * becomes the bias). */
tg_status tg_compact(const int32_t* kept_idx, int64_t m_rows, const tg_seq* seqs,
                     int32_t n_seqs, const tg_gather* gathers, int32_t n_gathers,
                     const int32_t* pos, int32_t* pos_kept, const float* scores,
                     float* bias_kept, hipStream_t stream);

/* Step 4 - token-gated attention over the kept rows. q [M, hq, head_dim],
 * k and v [M, hkv, head_dim], out [M, hq, head_dim] (all contiguous, dtype
 * dt, M = tg_kept_rows(seqs)); bias_kept fp32 [M]; pos_kept int32 [M],
 * non-decreasing within each prompt (tg_compact produces this whenever
 * the original positions grow with the row id); gain fp32 [hq] (device);
 * tau > 0. Query head h reads KV head h / (hq / hkv). For kept rows i, j of
 * the same prompt:
 *     logit_ij = q_i . k_j / (sqrt(head_dim) * tau) + gain[h] * bias_kept[j]
 * over the keys with pos_kept[j] <= pos_kept[i], softmax, times V.
 * lse (nullable) fp32 [hq, M] receives log sum_j exp(logit_ij). bf16 runs on
 * MFMA with fp32 softmax and accumulation; fp32 runs on plain FMA. Needs no
 * workspace. Positions that decrease inside a prompt break the contract and
 * give wrong outputs with TG_OK; tg_check_positions tests a pos_kept array.
 * head_dim in {64, 128}; hq % hkv == 0. Sources: section "Was ist
 * token-gated Attention?" (kept-token score as a bias on the attention
 * logits above the gate, per-head gain, temperature) and "Wie wird TokenGate
 * implementiert?" (a key-bias attention kernel). */
tg_status tg_gated_attention(tg_dtype dt, const void* q, const void* k, const void* v,
                             const float* bias_kept, const int32_t* pos_kept,
                             const tg_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                             int32_t head_dim, const float* gain, float tau, void* out,
                             float* lse, hipStream_t stream);

/* Device workspace tg_gated_attention_backward needs, in bytes (0 for an
 * invalid table, which the call then reports). */
size_t tg_attention_backward_workspace_bytes(const tg_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                                             int32_t head_dim);

/* Backward of token-gated attention: the gradients of sum(d_out * out)
 * with respect to q, k, v, bias_kept, gain and tau, where out and lse are
 * what tg_gated_attention returned for the same inputs (lse is required).
 * With c = 1/(sqrt(head_dim) tau), p = softmax of the visible logits and
 * dS_ij = p_ij (d_out_i . v_j - d_out_i . out_i):
 *     d_q_i = c sum_j dS_ij k_j,   d_k_j = c sum_{h,i} dS_ij q_i,
 *     d_v_j = sum_{h,i} p_ij d_out_i,   d_bias_j = sum_h gain[h] sum_i dS_ij,
 *     d_gain[h] = sum_ij dS_ij bias_j,  d_tau = -(c/tau) sum dS_ij q_i.k_j.
 * Inputs as for tg_gated_attention (bf16 only: dt must be TG_BF16), plus
 * d_out bf16 [M, hq, head_dim]. Outputs fp32: d_q [M, hq, head_dim],
 * d_k and d_v [M, hkv, head_dim], d_bias [M], d_gain [hq], d_tau [1]
 * (device). Workspace: tg_attention_backward_workspace_bytes bytes,
 * 4-byte aligned (scratch). Deterministic (partials are summed in a fixed
 * order). Sources: section "Was ist token-gated Attention?" (the bias on the
 * logits is the gradient's path back to the scorer, as for a
 * mixture-of-experts router). */
tg_status tg_gated_attention_backward(tg_dtype dt, const void* q, const void* k, const void* v,
                                      const float* bias_kept, const int32_t* pos_kept,
                                      const tg_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                                      int32_t head_dim, const float* gain, float tau, const void* out,
                                      const float* lse, const void* d_out, float* d_q, float* d_k,
                                      float* d_v, float* d_bias, float* d_gain, float* d_tau,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gradient of the gate scores from the gradient of bias_kept: d_scores
 * fp32 [n_rows] is set to 0 everywhere except the kept document rows,
 * which get d_bias_kept[m] * sigmoid(-scores[kept_idx[m]]) (the derivative
 * of the logsigmoid that tg_compact applied). Question rows have a constant
 * bias and pruned rows none, so both get 0. Same section. */
tg_status tg_score_grad(const float* d_bias_kept, const float* scores, const int32_t* kept_idx,
                        const tg_seq* seqs, int32_t n_seqs, int64_t n_rows, float* d_scores,
                        hipStream_t stream);

/* One cached sequence for decode (host memory): rows [start, start + len)
 * of the KV cache of an above-gate layer (the kept rows of its pruned
 * prefill, then the tokens generated since), whose last n_new rows are the
 * tokens being decoded now. The caller appends their K, V, bias (0: they are
 * not document tokens) and position before the call; their queries are the
 * next n_new rows of q_new, sequence after sequence. */
typedef struct {
    int64_t start;
    int32_t len;
    int32_t n_new;
} tg_kv_seq;

/* Epilogues of tg_linear. */
#define TG_LINEAR_STORE 0    /* out = x W^T                              */
#define TG_LINEAR_RESIDUAL 1 /* out = residual + x W^T                   */
#define TG_LINEAR_SWIGLU 2   /* out = SiLU(x W^T) * (x W_up^T)           */

/* A linear layer of the above-gate model on MFMA: for the m rows of x (bf16
 * [m, k] row-major) and weights in the nn.Linear layout (bf16 [n, k]),
 * out (bf16 [m, n]) per the epilogue; accumulation fp32, one bf16 rounding
 * of the result. residual bf16 [m, n] (TG_LINEAR_RESIDUAL; may not alias
 * out), w_up bf16 [n, k] (TG_LINEAR_SWIGLU: w holds the gate rows, w_up the
 * matching up rows). k a multiple of 64; n a multiple of 128 (SwiGLU: 64);
 * all pointers device, 16-byte aligned. bf16 only. Source: the layers above
 * the gate are the model's own (section "Wie hat TokenGate das Pruning von
 * Tokens verstanden?": they run on the kept tokens only). */
tg_status tg_linear(tg_dtype dt, int32_t epilogue, const void* x, int64_t m, int32_t k, const void* w,
                    const void* w_up, int32_t n, const void* residual, void* out, hipStream_t stream);

/* Weights of one above-gate decoder layer (Qwen3 layout), all bf16 device
 * pointers in the nn.Linear layout [out, in], 16-byte aligned: ln1, ln2
 * [d_model] (RMSNorm), wqkv [(hq + 2 hkv) head_dim, d_model] (query rows,
 * then key rows, then value rows), q_norm, k_norm [head_dim] (per-head
 * RMSNorm), wo [d_model, hq head_dim], w_gate, w_up [d_ff, d_model], w_down
 * [d_model, d_ff]; gain fp32 [hq] and tau of the token-gated attention; eps
 * of every RMSNorm; rope_theta of the rotary embedding. Built: head_dim 64
 * or 128, d_model a multiple of 128, d_ff a multiple of 64, (hq + 2 hkv)
 * head_dim a multiple of 128. */
typedef struct {
    int32_t d_model, hq, hkv, head_dim, d_ff;
    float eps, rope_theta, tau;
    const void *ln1, *wqkv, *q_norm, *k_norm, *wo, *ln2, *w_gate, *w_up, *w_down;
    const float* gain;
} tg_dense_weights;

/* Device workspace tg_dense_layer needs, in bytes (0 for invalid weights or
 * prompts, which the call then reports). */
size_t tg_dense_layer_workspace_bytes(const tg_seq* seqs, int32_t n_seqs, const tg_dense_weights* w);

/* One full decoder layer above the gate over the kept rows (the model's own
 * layer with token-gated attention):
 *     a = RMSNorm(h) ln1;  q|k|v = a Wqkv^T;
 *     q, k = rotary(RMSNorm_head(q) q_norm | RMSNorm_head(k) k_norm, pos);
 *     h2 = h + TokenGatedAttention(q, k, v; bias, pos, gain, tau) Wo^T;
 *     out = h2 + (SiLU(a2 Wg^T) * (a2 Wu^T)) Wd^T,  a2 = RMSNorm(h2) ln2.
 * RMSNorm: x / sqrt(mean(x^2) + eps); rotary: element i < head_dim/2 pairs
 * with i + head_dim/2 and turns by pos * rope_theta^(-2i/head_dim). hidden_kept
 * bf16 [M, d_model] (tg_compact's output), bias_kept, pos_kept and seqs as
 * for tg_gated_attention; out bf16 [M, d_model]. k_out, v_out (nullable)
 * receive the layer's keys (normalised and rotated) and values, bf16
 * [M, hkv, head_dim]: the layer's pruned KV cache, for tg_decode_attention.
 * Intermediates are stored in bf16. Workspace:
 * tg_dense_layer_workspace_bytes bytes, 256-byte aligned (scratch). Sources:
 * section "Wie hat TokenGate das Pruning von Tokens verstanden?" (layers
 * above the gate process only the kept tokens and build no KV for the
 * pruned ones) and "Was ist token-gated Attention?" (the bias on their
 * logits). */
tg_status tg_dense_layer(tg_dtype dt, const void* hidden_kept, const float* bias_kept, const int32_t* pos_kept,
                         const tg_seq* seqs, int32_t n_seqs, const tg_dense_weights* w, void* out, void* k_out,
                         void* v_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Device workspace tg_gated_delta_scan needs, in bytes (0 for invalid
 * arguments, which the call then reports, or no rows). */
size_t tg_delta_scan_workspace_bytes(const tg_seq* seqs, int32_t n_seqs, int32_t n_heads, int32_t dk, int32_t dv);

/* The gated delta rule (the token mixer of a Gated-DeltaNet layer) over the
 * kept rows of each prompt, in their packed order:
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     out_t = S_t q_t,
 * per prompt and head, with the state S [dv, dk] starting at state_in (fp32
 * [n_seqs, n_heads, dv, dk], nullable: zero) and ending in state_out
 * (nullable). q, k bf16 [M, n_heads, dk], v bf16 [M, n_heads, dv], g (log
 * decay) and beta fp32 [M, n_heads], out bf16 [M, n_heads, dv]; q and k are
 * used as given (a Gated-DeltaNet layer L2-normalises them first). Built: dk =
 * dv = 128, bf16. Computed in 64-row chunks: per chunk, a triangular solve
 * independent of the state (all chunks at once), then the chunks in order on
 * MFMA with the state in fp32. Workspace: tg_delta_scan_workspace_bytes bytes,
 * 16-byte aligned (scratch). Sources: the pages' sections on hybrid-attention
 * models (ai4bro.com post, spke.com article, ai.info news): the gate also
 * prunes at Gated-DeltaNet layers, whose mixers then run over the kept rows
 * only. */
tg_status tg_gated_delta_scan(tg_dtype dt, const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const tg_seq* seqs, int32_t n_seqs, int32_t n_heads, int32_t dk,
                              int32_t dv, const float* state_in, void* out, float* state_out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Device workspace tg_gate_backward needs, in bytes (0 when n_list is 0 or
 * the shape is not built, which the call then reports). */
size_t tg_gate_backward_workspace_bytes(int64_t n_rows, int32_t d_model, int32_t d_hidden, int64_t n_list);

/* Backward of the gate MLP of step 1: the gradients of sum_r d_scores[r] *
 * scores[r] for the rows listed in rows[0..n_list). With z_r = W1 x_r + b1:
 *     dz_r = d_scores[r] * w2 * SiLU'(z_r),
 *     d_w1 = sum_r dz_r x_r^T [d_hidden, d_model],  d_b1 = sum_r dz_r,
 *     d_w2 = sum_r d_scores[r] SiLU(z_r),  d_b2 = sum_r d_scores[r],
 *     d_x[r] += W1^T dz_r  (fp32 [n_rows, d_model], added to; nullable: skip).
 * x, W1, b1 (nullable: zero), w2 as for tg_gate_score (bf16 only: dt must be
 * TG_BF16; d_model a multiple of 64; d_hidden one of 64, 128, 192, 256; x and
 * w1 16-byte aligned). d_scores fp32 [n_rows] (device), e.g. from
 * tg_score_grad. rows: device int32, distinct row ids in [0, n_rows) (rows
 * with nonzero score gradient, such as kept_idx), or NULL for every row
 * (n_list == n_rows) or for none (n_list == 0); unlisted rows count as d_scores = 0 and their d_x rows
 * are not touched. d_w1, d_b1, d_w2, d_b2 fp32 (device) are overwritten.
 * Workspace: tg_gate_backward_workspace_bytes bytes, 256-byte aligned
 * (scratch). Deterministic (partials summed in a fixed order); a repeated
 * row id makes d_x undefined. Sources: section "Was ist token-gated
 * Attention?" (the score's bias on the logits carries the gradient back to
 * the scorer) and section "Wie hat TokenGate das Pruning von Tokens
 * verstanden?" (the scorer is the small MLP of step 1). */
tg_status tg_gate_backward(tg_dtype dt, const void* x, int64_t n_rows, int32_t d_model, const void* w1,
                           const void* b1, const void* w2, int32_t d_hidden, const float* d_scores,
                           const int32_t* rows, int64_t n_list, float* d_x, float* d_w1, float* d_b1,
                           float* d_w2, float* d_b2, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Device workspace tg_decode_attention needs, in bytes (0 if no sequence
 * has new tokens; also 0 for an invalid table, which the call reports). */
size_t tg_decode_workspace_bytes(const tg_kv_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                                 int32_t head_dim);

/* Decode over the pruned KV cache. For new token t of sequence b (cache row
 * i = start + len - n_new + t) and query head h (KV head h / (hq / hkv)):
 *     logit_j = q . k_j / (sqrt(head_dim) * tau) + gain[h] * bias[j]
 * over the sequence's cache rows j with pos[j] <= pos[i], softmax, times V.
 * q_new [R, hq, head_dim] (R = sum of n_new); k, v [rows, hkv, head_dim];
 * out [R, hq, head_dim] (all contiguous, dtype dt; q_new, k, v 16-byte
 * aligned); bias fp32 and pos int32 per cache row; gain fp32 [hq] (device);
 * tau > 0; lse (nullable) fp32 [hq, R]. (hq / hkv) * n_new <= 8 per
 * sequence; head_dim in {64, 128}; up to 2^20 sequences (run in launches of
 * TG_MAX_SEQS sequences, in stream order, sharing the workspace). Workspace: device memory of at least
 * tg_decode_workspace_bytes bytes, 4-byte aligned, owned by the caller
 * (scratch; two calls in flight need two). Deterministic: the key splits
 * are fixed by the table and merged in key order. Sources: section "Wie hat
 * TokenGate das Pruning von Tokens verstanden?" (no KV for pruned tokens:
 * the cache holds the kept rows), section "Was ist token-gated Attention?"
 * (the kept tokens' bias on the logits above the gate) and "Wie wird
 * TokenGate implementiert?" (generation after the pruned prefill). */
tg_status tg_decode_attention(tg_dtype dt, const void* q_new, const void* k, const void* v,
                              const float* bias, const int32_t* pos, const tg_kv_seq* seqs,
                              int32_t n_seqs, int32_t hq, int32_t hkv, int32_t head_dim,
                              const float* gain, float tau, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Bytes of the static per-device scratch behind tg_decode_attention_noalloc. */
#define TG_DECODE_SCRATCH_BYTES (16u << 20)

/* tg_decode_attention without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same inputs,
 * outputs, validation and kernels as tg_decode_attention; the split-KV
 * partials go to a static scratch array of TG_DECODE_SCRATCH_BYTES bytes that
 * the library holds on each GPU it runs on until the process ends (its
 * device address is looked up on the first call on each device; that first
 * call must therefore not be made under graph capture). A call whose
 * partials need more than that (tg_decode_workspace_bytes > 16 MiB, e.g. more
 * than ~8000 (split, KV head) pairs at 8 query slots) is refused with
 * TG_ERR_WORKSPACE before anything is enqueued. Every call on one GPU shares
 * that GPU's scratch, whose contents are scratch after each call: calls that
 * overlap on one GPU (two streams, two host threads) race and give undefined
 * results; serialise them, or use tg_decode_attention with a workspace each. */
tg_status tg_decode_attention_noalloc(tg_dtype dt, const void* q_new, const void* k, const void* v,
                                      const float* bias, const int32_t* pos, const tg_kv_seq* seqs, int32_t n_seqs,
                                      int32_t hq, int32_t hkv, int32_t head_dim, const float* gain, float tau,
                                      void* out, float* lse, hipStream_t stream);

/* Checks the original positions of kept rows (tg_compact's output, or a
 * caller's own) for the order tg_gated_attention, its backward and
 * tg_dense_layer rely on: non-decreasing within each prompt. Writes to
 * *n_bad (device int32) the number of kept rows whose position is below the
 * previous kept row's in the same prompt; 0 means the positions are valid.
 * pos_kept int32 [M], M = tg_kept_rows(seqs). A check for debugging and
 * checked modes: the attention calls themselves do not run it. Source:
 * causality by original position (the pruned rows keep their original
 * positions; section "Wie hat TokenGate das Pruning von Tokens verstanden?"). */
tg_status tg_check_positions(const int32_t* pos_kept, const tg_seq* seqs, int32_t n_seqs, int32_t* n_bad,
                             hipStream_t stream);

/* Static text of a status code. */
const char* tg_status_string(tg_status status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* tg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
