// Internal declarations shared by the HIP kernels and the C-ABI host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tokengate.h"

namespace tg {

// Per-prompt descriptor as the kernels see it (passed by value as a kernel
// argument, so no device allocation is needed for it).
struct SeqDesc {
    int64_t start;     // first packed input row
    int64_t kept_off;  // first packed kept row
    int32_t len;       // rows in the prompt
    int32_t doc_begin; // document span, relative to start
    int32_t doc_end;
    int32_t k_doc;     // document rows kept
    int32_t n_kept;    // k_doc + len - (doc_end - doc_begin)
    int32_t pad;
};

struct SeqTable {
    int32_t n;
    int32_t pad;
    SeqDesc s[TG_MAX_SEQS];
};

struct GatherDesc {
    const char* src;
    char* dst;
    int64_t units;       // 16-byte units per row
    int64_t src_stride;  // bytes
    int64_t dst_stride;  // bytes
};

struct GatherTable {
    int32_t n;
    int32_t pad;
    GatherDesc g[TG_MAX_GATHERS];
};

// Attention work decomposition: one entry per prompt.
struct AttnSeg {
    int64_t kept_off;   // first packed kept row of the prompt
    int32_t n;          // kept rows of the prompt
    int32_t n_qblk;     // query blocks of the prompt
    int32_t item_base;  // first work item of the prompt
    int32_t pad;
};

struct AttnTable {
    int32_t n_seg;
    int32_t n_items;
    int64_t m_total;
    int32_t cfg;   // kernel shape (attention_config().kind)
    int32_t cus;   // compute units of the device (0: unknown)
    AttnSeg s[TG_MAX_SEQS];
};

// Work decomposition of the attention kernel for a call: the query rows of
// one work item and the query heads it covers (chosen from the dtype, the
// head ratio and the longest prompt).
struct AttnConfig {
    int kind;            // kernel shape
    int block_rows;      // query rows per work item
    int heads_per_item;  // query heads per work item
};
AttnConfig attention_config(tg_dtype dt, int hq, int hkv, int64_t max_rows);

// Launchers (each returns hipGetLastError() after its launch).
hipError_t launch_gate_mfma_bf16(const void* x, int64_t n, int d, const void* w1, const void* b1,
                                 int h, const void* w2, float b2, float* scores, hipStream_t st);
hipError_t launch_gate_simple(tg_dtype dt, const void* x, int64_t n, int d, const void* w1,
                              const void* b1, int h, const void* w2, float b2, float* scores,
                              hipStream_t st);
// Select: prompts of up to SEL_REG_MAX rows are handled by one workgroup
// each; longer prompts by a multi-workgroup radix select over chunks of
// SEL_CHUNK rows, which keeps its histograms and chunk counts in a workspace.
constexpr int SEL_REG_MAX = 32768;
constexpr int SEL_CHUNK = 16384;
struct LongSeq {
    int32_t seq;        // index in SeqTable
    int32_t hist_base;  // first histogram workgroup (chunks of the document)
    int32_t n_hist;
    int32_t emit_base;  // first emission workgroup (chunks of the whole prompt)
    int32_t n_emit;
    int32_t pad;
};
struct LongTable {
    int32_t n;
    int32_t n_hist;     // histogram workgroups over all long prompts
    int32_t n_emit;     // emission workgroups over all long prompts
    int32_t pad;
    LongSeq s[TG_MAX_SEQS];
};
// Fills the long-prompt table; returns the workspace bytes it needs.
size_t select_plan(const SeqTable& t, LongTable* lt);
hipError_t launch_select(const float* scores, const SeqTable& t, const LongTable& lt, void* workspace,
                         int32_t* kept, hipStream_t st);
// *n_bad = number of kept rows whose position is below the previous kept
// row's in the same prompt.
hipError_t launch_check_positions(const int32_t* pos, int64_t m, const SeqTable& t, int32_t* n_bad,
                                  hipStream_t st);
hipError_t launch_compact(const int32_t* kept, int64_t m, const SeqTable& t, const GatherTable& g,
                          const int32_t* pos, int32_t* pos_kept, const float* scores,
                          float* bias_kept, hipStream_t st);
hipError_t launch_attention(tg_dtype dt, const void* q, const void* k, const void* v,
                            const float* bias, const int32_t* pos, const AttnTable& t, int hq,
                            int hkv, int head_dim, const float* gain, float tau, void* out,
                            float* lse, hipStream_t st);

// Decode over the pruned KV cache: one entry per sequence with new tokens.
struct DecSeq {
    int64_t start;       // first cache row
    int32_t len;         // cache rows (the new tokens are the last n_new)
    int32_t n_new;
    int32_t q_row0;      // first row of q_new / out for this sequence
    int32_t split_base;  // first global split id (splits of kpw keys)
};
// One launch's share of a decode call: up to TG_MAX_SEQS sequences with new
// tokens (a call with more is split into several launches in stream order,
// which reuse one workspace).
struct DecTable {
    int32_t n;
    int32_t kpw;      // keys per split (one wave per split and KV head), same in every launch of a call
    int32_t n_waves;  // splits x KV heads of this launch
    int32_t nq_max;   // largest (hq/hkv) * n_new over the call's sequences
    int32_t row0;     // first query row of this launch's sequences
    int32_t n_rows;   // query rows of this launch's sequences
    DecSeq s[TG_MAX_SEQS];
};
// Query slots per wave for nq queries (0: more than supported).
int decode_query_slots(int nq);
hipError_t launch_decode(tg_dtype dt, const void* q, const void* k, const void* v, const float* bias,
                         const int32_t* pos, const DecTable& t, int hq, int hkv, int head_dim, const float* gain,
                         float tau, void* out, float* lse, int64_t r_total, void* ws, hipStream_t st);
// Device address of this device's static decode scratch (TG_DECODE_SCRATCH_BYTES
// bytes), looked up on the first call on each device.
hipError_t decode_scratch(void** ptr);

// Backward of token-gated attention (bf16 inputs, fp32 gradients).
struct AttnBwdArgs {
    const void *q, *k, *v, *out, *d_out;
    const float* lse;
    const float* bias;
    const int32_t* pos;
    const float* gain;
    float tau;
    int hq, hkv, head_dim;
    float *d_q, *d_k, *d_v, *d_bias, *d_gain, *d_tau;
    void* workspace;
};
// Fills the opaque work table (attention_backward_table_bytes() bytes) and
// returns the workspace bytes.
size_t attention_backward_plan(const SeqTable& st, int hq, int hkv, int head_dim, void* table_out);
size_t attention_backward_table_bytes();

// Dense decoder layer pieces (bf16).
hipError_t launch_rmsnorm(const void* x, int64_t m, int d, const void* w, float eps, void* out, hipStream_t st);
hipError_t launch_qk_norm_rope(const void* qkv, int64_t m, int hq, int hkv, int head_dim, const void* qn,
                               const void* kn, const int32_t* pos, float eps, float theta, void* q, void* k, void* v,
                               hipStream_t st);
// epi: 0 store, 1 add residual, 2 SwiGLU (w = gate rows, w_up = up rows).
hipError_t launch_linear(int epi, const void* a, int64_t m, int k, const void* w, const void* w_up, int n_out,
                         const void* resid, void* out, hipStream_t st);

// Gated delta rule over the kept rows (bf16, dk = dv = 128).
size_t delta_scan_workspace_bytes(const SeqTable& t, int nh);
hipError_t launch_delta_scan(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const SeqTable& t, int nh, const float* state_in, void* out, float* state_out,
                             void* workspace, hipStream_t st);

// Gate MLP backward (bf16, d_model % 64 == 0, d_hidden % 64 == 0 and <= 256).
size_t gate_backward_workspace_bytes(int64_t n_list, int d_model, int d_hidden);
hipError_t launch_gate_backward(const void* x, int64_t n_rows, int d, const void* w1, const void* b1,
                                const void* w2, int hdim, const float* d_scores, const int32_t* rows,
                                int64_t n_list, float* d_x, float* d_w1, float* d_b1, float* d_w2, float* d_b2,
                                void* workspace, hipStream_t st);
hipError_t launch_attention_backward(const AttnBwdArgs& a, const void* table, hipStream_t st);
// Fill kernel (graph-capture safe, unlike a memset node): p[0 .. n) = 0.
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st);
hipError_t launch_score_grad(const float* d_bias, const float* scores, const int32_t* kept, const SeqTable& t,
                             int64_t m, int64_t n_rows, float* d_scores, hipStream_t st);



}  // namespace tg
