// C-ABI entry points: argument validation on the host, descriptor tables,
// kernel launches. Validation runs before anything touches the HIP runtime,
// so every invalid call returns its status without enqueueing work.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "tg_internal.hpp"

#include <atomic>

#include <vector>

namespace {

thread_local std::string g_err;

tg_status fail(tg_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

tg_status hip_fail(hipError_t e, const char* what) {
    return fail(TG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validates the prompt descriptors and fills the kernel-side table.
// Returns TG_OK and the total kept rows through *m_total.
tg_status build_seq_table(const tg_seq* seqs, int32_t n_seqs, tg::SeqTable* t, int64_t* m_total) {
    if (n_seqs < 0 || n_seqs > TG_MAX_SEQS)
        return fail(TG_ERR_INVALID_ARGUMENT, "n_seqs=%d outside [0, %d]", n_seqs, TG_MAX_SEQS);
    if (n_seqs > 0 && !seqs) return fail(TG_ERR_INVALID_ARGUMENT, "seqs is NULL");
    memset(t, 0, sizeof *t);
    t->n = n_seqs;
    int64_t next = 0, kept = 0;
    for (int32_t b = 0; b < n_seqs; ++b) {
        const tg_seq& s = seqs[b];
        if (s.start < next)
            return fail(TG_ERR_INVALID_ARGUMENT,
                        "prompt %d: start=%lld overlaps or precedes the previous prompt", b,
                        (long long)s.start);
        if (s.len < 0) return fail(TG_ERR_INVALID_ARGUMENT, "prompt %d: len=%d < 0", b, s.len);
        if (s.doc_begin < 0 || s.doc_begin > s.doc_end || s.doc_end > s.len)
            return fail(TG_ERR_INVALID_ARGUMENT,
                        "prompt %d: document span [%d, %d) outside the prompt (len %d)", b,
                        s.doc_begin, s.doc_end, s.len);
        const int32_t n_doc = s.doc_end - s.doc_begin;
        if (s.k_doc < 0 || s.k_doc > n_doc)
            return fail(TG_ERR_INVALID_ARGUMENT, "prompt %d: k_doc=%d outside [0, %d]", b, s.k_doc,
                        n_doc);
        if (s.start + s.len > (int64_t)INT32_MAX)
            return fail(TG_ERR_UNSUPPORTED, "prompt %d: rows beyond 2^31-1 (int32 row ids)", b);
        tg::SeqDesc& d = t->s[b];
        d.start = s.start;
        d.kept_off = kept;
        d.len = s.len;
        d.doc_begin = s.doc_begin;
        d.doc_end = s.doc_end;
        d.k_doc = s.k_doc;
        d.n_kept = s.k_doc + (s.len - n_doc);
        kept += d.n_kept;
        next = s.start + s.len;
    }
    *m_total = kept;
    return TG_OK;
}

}  // namespace

extern "C" {

const char* tg_status_string(tg_status st) {
    switch (st) {
        case TG_OK: return "ok";
        case TG_ERR_INVALID_ARGUMENT: return "invalid argument";
        case TG_ERR_UNSUPPORTED: return "unsupported shape or alignment";
        case TG_ERR_WORKSPACE: return "workspace missing or too small";
        case TG_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* tg_last_error(void) { return g_err.c_str(); }

tg_status tg_check_positions(const int32_t* pos_kept, const tg_seq* seqs, int32_t n_seqs, int32_t* n_bad,
                             hipStream_t stream) {
    g_err.clear();
    tg::SeqTable t;
    int64_t m = 0;
    tg_status st = build_seq_table(seqs, n_seqs, &t, &m);
    if (st != TG_OK) return st;
    if (!n_bad) return fail(TG_ERR_INVALID_ARGUMENT, "n_bad is NULL");
    if (m > 0 && !pos_kept) return fail(TG_ERR_INVALID_ARGUMENT, "pos_kept is NULL");
    hipError_t e = tg::launch_check_positions(pos_kept, m, t, n_bad, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_check_positions launch");
    return TG_OK;
}

int64_t tg_kept_rows(const tg_seq* seqs, int32_t n_seqs) {
    tg::SeqTable t;
    int64_t m = 0;
    if (build_seq_table(seqs, n_seqs, &t, &m) != TG_OK) return -1;
    return m;
}

tg_status tg_gate_score(tg_dtype dt, const void* x, int64_t n_rows, int32_t d_model, const void* w1,
                        const void* b1, int32_t d_hidden, const void* w2, float b2, float* scores,
                        hipStream_t stream) {
    g_err.clear();
    if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARGUMENT, "dtype %d unknown", (int)dt);
    if (n_rows < 0) return fail(TG_ERR_INVALID_ARGUMENT, "n_rows=%lld < 0", (long long)n_rows);
    if (d_model <= 0 || d_hidden <= 0)
        return fail(TG_ERR_INVALID_ARGUMENT, "d_model=%d and d_hidden=%d must be > 0", d_model, d_hidden);
    if (n_rows == 0) return TG_OK;
    if (!x || !w1 || !w2 || !scores) return fail(TG_ERR_INVALID_ARGUMENT, "x, w1, w2, scores must be non-NULL");
    if ((n_rows + 3) / 4 > (int64_t)INT32_MAX)
        return fail(TG_ERR_UNSUPPORTED, "n_rows=%lld too large for one launch", (long long)n_rows);
    const bool mfma = dt == TG_BF16 && d_model % 64 == 0 && (d_hidden == 64 || d_hidden == 128 || d_hidden == 192 || d_hidden == 256) &&
                      aligned16(x) && aligned16(w1);
    hipError_t e = mfma ? tg::launch_gate_mfma_bf16(x, n_rows, d_model, w1, b1, d_hidden, w2, b2, scores, stream)
                        : tg::launch_gate_simple(dt, x, n_rows, d_model, w1, b1, d_hidden, w2, b2, scores, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_gate_score launch");
    return TG_OK;
}

size_t tg_select_workspace_bytes(const tg_seq* seqs, int32_t n_seqs) {
    tg::SeqTable t;
    int64_t m = 0;
    if (build_seq_table(seqs, n_seqs, &t, &m) != TG_OK) return 0;
    g_err.clear();
    tg::LongTable lt;
    return tg::select_plan(t, &lt);
}

tg_status tg_select_topk(const float* scores, const tg_seq* seqs, int32_t n_seqs, int32_t* kept_idx,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err.clear();
    tg::SeqTable t;
    int64_t m = 0;
    tg_status st = build_seq_table(seqs, n_seqs, &t, &m);
    if (st != TG_OK) return st;
    if (n_seqs == 0) return TG_OK;
    bool any_rows = false;
    for (int b = 0; b < n_seqs; ++b) any_rows |= seqs[b].len > 0;
    if (!any_rows) return TG_OK;
    if (!scores) return fail(TG_ERR_INVALID_ARGUMENT, "scores is NULL");
    if (m > 0 && !kept_idx) return fail(TG_ERR_INVALID_ARGUMENT, "kept_idx is NULL");
    tg::LongTable lt;
    const size_t need = tg::select_plan(t, &lt);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(TG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                        need);
        if ((uintptr_t)workspace % 4 != 0) return fail(TG_ERR_INVALID_ARGUMENT, "workspace not 4-byte aligned");
    }
    hipError_t e = tg::launch_select(scores, t, lt, workspace, kept_idx, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_select_topk launch");
    return TG_OK;
}

tg_status tg_compact(const int32_t* kept_idx, int64_t m_rows, const tg_seq* seqs, int32_t n_seqs,
                     const tg_gather* gathers, int32_t n_gathers, const int32_t* pos,
                     int32_t* pos_kept, const float* scores, float* bias_kept, hipStream_t stream) {
    g_err.clear();
    tg::SeqTable t;
    int64_t m = 0;
    tg_status st = build_seq_table(seqs, n_seqs, &t, &m);
    if (st != TG_OK) return st;
    if (m_rows != m)
        return fail(TG_ERR_INVALID_ARGUMENT, "m_rows=%lld but the prompts keep %lld rows",
                    (long long)m_rows, (long long)m);
    if (n_gathers < 0 || n_gathers > TG_MAX_GATHERS)
        return fail(TG_ERR_INVALID_ARGUMENT, "n_gathers=%d outside [0, %d]", n_gathers, TG_MAX_GATHERS);
    if (n_gathers > 0 && !gathers) return fail(TG_ERR_INVALID_ARGUMENT, "gathers is NULL");
    if (bias_kept && !scores) return fail(TG_ERR_INVALID_ARGUMENT, "bias_kept needs scores");
    tg::GatherTable g;
    memset(&g, 0, sizeof g);
    g.n = n_gathers;
    for (int i = 0; i < n_gathers; ++i) {
        const tg_gather& d = gathers[i];
        if (!d.src || !d.dst) return fail(TG_ERR_INVALID_ARGUMENT, "gather %d: NULL pointer", i);
        if (d.row_bytes <= 0 || d.row_bytes > (int64_t)1 << 30)
            return fail(TG_ERR_INVALID_ARGUMENT, "gather %d: row_bytes=%lld outside (0, 2^30]", i,
                        (long long)d.row_bytes);
        if (d.src_stride < d.row_bytes || d.dst_stride < d.row_bytes)
            return fail(TG_ERR_INVALID_ARGUMENT, "gather %d: strides smaller than row_bytes", i);
        if (d.row_bytes % 16 || d.src_stride % 16 || d.dst_stride % 16 || !aligned16(d.src) ||
            !aligned16(d.dst))
            return fail(TG_ERR_UNSUPPORTED, "gather %d: sizes and pointers must be multiples of 16 bytes", i);
        g.g[i].src = (const char*)d.src;
        g.g[i].dst = (char*)d.dst;
        g.g[i].units = d.row_bytes / 16;
        g.g[i].src_stride = d.src_stride;
        g.g[i].dst_stride = d.dst_stride;
    }
    if (m == 0) return TG_OK;
    if (!kept_idx) return fail(TG_ERR_INVALID_ARGUMENT, "kept_idx is NULL");
    if (n_gathers == 0 && !pos_kept && !bias_kept) return TG_OK;
    hipError_t e = tg::launch_compact(kept_idx, m, t, g, pos, pos_kept, scores, bias_kept, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_compact launch");
    return TG_OK;
}

// Compute units of the current device, looked up once per device.
static int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = -1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? v : 0;
}

tg_status tg_gated_attention(tg_dtype dt, const void* q, const void* k, const void* v,
                             const float* bias_kept, const int32_t* pos_kept, const tg_seq* seqs,
                             int32_t n_seqs, int32_t hq, int32_t hkv, int32_t head_dim,
                             const float* gain, float tau, void* out, float* lse, hipStream_t stream) {
    g_err.clear();
    if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARGUMENT, "dtype %d unknown", (int)dt);
    if (hq <= 0 || hkv <= 0 || hq % hkv)
        return fail(TG_ERR_INVALID_ARGUMENT, "hq=%d must be a positive multiple of hkv=%d", hq, hkv);
    if (head_dim != 64 && head_dim != 128)
        return fail(TG_ERR_UNSUPPORTED, "head_dim=%d (built: 64, 128)", head_dim);
    if (!(tau > 0.0f) || tau != tau || tau > 3.0e38f)
        return fail(TG_ERR_INVALID_ARGUMENT, "tau must be finite and > 0");
    tg::SeqTable st_;
    int64_t m = 0;
    tg_status st = build_seq_table(seqs, n_seqs, &st_, &m);
    if (st != TG_OK) return st;
    if (m == 0) return TG_OK;
    if (!q || !k || !v || !bias_kept || !pos_kept || !gain || !out)
        return fail(TG_ERR_INVALID_ARGUMENT, "q, k, v, bias_kept, pos_kept, gain, out must be non-NULL");
    if (dt == TG_BF16 && !(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out)))
        return fail(TG_ERR_UNSUPPORTED, "bf16 q, k, v, out must be 16-byte aligned");
    int64_t max_rows = 0;
    for (int b = 0; b < n_seqs; ++b) max_rows = st_.s[b].n_kept > max_rows ? st_.s[b].n_kept : max_rows;
    const tg::AttnConfig cfg = tg::attention_config(dt, hq, hkv, max_rows);
    const int bm = cfg.block_rows;
    const int64_t items_per_blk = hq / cfg.heads_per_item;
    tg::AttnTable t;
    memset(&t, 0, sizeof t);
    t.n_seg = n_seqs;
    t.m_total = m;
    t.cfg = cfg.kind;
    t.cus = device_cus();
    int64_t items = 0;
    for (int b = 0; b < n_seqs; ++b) {
        const tg::SeqDesc& d = st_.s[b];
        t.s[b].kept_off = d.kept_off;
        t.s[b].n = d.n_kept;
        t.s[b].n_qblk = (d.n_kept + bm - 1) / bm;
        t.s[b].item_base = (int32_t)items;
        items += (int64_t)t.s[b].n_qblk * items_per_blk;
        if (items > (int64_t)INT32_MAX) return fail(TG_ERR_UNSUPPORTED, "too many work items for one launch");
    }
    t.n_items = (int32_t)items;
    hipError_t e = tg::launch_attention(dt, q, k, v, bias_kept, pos_kept, t, hq, hkv, head_dim, gain,
                                        tau, out, lse, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_gated_attention launch");
    return TG_OK;
}

}  // extern "C"

namespace {

// Decode tables: the sequences with new tokens, their splits and output
// rows, in launches of up to TG_MAX_SEQS sequences. Validates every sequence
// before returning, so a refused call enqueues nothing.
constexpr int32_t TG_MAX_DECODE_SEQS = 1 << 20;

tg_status build_decode_tables(tg_dtype dt, const tg_kv_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                              int32_t head_dim, std::vector<tg::DecTable>* tables, int64_t* r_total,
                              size_t* ws_bytes) {
    if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARGUMENT, "dtype %d unknown", (int)dt);
    if (hq <= 0 || hkv <= 0 || hq % hkv)
        return fail(TG_ERR_INVALID_ARGUMENT, "hq=%d must be a positive multiple of hkv=%d", hq, hkv);
    if (head_dim != 64 && head_dim != 128)
        return fail(TG_ERR_UNSUPPORTED, "head_dim=%d (built: 64, 128)", head_dim);
    if (n_seqs < 0 || n_seqs > TG_MAX_DECODE_SEQS)
        return fail(TG_ERR_INVALID_ARGUMENT, "n_seqs=%d outside [0, %d]", n_seqs, TG_MAX_DECODE_SEQS);
    if (n_seqs > 0 && !seqs) return fail(TG_ERR_INVALID_ARGUMENT, "seqs is NULL");
    tables->clear();
    const int g = hq / hkv;
    int64_t rows = 0, keys = 0, max_len = 0;
    int nq_max = 0;
    for (int b = 0; b < n_seqs; ++b) {
        const tg_kv_seq& s = seqs[b];
        if (s.start < 0 || s.len < 0 || s.n_new < 0 || s.n_new > s.len)
            return fail(TG_ERR_INVALID_ARGUMENT, "sequence %d: start=%lld len=%d n_new=%d", b, (long long)s.start,
                        s.len, s.n_new);
        if (s.n_new == 0) continue;
        if (tg::decode_query_slots(g * s.n_new) == 0)
            return fail(TG_ERR_UNSUPPORTED, "sequence %d: (hq/hkv) * n_new = %d > 8", b, g * s.n_new);
        nq_max = nq_max > g * s.n_new ? nq_max : g * s.n_new;
        keys += s.len;
        max_len = max_len > s.len ? max_len : s.len;
        rows += s.n_new;
    }
    if (rows > (int64_t)INT32_MAX / hq) return fail(TG_ERR_UNSUPPORTED, "too many new tokens for one call");
    *r_total = rows;
    *ws_bytes = 0;
    if (rows == 0) return TG_OK;
    // Keys per split: a power of two, a multiple of the keys one wave's lane
    // groups take per block, sized for about 4096 waves over the call and for
    // at most 256 splits per sequence (the merge walks a query's splits).
    const int esize = dt == TG_BF16 ? 2 : 4;
    const int lpk = head_dim * esize / 16;
    const int granule = (64 / lpk) * 8;
    int64_t kpw = granule;
    while (kpw < (1 << 20) && (kpw * 4096 < keys * hkv || kpw * 256 < max_len)) kpw *= 2;
    const int nq = tg::decode_query_slots(nq_max);
    tg::DecTable t;
    memset(&t, 0, sizeof t);
    int64_t q_row = 0, splits = 0;
    auto flush = [&]() -> tg_status {
        if (t.n == 0) return TG_OK;
        if (splits * hkv > (int64_t)INT32_MAX / 2) return fail(TG_ERR_UNSUPPORTED, "too many splits for one launch");
        t.n_waves = (int32_t)(splits * hkv);
        t.n_rows = (int32_t)(q_row - t.row0);
        const size_t need = (size_t)t.n_waves * nq * (head_dim + 2) * sizeof(float);
        *ws_bytes = need > *ws_bytes ? need : *ws_bytes;
        tables->push_back(t);
        memset(&t, 0, sizeof t);
        splits = 0;
        return TG_OK;
    };
    for (int b = 0; b < n_seqs; ++b) {
        const tg_kv_seq& s = seqs[b];
        if (s.n_new == 0) continue;
        if (t.n == TG_MAX_SEQS) {
            const tg_status st = flush();
            if (st != TG_OK) return st;
        }
        if (t.n == 0) {
            t.kpw = (int32_t)kpw;
            t.nq_max = nq_max;
            t.row0 = (int32_t)q_row;
        }
        tg::DecSeq& d = t.s[t.n++];
        d.start = s.start;
        d.len = s.len;
        d.n_new = s.n_new;
        d.q_row0 = (int32_t)q_row;
        d.split_base = (int32_t)splits;
        splits += (s.len + kpw - 1) / kpw;
        q_row += s.n_new;
    }
    return flush();
}

}  // namespace

extern "C" {

size_t tg_attention_backward_workspace_bytes(const tg_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                                             int32_t head_dim) {
    tg::SeqTable st_;
    int64_t m = 0;
    if (hq <= 0 || hkv <= 0 || hq % hkv || (head_dim != 64 && head_dim != 128)) return 0;
    if (build_seq_table(seqs, n_seqs, &st_, &m) != TG_OK) return 0;
    g_err.clear();
    std::vector<char> table(tg::attention_backward_table_bytes());
    return tg::attention_backward_plan(st_, hq, hkv, head_dim, table.data());
}

tg_status tg_gated_attention_backward(tg_dtype dt, const void* q, const void* k, const void* v, const float* bias_kept,
                                      const int32_t* pos_kept, const tg_seq* seqs, int32_t n_seqs, int32_t hq,
                                      int32_t hkv, int32_t head_dim, const float* gain, float tau, const void* out,
                                      const float* lse, const void* d_out, float* d_q, float* d_k, float* d_v,
                                      float* d_bias, float* d_gain, float* d_tau, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    g_err.clear();
    if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "the backward is built for bf16 inputs only");
    if (hq <= 0 || hkv <= 0 || hq % hkv)
        return fail(TG_ERR_INVALID_ARGUMENT, "hq=%d must be a positive multiple of hkv=%d", hq, hkv);
    if (head_dim != 64 && head_dim != 128)
        return fail(TG_ERR_UNSUPPORTED, "head_dim=%d (built: 64, 128)", head_dim);
    if (!(tau > 0.0f) || tau != tau || tau > 3.0e38f)
        return fail(TG_ERR_INVALID_ARGUMENT, "tau must be finite and > 0");
    tg::SeqTable st_;
    int64_t m = 0;
    tg_status st = build_seq_table(seqs, n_seqs, &st_, &m);
    if (st != TG_OK) return st;
    if (!d_gain || !d_tau) return fail(TG_ERR_INVALID_ARGUMENT, "d_gain, d_tau must be non-NULL");
    std::vector<char> table(tg::attention_backward_table_bytes());
    const size_t need = tg::attention_backward_plan(st_, hq, hkv, head_dim, table.data());
    if (m == 0) {
        hipError_t e = tg::launch_zero_f32(d_gain, hq, stream);
        if (e == hipSuccess) e = tg::launch_zero_f32(d_tau, 1, stream);
        if (e != hipSuccess) return hip_fail(e, "tg_gated_attention_backward clear");
        return TG_OK;
    }
    if (!q || !k || !v || !bias_kept || !pos_kept || !gain || !out || !lse || !d_out || !d_q || !d_k || !d_v ||
        !d_bias)
        return fail(TG_ERR_INVALID_ARGUMENT, "every tensor pointer must be non-NULL");
    if (!(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned16(d_out) && aligned16(d_q)))
        return fail(TG_ERR_UNSUPPORTED, "q, k, v, out, d_out, d_q must be 16-byte aligned");
    if ((int64_t)m * hq > (int64_t)INT32_MAX / 2) return fail(TG_ERR_UNSUPPORTED, "too many rows for one launch");
    if (!workspace || workspace_bytes < need)
        return fail(TG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                    need);
    if ((uintptr_t)workspace % 4 != 0) return fail(TG_ERR_INVALID_ARGUMENT, "workspace not 4-byte aligned");
    tg::AttnBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.d_out = d_out;
    a.lse = lse; a.bias = bias_kept; a.pos = pos_kept; a.gain = gain; a.tau = tau;
    a.hq = hq; a.hkv = hkv; a.head_dim = head_dim;
    a.d_q = d_q; a.d_k = d_k; a.d_v = d_v; a.d_bias = d_bias; a.d_gain = d_gain; a.d_tau = d_tau;
    a.workspace = workspace;
    hipError_t e = tg::launch_attention_backward(a, table.data(), stream);
    if (e != hipSuccess) return hip_fail(e, "tg_gated_attention_backward launch");
    return TG_OK;
}

tg_status tg_score_grad(const float* d_bias_kept, const float* scores, const int32_t* kept_idx, const tg_seq* seqs,
                        int32_t n_seqs, int64_t n_rows, float* d_scores, hipStream_t stream) {
    g_err.clear();
    tg::SeqTable t;
    int64_t m = 0;
    tg_status st = build_seq_table(seqs, n_seqs, &t, &m);
    if (st != TG_OK) return st;
    if (n_rows < 0) return fail(TG_ERR_INVALID_ARGUMENT, "n_rows=%lld < 0", (long long)n_rows);
    for (int b = 0; b < n_seqs; ++b)
        if (seqs[b].start + seqs[b].len > n_rows)
            return fail(TG_ERR_INVALID_ARGUMENT, "prompt %d ends past n_rows=%lld", b, (long long)n_rows);
    if (n_rows == 0) return TG_OK;
    if (!d_scores || (m > 0 && (!d_bias_kept || !scores || !kept_idx)))
        return fail(TG_ERR_INVALID_ARGUMENT, "d_bias_kept, scores, kept_idx, d_scores must be non-NULL");
    hipError_t e = tg::launch_score_grad(d_bias_kept, scores, kept_idx, t, m, n_rows, d_scores, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_score_grad launch");
    return TG_OK;
}

static tg_status check_gate_backward_shape(int64_t n_rows, int32_t d_model, int32_t d_hidden, int64_t n_list) {
    if (n_rows < 0 || n_list < 0 || n_list > n_rows)
        return fail(TG_ERR_INVALID_ARGUMENT, "need 0 <= n_list=%lld <= n_rows=%lld", (long long)n_list,
                    (long long)n_rows);
    if (d_model <= 0 || d_model % 64)
        return fail(TG_ERR_UNSUPPORTED, "d_model=%d (built: positive multiples of 64)", d_model);
    if (d_hidden <= 0 || d_hidden % 64 || d_hidden > 256)
        return fail(TG_ERR_UNSUPPORTED, "d_hidden=%d (built: 64, 128, 192, 256)", d_hidden);
    return TG_OK;
}

size_t tg_gate_backward_workspace_bytes(int64_t n_rows, int32_t d_model, int32_t d_hidden, int64_t n_list) {
    if (check_gate_backward_shape(n_rows, d_model, d_hidden, n_list) != TG_OK) return 0;
    g_err.clear();
    return tg::gate_backward_workspace_bytes(n_list, d_model, d_hidden);
}

tg_status tg_gate_backward(tg_dtype dt, const void* x, int64_t n_rows, int32_t d_model, const void* w1,
                           const void* b1, const void* w2, int32_t d_hidden, const float* d_scores,
                           const int32_t* rows, int64_t n_list, float* d_x, float* d_w1, float* d_b1, float* d_w2,
                           float* d_b2, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err.clear();
    if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "the gate backward is built for bf16 inputs only");
    tg_status st = check_gate_backward_shape(n_rows, d_model, d_hidden, n_list);
    if (st != TG_OK) return st;
    if (!w1 || !w2 || !d_w1 || !d_b1 || !d_w2 || !d_b2)
        return fail(TG_ERR_INVALID_ARGUMENT, "w1, w2, d_w1, d_b1, d_w2, d_b2 must be non-NULL");
    if (n_list > 0 && (!x || !d_scores)) return fail(TG_ERR_INVALID_ARGUMENT, "x and d_scores must be non-NULL");
    if (!rows && n_list > 0 && n_list != n_rows)
        return fail(TG_ERR_INVALID_ARGUMENT, "rows may be NULL only when n_list == n_rows (every row)");
    if (!(aligned16(x) && aligned16(w1))) return fail(TG_ERR_UNSUPPORTED, "x and w1 must be 16-byte aligned");
    const size_t need = tg::gate_backward_workspace_bytes(n_list, d_model, d_hidden);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(TG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                    need);
    if ((uintptr_t)workspace % 256 != 0) return fail(TG_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
    hipError_t e = tg::launch_gate_backward(x, n_rows, d_model, w1, b1, w2, d_hidden, d_scores, rows, n_list, d_x,
                                            d_w1, d_b1, d_w2, d_b2, workspace, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_gate_backward launch");
    return TG_OK;
}

tg_status tg_linear(tg_dtype dt, int32_t epilogue, const void* x, int64_t m, int32_t k, const void* w,
                    const void* w_up, int32_t n, const void* residual, void* out, hipStream_t stream) {
    g_err.clear();
    if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "tg_linear is built for bf16 only");
    if (epilogue < TG_LINEAR_STORE || epilogue > TG_LINEAR_SWIGLU)
        return fail(TG_ERR_INVALID_ARGUMENT, "epilogue %d unknown", epilogue);
    if (m < 0) return fail(TG_ERR_INVALID_ARGUMENT, "m=%lld < 0", (long long)m);
    if (k <= 0 || k % 64) return fail(TG_ERR_UNSUPPORTED, "k=%d (built: positive multiples of 64)", k);
    const int n_align = epilogue == TG_LINEAR_SWIGLU ? 64 : 128;
    if (n <= 0 || n % n_align) return fail(TG_ERR_UNSUPPORTED, "n=%d (built: positive multiples of %d)", n, n_align);
    if (m > INT32_MAX / 2) return fail(TG_ERR_UNSUPPORTED, "m=%lld too large", (long long)m);
    if (m == 0) return TG_OK;
    if (!x || !w || !out || (epilogue == TG_LINEAR_SWIGLU && !w_up) || (epilogue == TG_LINEAR_RESIDUAL && !residual))
        return fail(TG_ERR_INVALID_ARGUMENT, "x, w, out (and w_up or residual for that epilogue) must be non-NULL");
    if (!(aligned16(x) && aligned16(w) && aligned16(w_up) && aligned16(out) && aligned16(residual)))
        return fail(TG_ERR_UNSUPPORTED, "x, w, w_up, residual, out must be 16-byte aligned");
    hipError_t e = tg::launch_linear(epilogue, x, m, k, w, w_up, n, residual, out, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_linear launch");
    return TG_OK;
}

}  // extern "C"

namespace {
struct DenseLayout {
    size_t a, qkv, q, k, v, o, h2, mlp, total;
};
DenseLayout dense_layout(int64_t m, const tg_dense_weights& w) {
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t d = (size_t)w.d_model, dh = (size_t)w.head_dim;
    DenseLayout l{};
    size_t o = 0;
    auto take = [&](size_t elems) {
        const size_t at = o;
        o += up(elems * 2 * (size_t)m);
        return at;
    };
    l.a = take(d);
    l.qkv = take((size_t)(w.hq + 2 * w.hkv) * dh);
    l.q = take((size_t)w.hq * dh);
    l.k = take((size_t)w.hkv * dh);
    l.v = take((size_t)w.hkv * dh);
    l.o = take((size_t)w.hq * dh);
    l.h2 = take(d);
    l.mlp = take((size_t)w.d_ff);
    l.total = o;
    return l;
}
tg_status check_dense_weights(const tg_dense_weights* w) {
    if (!w) return fail(TG_ERR_INVALID_ARGUMENT, "weights must be non-NULL");
    if (w->hq <= 0 || w->hkv <= 0 || w->hq % w->hkv)
        return fail(TG_ERR_INVALID_ARGUMENT, "hq=%d must be a positive multiple of hkv=%d", w->hq, w->hkv);
    if (w->head_dim != 64 && w->head_dim != 128)
        return fail(TG_ERR_UNSUPPORTED, "head_dim=%d (built: 64, 128)", w->head_dim);
    if (w->d_model <= 0 || w->d_model % 128)
        return fail(TG_ERR_UNSUPPORTED, "d_model=%d (built: positive multiples of 128)", w->d_model);
    if (w->d_ff <= 0 || w->d_ff % 64) return fail(TG_ERR_UNSUPPORTED, "d_ff=%d (built: positive multiples of 64)", w->d_ff);
    if (((w->hq + 2 * w->hkv) * w->head_dim) % 128)
        return fail(TG_ERR_UNSUPPORTED, "(hq + 2 hkv) * head_dim must be a multiple of 128");
    if (!(w->eps > 0.0f) || !(w->rope_theta > 1.0f) || !(w->tau > 0.0f) || w->tau > 3.0e38f ||
        w->rope_theta > 3.0e38f)
        return fail(TG_ERR_INVALID_ARGUMENT, "eps and tau must be > 0, rope_theta > 1, all finite");
    const void* ptrs[] = {w->ln1, w->wqkv, w->q_norm, w->k_norm, w->wo, w->ln2, w->w_gate, w->w_up, w->w_down};
    for (const void* p : ptrs) {
        if (!p) return fail(TG_ERR_INVALID_ARGUMENT, "every weight pointer must be non-NULL");
        if (!aligned16(p)) return fail(TG_ERR_UNSUPPORTED, "weights must be 16-byte aligned");
    }
    if (!w->gain) return fail(TG_ERR_INVALID_ARGUMENT, "gain must be non-NULL");
    return TG_OK;
}
}  // namespace

extern "C" {

size_t tg_dense_layer_workspace_bytes(const tg_seq* seqs, int32_t n_seqs, const tg_dense_weights* w) {
    tg::SeqTable st_;
    int64_t m = 0;
    if (check_dense_weights(w) != TG_OK || build_seq_table(seqs, n_seqs, &st_, &m) != TG_OK) return 0;
    g_err.clear();
    return dense_layout(m, *w).total;
}

tg_status tg_dense_layer(tg_dtype dt, const void* hidden_kept, const float* bias_kept, const int32_t* pos_kept,
                         const tg_seq* seqs, int32_t n_seqs, const tg_dense_weights* w, void* out, void* k_out,
                         void* v_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err.clear();
    if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "the dense layer is built for bf16 only");
    tg_status st = check_dense_weights(w);
    if (st != TG_OK) return st;
    tg::SeqTable st_;
    int64_t m = 0;
    st = build_seq_table(seqs, n_seqs, &st_, &m);
    if (st != TG_OK) return st;
    if (m == 0) return TG_OK;
    if (!hidden_kept || !bias_kept || !pos_kept || !out)
        return fail(TG_ERR_INVALID_ARGUMENT, "hidden_kept, bias_kept, pos_kept, out must be non-NULL");
    if (!(aligned16(hidden_kept) && aligned16(out) && aligned16(k_out) && aligned16(v_out)))
        return fail(TG_ERR_UNSUPPORTED, "hidden_kept, out, k_out, v_out must be 16-byte aligned");
    const DenseLayout l = dense_layout(m, *w);
    if (!workspace || workspace_bytes < l.total)
        return fail(TG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                    l.total);
    if ((uintptr_t)workspace % 256) return fail(TG_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
    // The attention step's own checks, done here so that a refused call enqueues nothing.
    if ((m / 32 + n_seqs) * (int64_t)w->hq > (int64_t)INT32_MAX)
        return fail(TG_ERR_UNSUPPORTED, "too many attention work items for one launch");
    char* ws = (char*)workspace;
    void *a = ws + l.a, *qkv = ws + l.qkv, *q = ws + l.q, *o = ws + l.o, *h2 = ws + l.h2, *mlp = ws + l.mlp;
    void* k = k_out ? k_out : ws + l.k;
    void* v = v_out ? v_out : ws + l.v;
    const int d = w->d_model, dh = w->head_dim, hq = w->hq, hkv = w->hkv;
    hipError_t e = tg::launch_rmsnorm(hidden_kept, m, d, w->ln1, w->eps, a, stream);
    if (e == hipSuccess)
        e = tg::launch_linear(TG_LINEAR_STORE, a, m, d, w->wqkv, nullptr, (hq + 2 * hkv) * dh, nullptr, qkv, stream);
    if (e == hipSuccess)
        e = tg::launch_qk_norm_rope(qkv, m, hq, hkv, dh, w->q_norm, w->k_norm, pos_kept, w->eps, w->rope_theta, q, k,
                                    v, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_dense_layer launch");
    st = tg_gated_attention(TG_BF16, q, k, v, bias_kept, pos_kept, seqs, n_seqs, hq, hkv, dh, w->gain, w->tau, o,
                            nullptr, stream);
    if (st != TG_OK) return st;
    e = tg::launch_linear(TG_LINEAR_RESIDUAL, o, m, hq * dh, w->wo, nullptr, d, hidden_kept, h2, stream);
    if (e == hipSuccess) e = tg::launch_rmsnorm(h2, m, d, w->ln2, w->eps, a, stream);
    if (e == hipSuccess)
        e = tg::launch_linear(TG_LINEAR_SWIGLU, a, m, d, w->w_gate, w->w_up, w->d_ff, nullptr, mlp, stream);
    if (e == hipSuccess)
        e = tg::launch_linear(TG_LINEAR_RESIDUAL, mlp, m, w->d_ff, w->w_down, nullptr, d, h2, out, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_dense_layer launch");
    return TG_OK;
}

size_t tg_delta_scan_workspace_bytes(const tg_seq* seqs, int32_t n_seqs, int32_t n_heads, int32_t dk, int32_t dv) {
    tg::SeqTable st_;
    int64_t m = 0;
    if (n_heads <= 0 || dk != 128 || dv != 128 || build_seq_table(seqs, n_seqs, &st_, &m) != TG_OK) return 0;
    g_err.clear();
    return tg::delta_scan_workspace_bytes(st_, n_heads);
}

tg_status tg_gated_delta_scan(tg_dtype dt, const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const tg_seq* seqs, int32_t n_seqs, int32_t n_heads, int32_t dk,
                              int32_t dv, const float* state_in, void* out, float* state_out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    g_err.clear();
    if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "the delta scan is built for bf16 q, k, v only");
    if (n_heads <= 0 || n_heads > 65535) return fail(TG_ERR_INVALID_ARGUMENT, "n_heads=%d out of range", n_heads);
    if (dk != 128 || dv != 128) return fail(TG_ERR_UNSUPPORTED, "dk=%d dv=%d (built: 128, 128)", dk, dv);
    tg::SeqTable st_;
    int64_t m = 0;
    tg_status st = build_seq_table(seqs, n_seqs, &st_, &m);
    if (st != TG_OK) return st;
    if (m == 0 && !state_out) return TG_OK;
    if (m > 0 && (!q || !k || !v || !g || !beta || !out))
        return fail(TG_ERR_INVALID_ARGUMENT, "q, k, v, g, beta, out must be non-NULL");
    if (!(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out)))
        return fail(TG_ERR_UNSUPPORTED, "q, k, v, out must be 16-byte aligned");
    const size_t need = tg::delta_scan_workspace_bytes(st_, n_heads);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(TG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                    need);
    if ((uintptr_t)workspace % 16) return fail(TG_ERR_INVALID_ARGUMENT, "workspace not 16-byte aligned");
    hipError_t e = tg::launch_delta_scan(q, k, v, g, beta, st_, n_heads, state_in, out, state_out, workspace, stream);
    if (e != hipSuccess) return hip_fail(e, "tg_gated_delta_scan launch");
    return TG_OK;
}

size_t tg_decode_workspace_bytes(const tg_kv_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv, int32_t head_dim) {
    std::vector<tg::DecTable> t;
    int64_t r = 0;
    size_t ws = 0;
    if (build_decode_tables(TG_BF16, seqs, n_seqs, hq, hkv, head_dim, &t, &r, &ws) != TG_OK) return 0;
    size_t ws32 = 0;
    build_decode_tables(TG_F32, seqs, n_seqs, hq, hkv, head_dim, &t, &r, &ws32);
    g_err.clear();
    return ws > ws32 ? ws : ws32;  // enough for either dtype
}

}  // extern "C"

namespace {

// Shared by both decode entry points. workspace == nullptr with use_static
// selects the library's static per-device scratch.
tg_status decode_common(tg_dtype dt, const void* q_new, const void* k, const void* v, const float* bias,
                        const int32_t* pos, const tg_kv_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                        int32_t head_dim, const float* gain, float tau, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, bool use_static, hipStream_t stream) {
    g_err.clear();
    if (!(tau > 0.0f) || tau != tau || tau > 3.0e38f)
        return fail(TG_ERR_INVALID_ARGUMENT, "tau must be finite and > 0");
    std::vector<tg::DecTable> tables;
    int64_t r_total = 0;
    size_t need = 0;
    tg_status st = build_decode_tables(dt, seqs, n_seqs, hq, hkv, head_dim, &tables, &r_total, &need);
    if (st != TG_OK) return st;
    if (tables.empty()) return TG_OK;
    if (!q_new || !k || !v || !bias || !pos || !gain || !out)
        return fail(TG_ERR_INVALID_ARGUMENT, "q_new, k, v, bias, pos, gain, out must be non-NULL");
    if (!(aligned16(q_new) && aligned16(k) && aligned16(v)))
        return fail(TG_ERR_UNSUPPORTED, "q_new, k, v must be 16-byte aligned");
    if (use_static) {
        if (need > (size_t)TG_DECODE_SCRATCH_BYTES)
            return fail(TG_ERR_WORKSPACE, "this call needs %zu bytes of scratch, the static scratch holds %zu; "
                        "use tg_decode_attention with a workspace", need, (size_t)TG_DECODE_SCRATCH_BYTES);
        hipError_t e = tg::decode_scratch(&workspace);
        if (e != hipSuccess) return hip_fail(e, "tg_decode_attention_noalloc scratch address");
    } else {
        if (!workspace || workspace_bytes < need)
            return fail(TG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                        need);
        if ((uintptr_t)workspace % 4 != 0) return fail(TG_ERR_INVALID_ARGUMENT, "workspace not 4-byte aligned");
    }
    // Launch groups of sequences in stream order; they reuse the workspace
    // (each group's combine finishes before the next group's splits start).
    for (const tg::DecTable& t : tables) {
        hipError_t e = tg::launch_decode(dt, q_new, k, v, bias, pos, t, hq, hkv, head_dim, gain, tau, out, lse,
                                         r_total, workspace, stream);
        if (e != hipSuccess) return hip_fail(e, "tg_decode_attention launch");
    }
    return TG_OK;
}

}  // namespace

extern "C" {

tg_status tg_decode_attention(tg_dtype dt, const void* q_new, const void* k, const void* v, const float* bias,
                              const int32_t* pos, const tg_kv_seq* seqs, int32_t n_seqs, int32_t hq, int32_t hkv,
                              int32_t head_dim, const float* gain, float tau, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_common(dt, q_new, k, v, bias, pos, seqs, n_seqs, hq, hkv, head_dim, gain, tau, out, lse, workspace,
                         workspace_bytes, false, stream);
}

tg_status tg_decode_attention_noalloc(tg_dtype dt, const void* q_new, const void* k, const void* v,
                                      const float* bias, const int32_t* pos, const tg_kv_seq* seqs, int32_t n_seqs,
                                      int32_t hq, int32_t hkv, int32_t head_dim, const float* gain, float tau,
                                      void* out, float* lse, hipStream_t stream) {
    return decode_common(dt, q_new, k, v, bias, pos, seqs, n_seqs, hq, hkv, head_dim, gain, tau, out, lse, nullptr, 0,
                         true, stream);
}

}  // extern "C"
