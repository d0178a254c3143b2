// Step 3 - compaction: gather the kept rows of several row-major tensors,
// their original positions, and their attention bias, in one launch.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (layers above the gate
// process only the kept tokens and create no KV entries for the pruned
// ones); ai.info news, section "TokenGate impara quali token mantenere" (only
// the kept tokens' representations are sent upward); the bias is the kept
// token's score per section "Was ist token-gated Attention?" of the spke.com
// article, in the form logsigmoid(s) for document rows and 0 for the rest.
//
// HBM-bound row copy. A workgroup owns a few consecutive kept rows and
// flattens (tensor, row, 16-byte unit) of every gathered tensor into one
// index space; each thread issues all of its loads (up to CU units) before
// any store, so a workgroup keeps its whole share of bytes in flight at
// once, and consecutive lanes touch consecutive bytes of a row (coalesced)
// on both sides.
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

#define GLOBAL_AS __attribute__((address_space(1)))
typedef const GLOBAL_AS u32x4* gsrc_t;
typedef GLOBAL_AS u32x4* gdst_t;

constexpr int CT = 256;
constexpr int CU = 12;       // 16-byte units per thread (in flight at once)
constexpr int MAX_RPB = 16;

// The prompt holding row `row`: its first row and document range. Walks
// the table with uniform indices (a per-lane index into the kernel argument
// would put the table in scratch memory).
struct RowSeq {
    int64_t start, len;
    int32_t doc_begin, doc_end;
};
__device__ __forceinline__ RowSeq find_seq(const SeqTable& t, int64_t row) {
    RowSeq q{t.s[0].start, t.s[0].len, t.s[0].doc_begin, t.s[0].doc_end};
    for (int i = 1; i < t.n; ++i)
        if (t.s[i].start <= row) q = RowSeq{t.s[i].start, t.s[i].len, t.s[i].doc_begin, t.s[i].doc_end};
    return q;
}

__device__ __forceinline__ float log_sigmoid(float s) {
    return fminf(s, 0.0f) - log1pf(expf(-fabsf(s)));
}

__global__ __launch_bounds__(CT) void compact_kernel(const int32_t* __restrict__ kept, int64_t m,
                                                     SeqTable t, GatherTable g, int rpb,
                                                     const int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ pos_kept,
                                                     const float* __restrict__ scores,
                                                     float* __restrict__ bias_kept) {
    __shared__ int64_t src_row[MAX_RPB];
    __shared__ int32_t unit_base[TG_MAX_GATHERS + 1];  // prefix of units per row over tensors
    __shared__ GatherDesc gds[TG_MAX_GATHERS];         // descriptors, indexable per thread
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.x * rpb;
    const int nr = (int)((m - m0) < rpb ? (m - m0) : rpb);
    // Only the kept index precedes the barrier: the row copies depend on it,
    // while the position and bias loads go out after the copies' loads.
    int64_t my_row = -1;
    RowSeq sd{};
    if (tid < nr) {
        const int64_t r = kept[m0 + tid];
        sd = find_seq(t, r);
        // A row id outside every prompt breaks the contract; it is never
        // dereferenced (its outputs are left untouched).
        my_row = (r >= sd.start && r < sd.start + sd.len) ? r : -1;
        src_row[tid] = my_row;
    }
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < g.n; ++i) {  // uniform index into the kernel argument
            gds[i] = g.g[i];
            unit_base[i] = acc;
            acc += (int)g.g[i].units;
        }
        unit_base[g.n] = acc;
    }
    __syncthreads();
    const int per_row = unit_base[g.n];
    const int total = nr * per_row;
    for (int u0 = 0; u0 < total; u0 += CU * CT) {
        u32x4 val[CU];
        gdst_t dst[CU];
#pragma unroll
        for (int q = 0; q < CU; ++q) {
            const int u = u0 + q * CT + tid;
            // Loads are unconditional (a lane with nothing to copy re-reads the
            // first unit of the first tensor) so they all issue together.
            gsrc_t src = (gsrc_t)gds[0].src;
            dst[q] = nullptr;
            if (u < total) {
                const int rr = u / per_row;
                int w = u - rr * per_row;
                int gi = 0;
#pragma unroll
                for (int i = 1; i < TG_MAX_GATHERS; ++i) gi += (i < g.n && unit_base[i] <= w) ? 1 : 0;
                w -= unit_base[gi];
                const int64_t sr = src_row[rr];
                if (sr >= 0) {
                    const GatherDesc& gd = gds[gi];
                    src = (gsrc_t)(gd.src + sr * gd.src_stride + (int64_t)w * 16);
                    dst[q] = (gdst_t)(gd.dst + (m0 + rr) * gd.dst_stride + (int64_t)w * 16);
                }
            }
            val[q] = *src;
        }
        if (u0 == 0 && my_row >= 0) {
            if (pos_kept) pos_kept[m0 + tid] = pos ? pos[my_row] : (int32_t)(my_row - sd.start);
            if (bias_kept) {
                const int64_t rel = my_row - sd.start;
                const bool in_doc = rel >= sd.doc_begin && rel < sd.doc_end;
                bias_kept[m0 + tid] = in_doc ? log_sigmoid(scores[my_row]) : 0.0f;
            }
        }
#pragma unroll
        for (int q = 0; q < CU; ++q)
            if (dst[q]) *dst[q] = val[q];
    }
    if (total == 0 && my_row >= 0) {  // no tensors to gather: positions and bias only
        if (pos_kept) pos_kept[m0 + tid] = pos ? pos[my_row] : (int32_t)(my_row - sd.start);
        if (bias_kept) {
            const int64_t rel = my_row - sd.start;
            const bool in_doc = rel >= sd.doc_begin && rel < sd.doc_end;
            bias_kept[m0 + tid] = in_doc ? log_sigmoid(scores[my_row]) : 0.0f;
        }
    }
}

// Position check: counts the kept rows whose position is below the previous
// kept row's in the same prompt (one thread per kept row; integer atomics,
// so the count is exact and deterministic).
__global__ __launch_bounds__(64) void pos_check_zero_kernel(int32_t* __restrict__ n_bad) {
    if (threadIdx.x == 0) *n_bad = 0;
}
__global__ __launch_bounds__(256) void pos_check_kernel(const int32_t* __restrict__ pos, int64_t m, SeqTable t,
                                                       int32_t* __restrict__ n_bad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m) return;
    int b = 0;
    for (int s = 1; s < t.n; ++s)
        if (t.s[s].kept_off <= i) b = s;
    if (i > t.s[b].kept_off && pos[i] < pos[i - 1]) atomicAdd(n_bad, 1);
}

}  // namespace

hipError_t launch_check_positions(const int32_t* pos, int64_t m, const SeqTable& t, int32_t* n_bad,
                                  hipStream_t st) {
    hipLaunchKernelGGL(pos_check_zero_kernel, dim3(1), dim3(64), 0, st, n_bad);
    if (m > 0)
        hipLaunchKernelGGL(pos_check_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, pos, m, t, n_bad);
    return hipGetLastError();
}

hipError_t launch_compact(const int32_t* kept, int64_t m, const SeqTable& t, const GatherTable& g,
                          const int32_t* pos, int32_t* pos_kept, const float* scores,
                          float* bias_kept, hipStream_t st) {
    // Rows per workgroup: as many as fit CU units per thread, so every
    // thread's loads are issued together; at most 16 rows.
    int64_t per_row = 0;
    for (int i = 0; i < g.n; ++i) per_row += g.g[i].units;
    int64_t rpb = per_row > 0 ? (int64_t)(CU * CT) / per_row : MAX_RPB;
    if (rpb < 1) rpb = 1;
    if (rpb > MAX_RPB) rpb = MAX_RPB;
    const int64_t blocks = (m + rpb - 1) / rpb;
    hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(CT), 0, st, kept, m, t, g,
                       (int)rpb, pos, pos_kept, scores, bias_kept);
    return hipGetLastError();
}

}  // namespace tg
