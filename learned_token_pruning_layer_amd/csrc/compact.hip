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
// HBM-bound row copy. Each workgroup owns a few consecutive kept rows and
// copies every tensor's rows in 16-byte units, four loads in flight per
// thread before the stores, so consecutive lanes touch consecutive bytes of
// a row (coalesced) on both sides.
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int CT = 256;
constexpr int MAX_RPB = 16;

__device__ __forceinline__ int find_seq(const SeqTable& t, int64_t row) {
    int b = 0;
    for (int i = 1; i < t.n; ++i)
        if (t.s[i].start <= row) b = i;
    return b;
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
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.x * rpb;
    const int nr = (int)((m - m0) < rpb ? (m - m0) : rpb);
    if (tid < nr) {
        const int64_t r = kept[m0 + tid];
        const SeqDesc& sd = t.s[find_seq(t, r)];
        // A row id outside every prompt breaks the contract; it is never
        // dereferenced (its outputs are left untouched).
        const bool ok = r >= sd.start && r < sd.start + sd.len;
        src_row[tid] = ok ? r : -1;
        if (ok) {
            if (pos_kept) pos_kept[m0 + tid] = pos ? pos[r] : (int32_t)(r - sd.start);
            if (bias_kept) {
                const int64_t rel = r - sd.start;
                const bool in_doc = rel >= sd.doc_begin && rel < sd.doc_end;
                bias_kept[m0 + tid] = in_doc ? log_sigmoid(scores[r]) : 0.0f;
            }
        }
    }
    __syncthreads();
    for (int gi = 0; gi < g.n; ++gi) {
        const GatherDesc gd = g.g[gi];
        const int units = (int)gd.units;
        const int total = nr * units;
        for (int u0 = 0; u0 < total; u0 += 4 * CT) {
            uint4 val[4];
            int rr[4], cc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = u0 + q * CT + tid;
                rr[q] = u / units;
                cc[q] = u - rr[q] * units;
                if (u < total && src_row[rr[q]] >= 0)
                    val[q] = *(const uint4*)(gd.src + src_row[rr[q]] * gd.src_stride + (int64_t)cc[q] * 16);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = u0 + q * CT + tid;
                if (u < total && src_row[rr[q]] >= 0)
                    *(uint4*)(gd.dst + (m0 + rr[q]) * gd.dst_stride + (int64_t)cc[q] * 16) = val[q];
            }
        }
    }
}

}  // namespace

hipError_t launch_compact(const int32_t* kept, int64_t m, const SeqTable& t, const GatherTable& g,
                          const int32_t* pos, int32_t* pos_kept, const float* scores,
                          float* bias_kept, hipStream_t st) {
    // Aim for >= ~1024 workgroups so all 256 CUs stay busy; at most 16 rows each.
    int64_t rpb = (m + 1023) / 1024;
    if (rpb < 1) rpb = 1;
    if (rpb > MAX_RPB) rpb = MAX_RPB;
    const int64_t blocks = (m + rpb - 1) / rpb;
    hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(CT), 0, st, kept, m, t, g,
                       (int)rpb, pos, pos_kept, scores, bias_kept);
    return hipGetLastError();
}

}  // namespace tg
