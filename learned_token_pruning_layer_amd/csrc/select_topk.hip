// Step 2 - per-prompt top-K selection over document rows, stable by row id.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (a top-K selector keeps the
// best-scored tokens; only the document part of the prompt may be removed,
// the question never); ai4bro.com post, section on how learned token pruning
// works (same rule). The pages do not say how ties break: here the lower row
// id wins, -0 equals +0 and NaN ranks below every number.
//
// One 1024-thread workgroup per prompt:
//  1. Scores map to order-preserving u32 keys (larger key = better rank).
//  2. A 4-pass MSB radix select (8-bit digits, LDS histograms with integer
//     atomics, a block scan over the 256 bins from the top) finds the k-th
//     largest key T and rem = how many keys equal to T are kept.
//  3. Emission walks the prompt in row order, 1024 rows per step. Each row
//     is "above" (outside the document, or key > T) or "tied" (document key
//     == T); wavefront ballots plus mbcnt give the rank of each row within
//     its wave, a 16-entry LDS table of wave totals gives the block prefix.
//     Kept rows are the above rows and the first rem tied rows; a kept row's
//     output slot is (#above before it) + min(#tied before it, rem), so rows
//     land in ascending order without a sort.
// Integer work only: the result is bit-exact and deterministic.
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int ST = 1024;   // threads per workgroup (16 waves)
constexpr int NW = ST / 64;
constexpr int UNR = 8;     // rows loaded per thread before use (memory-level parallelism)

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number
    if ((b & 0x7fffffffu) == 0u) b = 0u;             // -0 ranks as +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ __launch_bounds__(ST) void select_kernel(const float* __restrict__ scores, SeqTable t,
                                                    int32_t* __restrict__ kept) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wtot[NW][2];
    __shared__ uint32_t pick[2];

    const SeqDesc sd = t.s[blockIdx.x];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t dbeg = sd.start + sd.doc_begin;
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const int32_t k = sd.k_doc;

    // mode 0: keep no document row; 1: keep all; 2: threshold T with rem ties.
    const int mode = (k == 0) ? 0 : (k == n_doc ? 1 : 2);
    uint32_t thr = 0, rem = 0;
    if (mode == 2) {
        uint32_t prefix = 0, mask = 0;
        rem = (uint32_t)k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int32_t i0 = 0; i0 < n_doc; i0 += ST * UNR) {
                float v[UNR];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int32_t i = i0 + u * ST + tid;
                    v[u] = (i < n_doc) ? scores[dbeg + i] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int32_t i = i0 + u * ST + tid;
                    const uint32_t key = score_key(v[u]);
                    if (i < n_doc && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
            // Bins from the top: thread b < 256 owns bin 255 - b. Inclusive scan
            // within each wave, then add the totals of the waves before.
            uint32_t c = 0, inc = 0;
            if (tid < 256) {
                c = hist[255 - tid];
                inc = c;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t o = __shfl_up(inc, off);
                    if (lane >= off) inc += o;
                }
                if (lane == 63) wtot[wave][0] = inc;
            }
            __syncthreads();
            if (tid < 256) {
                for (int w = 0; w < wave; ++w) inc += wtot[w][0];
                const uint32_t exc = inc - c;
                if (exc < rem && rem <= inc) {
                    pick[0] = 255u - (uint32_t)tid;
                    pick[1] = rem - exc;
                }
            }
            __syncthreads();
            prefix |= pick[0] << shift;
            mask |= 255u << shift;
            rem = pick[1];
            __syncthreads();
        }
        thr = prefix;
    }

    // Emission in row order.
    uint32_t carry_above = 0, carry_tied = 0;
    const int32_t len = sd.len;
    for (int32_t r0 = 0; r0 < len; r0 += ST * UNR) {
        float v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int32_t r = r0 + u * ST + tid;
            const bool in_doc = r < len && r >= sd.doc_begin && r < sd.doc_end;
            v[u] = (mode == 2 && in_doc) ? scores[sd.start + r] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int32_t r = r0 + u * ST + tid;
            const bool valid = r < len;
            const bool in_doc = valid && r >= sd.doc_begin && r < sd.doc_end;
            bool above, tied = false;
            if (mode == 0) {
                above = valid && !in_doc;
            } else if (mode == 1) {
                above = valid;
            } else {
                const uint32_t key = score_key(v[u]);
                above = valid && (!in_doc || key > thr);
                tied = in_doc && key == thr;
            }
            const uint64_t ba = __ballot(above);
            const uint64_t bt = __ballot(tied);
            if (lane == 0) {
                wtot[wave][0] = (uint32_t)__popcll(ba);
                wtot[wave][1] = (uint32_t)__popcll(bt);
            }
            __syncthreads();
            uint32_t pa = 0, pt = 0, ta = 0, tt = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const uint32_t a = wtot[w][0], b = wtot[w][1];
                if (w < wave) { pa += a; pt += b; }
                ta += a;
                tt += b;
            }
            const uint32_t above_before = carry_above + pa + lanes_below(ba);
            const uint32_t tied_before = carry_tied + pt + lanes_below(bt);
            if (above || (tied && tied_before < rem)) {
                const uint32_t slot = above_before + (tied_before < rem ? tied_before : rem);
                if (slot < (uint32_t)sd.n_kept)  // always true when the counts are right
                    kept[sd.kept_off + slot] = (int32_t)(sd.start + r);
            }
            carry_above += ta;
            carry_tied += tt;
            __syncthreads();
        }
    }
}

}  // namespace

hipError_t launch_select(const float* scores, const SeqTable& t, int32_t* kept, hipStream_t st) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)t.n), dim3(ST), 0, st, scores, t, kept);
    return hipGetLastError();
}

}  // namespace tg
