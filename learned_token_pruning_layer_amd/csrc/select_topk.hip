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
//     Prompts whose document fits (up to 36864 rows) keep their keys in LDS
//     for the whole kernel, so HBM is read once.
//  2. A 3-pass MSB radix select (11, 11 and 10-bit digits; LDS histograms
//     with integer atomics; a block scan over the bins from the top) finds
//     the k-th largest key T and rem = how many keys equal to T are kept.
//  3. Emission: each wave owns 1024 consecutive rows, walked 64 at a time
//     (lane-consecutive, conflict-free LDS reads). A row is "above"
//     (outside the document, or key > T) or "tied" (document key == T);
//     wavefront ballots + popcounts give each wave its totals, one scan of
//     the 16 wave totals gives each wave its starting rank, and a second walk
//     ranks every row with ballot + mbcnt. Kept rows are the above rows and
//     the first rem tied rows; a kept row's output slot is
//     (#above before it) + min(#tied before it, rem), so rows land in
//     ascending order without a sort.
// Integer work only: the result is bit-exact and deterministic.
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int ST = 1024;    // threads per workgroup (16 waves)
constexpr int NW = ST / 64;
constexpr int WROWS = 1024; // consecutive rows per wave in the emission
constexpr int CAP = 36864;  // document keys kept in LDS (144 KB)
constexpr int NB = 2048;    // histogram bins (11-bit digits)

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number
    if ((b & 0x7fffffffu) == 0u) b = 0u;             // -0 ranks as +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive scan of v over the wave (shuffle-up ladder).
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

__global__ __launch_bounds__(ST) void select_kernel(const float* __restrict__ scores, SeqTable t,
                                                    int32_t* __restrict__ kept) {
    __shared__ uint32_t keys[CAP];
    __shared__ uint32_t hist[NB];
    __shared__ uint32_t wtot[NW][2];
    __shared__ uint32_t pick[2];

    const SeqDesc sd = t.s[blockIdx.x];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t dbeg = sd.start + sd.doc_begin;
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const int32_t k = sd.k_doc;
    const bool resident = n_doc <= CAP;

    // mode 0: keep no document row; 1: keep all; 2: threshold T with rem ties.
    const int mode = (k == 0) ? 0 : (k == n_doc ? 1 : 2);
    uint32_t thr = 0, rem = 0;
    if (mode == 2) {
        if (resident) {
            for (int32_t i0 = 0; i0 < n_doc; i0 += ST * 16) {
                float v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int32_t i = i0 + u * ST + tid;
                    v[u] = (i < n_doc) ? scores[dbeg + i] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int32_t i = i0 + u * ST + tid;
                    if (i < n_doc) keys[i] = score_key(v[u]);
                }
            }
        }
        uint32_t prefix = 0, mask = 0;
        rem = (uint32_t)k;
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const uint32_t dmask = pass == 2 ? 1023u : 2047u;
            const int nbins = (int)dmask + 1;
            hist[tid] = 0;
            hist[tid + ST] = 0;
            __syncthreads();
            for (int32_t i0 = 0; i0 < n_doc; i0 += ST * 4) {
                uint32_t kv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int32_t i = i0 + u * ST + tid;
                    kv[u] = (i < n_doc) ? (resident ? keys[i] : score_key(scores[dbeg + i])) : 0u;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int32_t i = i0 + u * ST + tid;
                    if (i < n_doc && (kv[u] & mask) == prefix) atomicAdd(&hist[(kv[u] >> shift) & dmask], 1u);
                }
            }
            __syncthreads();
            // Bins from the top, two per thread: bins nbins-1-2t and nbins-2-2t.
            const int b0 = nbins - 1 - 2 * tid, b1 = b0 - 1;
            const uint32_t c0 = b0 >= 0 ? hist[b0] : 0u, c1 = b1 >= 0 ? hist[b1] : 0u;
            const uint32_t inc = wave_scan(c0 + c1, lane);
            if (lane == 63) wtot[wave][0] = inc;
            __syncthreads();
            uint32_t before = inc - (c0 + c1);
            for (int w = 0; w < wave; ++w) before += wtot[w][0];
            if (before < rem && rem <= before + c0) {
                pick[0] = (uint32_t)b0;
                pick[1] = rem - before;
            } else if (before + c0 < rem && rem <= before + c0 + c1) {
                pick[0] = (uint32_t)b1;
                pick[1] = rem - before - c0;
            }
            __syncthreads();
            prefix |= pick[0] << shift;
            mask |= dmask << shift;
            rem = pick[1];
            __syncthreads();
        }
        thr = prefix;
    }

    // Emission in row order, NW*WROWS rows per step.
    // Row class: 0 dropped, 1 above, 2 tied.
    const int32_t len = sd.len;
    auto classify = [&](int32_t r) -> uint32_t {
        if (r >= len) return 0u;
        const bool in_doc = r >= sd.doc_begin && r < sd.doc_end;
        if (!in_doc || mode == 1) return 1u;
        if (mode == 0) return 0u;
        const int32_t i = r - sd.doc_begin;
        const uint32_t key = resident ? keys[i] : score_key(scores[dbeg + i]);
        return key > thr ? 1u : (key == thr ? 2u : 0u);
    };
    uint32_t carry_above = 0, carry_tied = 0;
    for (int32_t r0 = 0; r0 < len; r0 += NW * WROWS) {
        const int32_t wbase = r0 + wave * WROWS;
        uint32_t na = 0, nt = 0;
        for (int u = 0; u < WROWS / 64; ++u) {
            const uint32_t c = classify(wbase + u * 64 + lane);
            na += (uint32_t)__popcll(__ballot(c == 1u));
            nt += (uint32_t)__popcll(__ballot(c == 2u));
        }
        if (lane == 0) {
            wtot[wave][0] = na;
            wtot[wave][1] = nt;
        }
        __syncthreads();
        uint32_t pa = carry_above, pt = carry_tied, ta = 0, tt = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t a = wtot[w][0], b = wtot[w][1];
            if (w < wave) { pa += a; pt += b; }
            ta += a;
            tt += b;
        }
        if (pa < (uint32_t)sd.n_kept) {  // this wave has kept rows to place
            for (int u = 0; u < WROWS / 64; ++u) {
                const int32_t r = wbase + u * 64 + lane;
                const uint32_t c = classify(r);
                const uint64_t ba = __ballot(c == 1u), bt = __ballot(c == 2u);
                const uint32_t ma = pa + lanes_below(ba), mt = pt + lanes_below(bt);
                if (c == 1u || (c == 2u && mt < rem)) {
                    const uint32_t slot = ma + (mt < rem ? mt : rem);
                    if (slot < (uint32_t)sd.n_kept)  // always true when the counts are right
                        kept[sd.kept_off + slot] = (int32_t)(sd.start + r);
                }
                pa += (uint32_t)__popcll(ba);
                pt += (uint32_t)__popcll(bt);
            }
        }
        carry_above += ta;
        carry_tied += tt;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_select(const float* scores, const SeqTable& t, int32_t* kept, hipStream_t st) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)t.n), dim3(ST), 0, st, scores, t, kept);
    return hipGetLastError();
}

}  // namespace tg
