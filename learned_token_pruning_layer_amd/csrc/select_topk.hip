// Step 2 - per-prompt top-K selection over document rows, stable by row id.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (a top-K selector keeps the
// best-scored tokens; only the document part of the prompt may be removed,
// the question never); ai4bro.com post, section on how learned token pruning
// works (same rule). The pages do not say how ties break: here the lower row
// id wins, -0 equals +0 and NaN ranks below every number.
//
// One 1024-thread workgroup per prompt.
//  1. Scores map to order-preserving u32 keys (larger key = better rank).
//     Prompts of up to 32768 rows keep every key in registers (WU = 16 or
//     32 per lane) for the whole kernel: HBM is read once (coalesced, then
//     transposed through LDS so that lane l of wave w holds the WU
//     consecutive rows starting at (64w + l) * WU). Rows outside the
//     document hold key 0 and are not counted: while the chosen digits are
//     all zero they fall into bin 0, whose count is corrected by their known
//     number, so the inner loops carry no bounds or document tests. Longer
//     prompts stream their scores from global memory in every pass.
//  2. A 3-pass MSB radix select (11, 11 and 10-bit digits; LDS histograms
//     with integer atomics; a DPP wave scan over the bins from the top)
//     finds the k-th largest key T and rem = how many keys equal to T are
//     kept.
//  3. Emission: a row is "above" (outside the document, or key > T) or
//     "tied" (document key == T); each lane classifies its rows into two bit
//     masks. Kept rows are the above rows and the first rem tied rows; a
//     kept row's output slot is (#above before it) + min(#tied before it,
//     rem), so rows land in ascending order without a sort. Register path:
//     popcounts of the masks, a DPP scan over the wave and one pass over the
//     16 wave totals rank every lane's first row; the lane then walks its
//     own consecutive rows, writing each kept row id to its slot of an LDS
//     staging array (rows not kept write a per-lane scratch word, so no lane
//     masking is needed), and the staged slots go out in one coalesced copy.
//     Streaming path: lane l of a wave step holds rows l, l+64, ...; ballots
//     + mbcnt rank them and kept rows are stored directly.
// The kernel is bound by its own instruction count on one CU, so the hot
// loops are kept to a few instructions per key.
// Integer work only: the result is bit-exact and deterministic.
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int ST = 1024;               // threads per workgroup (16 waves)
constexpr int NW = ST / 64;
constexpr int NB = 2048;               // histogram bins (11-bit digits)
constexpr int HTOT = 2 * NB + NB / 2;  // the three passes' histograms (11, 11 and 10 bits)
constexpr int SU = 16;                 // rows per lane per emission step of the streaming path

constexpr int RMAX = ST * 32;                // rows of the largest register path
constexpr int STAGE = RMAX + RMAX / 64 + 64;  // padded transpose / staging words + scratch words

struct Smem {
    uint32_t hist[HTOT];  // one histogram per pass, cleared once
    uint32_t wtot[NW][2];
    uint32_t pick[3][2];  // per pass: chosen bin, rank inside it
    uint32_t stage[STAGE];  // register path: key transpose, then kept-slot staging
};

// Padded LDS index of row r in the key transpose: one spare word per 64
// rows spreads both the row-order writes and the lane-contiguous reads
// (stride 16 or 32 words) over all 64 banks.
__device__ __forceinline__ int tpad(int r) { return r + (r >> 6); }

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number
    if ((b & 0x7fffffffu) == 0u) b = 0u;             // -0 ranks as +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive scan of v over the wave with DPP moves (no LDS round trips):
// shifts by 1, 2, 4 and 8 inside each 16-lane row, then lane 15 of each
// row is added to the next row and lane 31 to the upper half. Lanes whose
// source falls outside the row, and rows masked off, add 0.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return (uint32_t)x;
}

// Radix digit of pass p: bits [shift, shift + width) of the key.
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 1023u : 2047u; }

// After pass `pass`'s histogram is complete: find the bin that holds the
// rem-th largest counted key (bins scanned from the top; bin 0 is first
// reduced by `excess` uncounted keys) and narrow prefix/mask/rem to it.
__device__ __forceinline__ void pick_bin(Smem& sm, int pass, uint32_t excess, uint32_t& prefix,
                                         uint32_t& mask, uint32_t& rem, int tid, int lane, int wave) {
    const int shift = digit_shift(pass);
    const uint32_t dmask = digit_mask(pass);
    const uint32_t* h = sm.hist + pass * NB;
    const int b0 = (int)dmask - 2 * tid, b1 = b0 - 1;  // two bins per thread, from the top
    uint32_t c0 = b0 >= 0 ? h[b0] : 0u, c1 = b1 >= 0 ? h[b1] : 0u;
    if (b0 == 0) c0 -= excess;
    if (b1 == 0) c1 -= excess;
    const uint32_t inc = wave_scan(c0 + c1);
    if (lane == 63) sm.wtot[wave][0] = inc;
    __syncthreads();
    uint32_t before = inc - (c0 + c1);
#pragma unroll
    for (int w = 0; w < NW; ++w) before += (w < wave) ? sm.wtot[w][0] : 0u;
    if (before < rem && rem <= before + c0) {
        sm.pick[pass][0] = (uint32_t)b0;
        sm.pick[pass][1] = rem - before;
    } else if (before + c0 < rem && rem <= before + c0 + c1) {
        sm.pick[pass][0] = (uint32_t)b1;
        sm.pick[pass][1] = rem - before - c0;
    }
    __syncthreads();
    prefix |= sm.pick[pass][0] << shift;
    mask |= dmask << shift;
    rem = sm.pick[pass][1];
}

// Ranks and stores one emission step: the wave's rows wbase + 64u + lane,
// u < U, classified in ma_bits (above) / mt_bits (tied), with na / nt this
// wave's totals. carry_* count the rows of earlier steps; updated here.
template <int U>
__device__ __forceinline__ void place_rows(Smem& sm, const SeqDesc& sd, int32_t* __restrict__ kept,
                                           int32_t wbase, uint32_t ma_bits, uint32_t mt_bits,
                                           uint32_t na, uint32_t nt, uint32_t rem,
                                           uint32_t& carry_above, uint32_t& carry_tied, int lane,
                                           int wave) {
    if (lane == 0) {
        sm.wtot[wave][0] = na;
        sm.wtot[wave][1] = nt;
    }
    __syncthreads();
    uint32_t pa = carry_above, pt = carry_tied, ta = 0, tt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t a = sm.wtot[w][0], b = sm.wtot[w][1];
        if (w < wave) { pa += a; pt += b; }
        ta += a;
        tt += b;
    }
    if (pa < (uint32_t)sd.n_kept) {  // this wave has kept rows to place
#pragma nounroll
        for (int u = 0; u < U; ++u) {
            const bool above = (ma_bits >> u) & 1u, tied = (mt_bits >> u) & 1u;
            const uint64_t ba = __ballot(above), bt = __ballot(tied);
            const uint32_t ma = pa + lanes_below(ba), mt = pt + lanes_below(bt);
            if (above || (tied && mt < rem)) {
                const uint32_t slot = ma + (mt < rem ? mt : rem);
                if (slot < (uint32_t)sd.n_kept)  // always true when the counts are right
                    kept[sd.kept_off + slot] = (int32_t)(sd.start + wbase + u * 64 + lane);
            }
            pa += (uint32_t)__popcll(ba);
            pt += (uint32_t)__popcll(bt);
        }
    }
    carry_above += ta;
    carry_tied += tt;
    __syncthreads();  // wtot is rewritten by the next step
}

// Prompts of at most NW*64*WU rows: every key in registers.
template <int WU>  // WU <= 32: a lane's rows fit one 32-bit mask
__device__ __forceinline__ void select_registers(Smem& sm, const SeqDesc& sd,
                                                 const float* __restrict__ scores,
                                                 int32_t* __restrict__ kept, int tid, int lane,
                                                 int wave) {
    static_assert(WU <= 32, "a lane's rows must fit one 32-bit mask");
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const int32_t k = sd.k_doc;
    const int mode = (k == 0) ? 0 : (k == n_doc ? 1 : 2);  // keep no / all / top-k document rows
    const int32_t wbase = wave * 64 * WU;
    const int32_t rbase = (wave * 64 + lane) * WU;  // this lane's WU consecutive rows
    uint32_t key[WU];
    uint32_t thr = 0, rem = 0;
    if (mode == 2) {
        for (int i = tid; i < HTOT; i += ST) sm.hist[i] = 0u;
        float f[WU];
#pragma unroll
        for (int u = 0; u < WU; ++u) {  // row order, clamped into the document: every load is valid
            const int32_t r = wbase + u * 64 + lane;
            f[u] = scores[sd.start + min(max(r, sd.doc_begin), sd.doc_end - 1)];
        }
#pragma unroll
        for (int u = 0; u < WU; ++u) {
            const int32_t r = wbase + u * 64 + lane;
            sm.stage[tpad(r)] = (r >= sd.doc_begin && r < sd.doc_end) ? score_key(f[u]) : 0u;
        }
        __syncthreads();  // histograms cleared, keys staged
#pragma unroll
        for (int u = 0; u < WU; ++u) key[u] = sm.stage[tpad(rbase + u)];
        // Rows of this workgroup's range that are not document rows (key 0).
        const uint32_t npad = (uint32_t)(NW * 64 * WU - n_doc);
        uint32_t prefix = 0, mask = 0;
        rem = (uint32_t)k;
        // Pass 0 counts every key.
#pragma unroll
        for (int u = 0; u < WU; ++u) atomicAdd(&sm.hist[key[u] >> 21], 1u);
        __syncthreads();
        pick_bin(sm, 0, npad, prefix, mask, rem, tid, lane, wave);
#pragma nounroll
        for (int pass = 1; pass < 3; ++pass) {
            const int shift = digit_shift(pass);
            const uint32_t dmask = digit_mask(pass);
            uint32_t* const h = sm.hist + pass * NB;
#pragma unroll
            for (int u = 0; u < WU; ++u)
                if ((key[u] & mask) == prefix) atomicAdd(&h[(key[u] >> shift) & dmask], 1u);
            __syncthreads();
            pick_bin(sm, pass, prefix == 0 ? npad : 0u, prefix, mask, rem, tid, lane, wave);
        }
        thr = prefix;
    } else {
#pragma unroll
        for (int u = 0; u < WU; ++u) key[u] = 0u;
    }

    // Bit u of each mask describes row rbase + u. A lane's rows are
    // consecutive, so "inside the prompt" and "inside the document" are bit
    // ranges; only the key comparisons are per row.
    auto range_bits = [&](int32_t lo, int32_t hi) -> uint32_t {  // rows [lo, hi) of this lane
        const int32_t a = min(max(lo - rbase, 0), WU), b = min(max(hi - rbase, 0), WU);
        const uint32_t upto_b = b >= 32 ? 0xffffffffu : ((1u << b) - 1u);
        const uint32_t upto_a = a >= 32 ? 0xffffffffu : ((1u << a) - 1u);
        return upto_b & ~upto_a;
    };
    const uint32_t in_len = range_bits(0, sd.len);
    const uint32_t in_doc = range_bits(sd.doc_begin, sd.doc_end);
    uint32_t ma_bits, mt_bits;  // above / tied
    if (mode == 2) {
        uint32_t gt_bits = 0, eq_bits = 0;
#pragma unroll
        for (int u = 0; u < WU; ++u) {
            gt_bits |= (key[u] > thr ? 1u : 0u) << u;
            eq_bits |= (key[u] == thr ? 1u : 0u) << u;
        }
        ma_bits = in_len & (~in_doc | gt_bits);
        mt_bits = in_doc & eq_bits;
    } else {
        ma_bits = mode == 1 ? in_len : (in_len & ~in_doc);
        mt_bits = 0u;
    }
    const uint32_t ca = (uint32_t)__popc(ma_bits), ct = (uint32_t)__popc(mt_bits);
    const uint32_t ia = wave_scan(ca), it = wave_scan(ct);
    if (lane == 63) {
        sm.wtot[wave][0] = ia;
        sm.wtot[wave][1] = it;
    }
    __syncthreads();  // also: every lane has read its keys from the stage
    uint32_t pa = ia - ca, pt = it - ct;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        pa += (w < wave) ? sm.wtot[w][0] : 0u;
        pt += (w < wave) ? sm.wtot[w][1] : 0u;
    }
    const uint32_t n_kept = (uint32_t)sd.n_kept;
    const int trash = RMAX + RMAX / 64 + lane;
#pragma unroll
    for (int u = 0; u < WU; ++u) {
        const uint32_t above = (ma_bits >> u) & 1u, tied = (mt_bits >> u) & 1u;
        const uint32_t slot = pa + min(pt, rem);
        // slot < n_kept always holds for a kept row when the counts are right
        const uint32_t keep = (above | (tied & (uint32_t)(pt < rem))) & (uint32_t)(slot < n_kept);
        sm.stage[keep ? (int)slot : trash] = (uint32_t)(sd.start + rbase + u);
        pa += above;
        pt += tied;
    }
    __syncthreads();
    for (int j = tid; j < sd.n_kept; j += ST) kept[sd.kept_off + j] = (int32_t)sm.stage[j];
}

// Longer prompts: scores are re-read from global memory in every pass and
// in the emission (NW*64*SU rows per step).
__device__ __forceinline__ void select_streaming(Smem& sm, const SeqDesc& sd,
                                                 const float* __restrict__ scores,
                                                 int32_t* __restrict__ kept, int tid, int lane,
                                                 int wave) {
    const int64_t dbeg = sd.start + sd.doc_begin;
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const int32_t k = sd.k_doc;
    const int mode = (k == 0) ? 0 : (k == n_doc ? 1 : 2);
    uint32_t thr = 0, rem = 0;
    if (mode == 2) {
        for (int i = tid; i < HTOT; i += ST) sm.hist[i] = 0u;
        __syncthreads();
        uint32_t prefix = 0, mask = 0;
        rem = (uint32_t)k;
#pragma nounroll
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = digit_shift(pass);
            const uint32_t dmask = digit_mask(pass);
            uint32_t* const h = sm.hist + pass * NB;
            for (int32_t i0 = 0; i0 < n_doc; i0 += ST * 4) {
                float f[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) f[u] = scores[dbeg + min(i0 + u * ST + tid, n_doc - 1)];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t kv = score_key(f[u]);
                    if (i0 + u * ST + tid < n_doc && (kv & mask) == prefix)
                        atomicAdd(&h[(kv >> shift) & dmask], 1u);
                }
            }
            __syncthreads();
            pick_bin(sm, pass, 0u, prefix, mask, rem, tid, lane, wave);
        }
        thr = prefix;
    }
    uint32_t carry_above = 0, carry_tied = 0;
    for (int32_t r0 = 0; r0 < sd.len; r0 += NW * 64 * SU) {
        const int32_t wbase = r0 + wave * 64 * SU;
        uint32_t ma_bits = 0, mt_bits = 0, na = 0, nt = 0;
#pragma unroll 4
        for (int u = 0; u < SU; ++u) {
            const int32_t r = wbase + u * 64 + lane;
            const bool in_doc = r >= sd.doc_begin && r < sd.doc_end;
            const uint32_t key =
                mode == 2 ? score_key(scores[dbeg + min(max(r - sd.doc_begin, 0), n_doc - 1)]) : 0u;
            const bool above = r < sd.len && (!in_doc || mode == 1 || (mode == 2 && key > thr));
            const bool tied = in_doc && mode == 2 && key == thr;
            ma_bits |= (uint32_t)above << u;
            mt_bits |= (uint32_t)tied << u;
            na += (uint32_t)__popcll(__ballot(above));
            nt += (uint32_t)__popcll(__ballot(tied));
        }
        place_rows<SU>(sm, sd, kept, wbase, ma_bits, mt_bits, na, nt, rem, carry_above, carry_tied,
                       lane, wave);
    }
}

__global__ __launch_bounds__(ST) void select_kernel(const float* __restrict__ scores, SeqTable t,
                                                    int32_t* __restrict__ kept) {
    __shared__ Smem sm;
    const SeqDesc sd = t.s[blockIdx.x];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave tests stay scalar
    if (sd.len <= ST * 16)
        select_registers<16>(sm, sd, scores, kept, tid, lane, wave);
    else if (sd.len <= ST * 32)
        select_registers<32>(sm, sd, scores, kept, tid, lane, wave);
    else
        select_streaming(sm, sd, scores, kept, tid, lane, wave);
}

}  // namespace

hipError_t launch_select(const float* scores, const SeqTable& t, int32_t* kept, hipStream_t st) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)t.n), dim3(ST), 0, st, scores, t, kept);
    return hipGetLastError();
}

}  // namespace tg
