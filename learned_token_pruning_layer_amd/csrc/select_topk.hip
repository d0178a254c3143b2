// Step 2 - per-prompt top-K selection over document rows, stable by row id.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (a top-K selector keeps the
// best-scored tokens; only the document part of the prompt may be removed,
// the question never); ai4bro.com post, section on how learned token pruning
// works (same rule). The pages do not say how ties break: here the lower row
// id wins, -0 equals +0 and NaN ranks below every number.
//
// One 1024-thread workgroup per prompt of up to 32768 rows.
//  1. Scores map to order-preserving u32 keys (larger key = better rank).
//     Prompts of up to 32768 rows keep every key in registers (WU = 16 or
//     32 per lane) for the whole kernel: HBM is read once (coalesced, then
//     transposed through LDS so that lane l of wave w holds the WU
//     consecutive rows starting at (64w + l) * WU). Rows outside the
//     document hold key 0 and are not counted: while the chosen digits are
//     all zero they fall into bin 0, whose count is corrected by their known
//     number, so the inner loops carry no bounds or document tests. Longer
//     prompts are split into chunks of 16384 rows, one workgroup each, and
//     the per-prompt histograms and chunk counts meet in a workspace (the
//     multi-workgroup kernels at the end of this file).
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

constexpr int RMAX = ST * 32;                // rows of the largest register path
constexpr int STAGE = RMAX + RMAX / 64 + 64;  // padded transpose / staging words + scratch words

struct PickSmem {
    uint32_t hist[HTOT];  // one histogram per pass, cleared once
    uint32_t wtot[NW][2];
    uint32_t pick[3][2];  // per pass: chosen bin, rank inside it
};

struct Smem : PickSmem {
    uint32_t stage[STAGE];  // key transpose, then kept-slot staging
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
__device__ __forceinline__ void pick_bin(PickSmem& sm, int pass, uint32_t excess, uint32_t& prefix,
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

__global__ __launch_bounds__(ST) void select_kernel(const float* __restrict__ scores, SeqTable t,
                                                    int32_t* __restrict__ kept) {
    __shared__ Smem sm;
    const SeqDesc sd = t.s[blockIdx.x];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave tests stay scalar
    static_assert(ST * 32 == SEL_REG_MAX, "register path bound");
    if (sd.len <= ST * 16)
        select_registers<16>(sm, sd, scores, kept, tid, lane, wave);
    else if (sd.len <= ST * 32)
        select_registers<32>(sm, sd, scores, kept, tid, lane, wave);
    // longer prompts: the multi-workgroup kernels below
}

// ---------------------------------------------------------------------------
// Long prompts (more than SEL_REG_MAX rows): the same radix select and
// emission spread over chunks of SEL_CHUNK rows, one 1024-thread workgroup
// per chunk, in six kernels on the stream:
//   zero   clears the per-prompt histograms;
//   hist   (per pass) each chunk of the document builds its histogram of
//          the pass's digit in LDS and adds it into the prompt's histogram;
//   pick   (per pass) one workgroup per prompt finds the bin holding the
//          rem-th largest key and records (prefix, mask, rem);
//   count  each chunk of the prompt counts its "above" and "tied" rows;
//   scan   one workgroup per prompt turns the chunk counts into each
//          chunk's number of above/tied rows before it;
//   place  each chunk ranks its rows (block scan of per-thread counts) and
//          writes its kept row ids, staged in LDS: a chunk's kept rows take
//          a contiguous run of output slots, written out coalesced.
// Workspace, in 32-bit words: hist [n_long][3][NB], state [n_long][4]
// (prefix, mask, rem), counts [n_emit][2], offsets [n_emit][2].
// ---------------------------------------------------------------------------

struct SelWs {
    uint32_t* hist;
    uint32_t* state;
    uint32_t* counts;
    uint32_t* offs;
};

__device__ __forceinline__ SelWs sel_ws(void* base, const LongTable& lt) {
    SelWs w;
    w.hist = (uint32_t*)base;
    w.state = w.hist + (size_t)lt.n * 3 * NB;
    w.counts = w.state + (size_t)lt.n * 4;
    w.offs = w.counts + (size_t)lt.n_emit * 2;
    return w;
}

// Long prompt and chunk of workgroup b, given each prompt's first workgroup.
__device__ __forceinline__ void long_item(const LongTable& lt, int b, bool emit, int& li, int& chunk) {
    li = 0;
    for (int i = 1; i < lt.n; ++i)
        if ((emit ? lt.s[i].emit_base : lt.s[i].hist_base) <= b) li = i;
    chunk = b - (emit ? lt.s[li].emit_base : lt.s[li].hist_base);
}

__global__ __launch_bounds__(256) void sel_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(ST) void sel_hist_kernel(const float* __restrict__ scores, SeqTable t, LongTable lt,
                                                     void* ws_base, int pass) {
    __shared__ uint32_t h[NB];
    int li, chunk;
    long_item(lt, blockIdx.x, false, li, chunk);
    const SeqDesc sd = t.s[lt.s[li].seq];
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    if (!(sd.k_doc > 0 && sd.k_doc < n_doc)) return;  // keep none / all: no threshold needed
    const SelWs ws = sel_ws(ws_base, lt);
    const int tid = threadIdx.x;
    const uint32_t prefix = pass ? ws.state[li * 4 + 0] : 0u, mask = pass ? ws.state[li * 4 + 1] : 0u;
    const int shift = digit_shift(pass);
    const uint32_t dmask = digit_mask(pass);
    h[tid] = 0u;
    h[tid + ST] = 0u;
    __syncthreads();
    const int64_t dbeg = sd.start + sd.doc_begin;
    const int32_t i0 = chunk * SEL_CHUNK;
    float f[SEL_CHUNK / ST];
#pragma unroll
    for (int u = 0; u < SEL_CHUNK / ST; ++u) f[u] = scores[dbeg + min(i0 + u * ST + tid, n_doc - 1)];
#pragma unroll
    for (int u = 0; u < SEL_CHUNK / ST; ++u) {
        const uint32_t key = score_key(f[u]);
        if (i0 + u * ST + tid < n_doc && (key & mask) == prefix) atomicAdd(&h[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    uint32_t* g = ws.hist + ((size_t)li * 3 + pass) * NB;
    for (int b = tid; b < NB; b += ST)
        if (h[b]) atomicAdd(&g[b], h[b]);
}

__global__ __launch_bounds__(ST) void sel_pick_kernel(SeqTable t, LongTable lt, void* ws_base, int pass) {
    __shared__ PickSmem sm;
    const int li = blockIdx.x;
    const SeqDesc sd = t.s[lt.s[li].seq];
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    if (!(sd.k_doc > 0 && sd.k_doc < n_doc)) return;
    const SelWs ws = sel_ws(ws_base, lt);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t prefix = pass ? ws.state[li * 4 + 0] : 0u, mask = pass ? ws.state[li * 4 + 1] : 0u;
    uint32_t rem = pass ? ws.state[li * 4 + 2] : (uint32_t)sd.k_doc;
    const uint32_t* g = ws.hist + ((size_t)li * 3 + pass) * NB;
    for (int b = tid; b <= (int)digit_mask(pass); b += ST) sm.hist[pass * NB + b] = g[b];
    __syncthreads();
    pick_bin(sm, pass, 0u, prefix, mask, rem, tid, lane, wave);
    if (tid == 0) {
        ws.state[li * 4 + 0] = prefix;
        ws.state[li * 4 + 1] = mask;
        ws.state[li * 4 + 2] = rem;
    }
}

// Classification of this thread's SEL_CHUNK/ST consecutive rows of chunk
// `chunk` (rows rbase + u): bit u of *ma (above) / *mt (tied). Keys are read
// coalesced and transposed through LDS (padded, conflict-free).
constexpr int CU_ROWS = SEL_CHUNK / ST;  // rows per thread in a chunk
__device__ __forceinline__ void classify_chunk(const float* __restrict__ scores, const SeqDesc& sd, const SelWs& ws,
                                               int li, int chunk, uint32_t* stage, uint32_t& ma, uint32_t& mt,
                                               uint32_t& rem_out) {
    const int tid = threadIdx.x;
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const int mode = (sd.k_doc == 0) ? 0 : (sd.k_doc == n_doc ? 1 : 2);
    const int32_t cbase = chunk * SEL_CHUNK;  // first row of the chunk (prompt-relative)
    const int32_t rbase = cbase + tid * CU_ROWS;
    uint32_t thr = 0, rem = 0;
    uint32_t key[CU_ROWS];
    if (mode == 2) {
        thr = ws.state[li * 4 + 0];
        rem = ws.state[li * 4 + 2];
        float f[CU_ROWS];
#pragma unroll
        for (int u = 0; u < CU_ROWS; ++u)
            f[u] = scores[sd.start + min(max(cbase + u * ST + tid, sd.doc_begin), sd.doc_end - 1)];
#pragma unroll
        for (int u = 0; u < CU_ROWS; ++u) stage[tpad(u * ST + tid)] = score_key(f[u]);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < CU_ROWS; ++u) key[u] = stage[tpad(tid * CU_ROWS + u)];
    } else {
#pragma unroll
        for (int u = 0; u < CU_ROWS; ++u) key[u] = 0u;
    }
    auto range_bits = [&](int32_t lo, int32_t hi) -> uint32_t {  // rows [lo, hi) of this thread
        const int32_t a = min(max(lo - rbase, 0), CU_ROWS), b = min(max(hi - rbase, 0), CU_ROWS);
        const uint32_t upto_b = b >= 32 ? 0xffffffffu : ((1u << b) - 1u);
        const uint32_t upto_a = a >= 32 ? 0xffffffffu : ((1u << a) - 1u);
        return upto_b & ~upto_a;
    };
    const uint32_t in_len = range_bits(0, sd.len);
    const uint32_t in_doc = range_bits(sd.doc_begin, sd.doc_end);
    if (mode == 2) {
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int u = 0; u < CU_ROWS; ++u) {
            gt |= (key[u] > thr ? 1u : 0u) << u;
            eq |= (key[u] == thr ? 1u : 0u) << u;
        }
        ma = in_len & (~in_doc | gt);
        mt = in_doc & eq;
    } else {
        ma = mode == 1 ? in_len : (in_len & ~in_doc);
        mt = 0u;
    }
    rem_out = rem;
}

// Block-wide exclusive prefix of a per-thread count (wave DPP scans + one
// pass over the wave totals); also returns the block total.
__device__ __forceinline__ uint32_t block_prefix(uint32_t v, uint32_t* wtot, uint32_t& total) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t inc = wave_scan(v);
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    uint32_t before = inc - v, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = wtot[w];
        before += (w < wave) ? x : 0u;
        tot += x;
    }
    total = tot;
    return before;
}

__global__ __launch_bounds__(ST) void sel_count_kernel(const float* __restrict__ scores, SeqTable t, LongTable lt,
                                                      void* ws_base) {
    __shared__ uint32_t stage[SEL_CHUNK + SEL_CHUNK / 64];
    __shared__ uint32_t wtot[2][NW];
    int li, chunk;
    long_item(lt, blockIdx.x, true, li, chunk);
    const SeqDesc sd = t.s[lt.s[li].seq];
    const SelWs ws = sel_ws(ws_base, lt);
    uint32_t ma, mt, rem;
    classify_chunk(scores, sd, ws, li, chunk, stage, ma, mt, rem);
    uint32_t ta, tt;
    block_prefix((uint32_t)__popc(ma), wtot[0], ta);
    block_prefix((uint32_t)__popc(mt), wtot[1], tt);
    if (threadIdx.x == 0) {
        ws.counts[(size_t)(lt.s[li].emit_base + chunk) * 2 + 0] = ta;
        ws.counts[(size_t)(lt.s[li].emit_base + chunk) * 2 + 1] = tt;
    }
}

__global__ __launch_bounds__(ST) void sel_scan_kernel(LongTable lt, void* ws_base) {
    __shared__ uint32_t wtot[2][NW];
    const int li = blockIdx.x;
    const SelWs ws = sel_ws(ws_base, lt);
    const int n = lt.s[li].n_emit;
    uint32_t* c = ws.counts + (size_t)lt.s[li].emit_base * 2;
    uint32_t* o = ws.offs + (size_t)lt.s[li].emit_base * 2;
    uint32_t carry_a = 0, carry_t = 0;
    for (int i0 = 0; i0 < n; i0 += ST) {
        const int i = i0 + (int)threadIdx.x;
        const uint32_t a = i < n ? c[i * 2 + 0] : 0u, b = i < n ? c[i * 2 + 1] : 0u;
        uint32_t ta, tb;
        const uint32_t pa = block_prefix(a, wtot[0], ta), pb = block_prefix(b, wtot[1], tb);
        if (i < n) {
            o[i * 2 + 0] = carry_a + pa;
            o[i * 2 + 1] = carry_t + pb;
        }
        carry_a += ta;
        carry_t += tb;
        __syncthreads();  // wtot is rewritten by the next block
    }
}

__global__ __launch_bounds__(ST) void sel_place_kernel(const float* __restrict__ scores, SeqTable t, LongTable lt,
                                                      void* ws_base, int32_t* __restrict__ kept) {
    // The key transpose is dead once block_prefix has synchronised; it then
    // stages the chunk's kept row ids by slot, plus one scratch word per lane.
    __shared__ uint32_t stage[SEL_CHUNK + SEL_CHUNK / 64];
    static_assert(SEL_CHUNK / 64 >= 64, "scratch words fit the transpose padding");
    __shared__ uint32_t wtot[2][NW];
    int li, chunk;
    long_item(lt, blockIdx.x, true, li, chunk);
    const SeqDesc sd = t.s[lt.s[li].seq];
    const SelWs ws = sel_ws(ws_base, lt);
    uint32_t ma, mt, rem;
    classify_chunk(scores, sd, ws, li, chunk, stage, ma, mt, rem);
    uint32_t* const slots = stage;
    const size_t ci = (size_t)(lt.s[li].emit_base + chunk) * 2;
    const uint32_t oa = ws.offs[ci + 0], ot = ws.offs[ci + 1];  // above / tied rows before the chunk
    const uint32_t ca = ws.counts[ci + 0], ct = ws.counts[ci + 1];
    const uint32_t first = oa + min(ot, rem);                 // the chunk's first output slot
    const uint32_t n_out = oa + ca + min(ot + ct, rem) - first;  // and how many slots it fills
    uint32_t tot;
    uint32_t pa = oa + block_prefix((uint32_t)__popc(ma), wtot[0], tot);
    uint32_t pt = ot + block_prefix((uint32_t)__popc(mt), wtot[1], tot);
    const int tid = threadIdx.x;
    const int32_t rbase = chunk * SEL_CHUNK + tid * CU_ROWS;
    const int trash = SEL_CHUNK + (tid & 63);
#pragma unroll
    for (int u = 0; u < CU_ROWS; ++u) {
        const uint32_t above = (ma >> u) & 1u, tied = (mt >> u) & 1u;
        const uint32_t slot = pa + min(pt, rem);
        const uint32_t keep = above | (tied & (uint32_t)(pt < rem));
        // slot - first < n_out always holds for a kept row when the counts are right
        const bool ok = keep && slot - first < n_out;
        slots[ok ? (int)(slot - first) : trash] = (uint32_t)(sd.start + rbase + u);
        pa += above;
        pt += tied;
    }
    __syncthreads();
    for (uint32_t j = tid; j < n_out; j += ST) kept[sd.kept_off + first + j] = (int32_t)slots[j];
}

}  // namespace

size_t select_plan(const SeqTable& t, LongTable* lt) {
    *lt = LongTable{};
    for (int b = 0; b < t.n; ++b) {
        const SeqDesc& d = t.s[b];
        if (d.len <= SEL_REG_MAX) continue;
        LongSeq& l = lt->s[lt->n++];
        l.seq = b;
        const int32_t n_doc = d.doc_end - d.doc_begin;
        l.hist_base = lt->n_hist;
        l.n_hist = (n_doc + SEL_CHUNK - 1) / SEL_CHUNK;
        l.emit_base = lt->n_emit;
        l.n_emit = (d.len + SEL_CHUNK - 1) / SEL_CHUNK;
        lt->n_hist += l.n_hist;
        lt->n_emit += l.n_emit;
    }
    if (lt->n == 0) return 0;
    return ((size_t)lt->n * (3 * NB + 4) + (size_t)lt->n_emit * 4) * sizeof(uint32_t);
}

hipError_t launch_select(const float* scores, const SeqTable& t, const LongTable& lt, void* workspace,
                         int32_t* kept, hipStream_t st) {
    bool any_short = false;
    for (int b = 0; b < t.n; ++b) any_short |= t.s[b].len > 0 && t.s[b].len <= SEL_REG_MAX;
    if (any_short) hipLaunchKernelGGL(select_kernel, dim3((unsigned)t.n), dim3(ST), 0, st, scores, t, kept);
    if (lt.n == 0) return hipGetLastError();
    hipLaunchKernelGGL(sel_zero_kernel, dim3((unsigned)lt.n * 6), dim3(256), 0, st, (uint32_t*)workspace,
                       (int64_t)lt.n * 3 * NB);
    for (int pass = 0; pass < 3; ++pass) {
        if (lt.n_hist)
            hipLaunchKernelGGL(sel_hist_kernel, dim3((unsigned)lt.n_hist), dim3(ST), 0, st, scores, t, lt, workspace, pass);
        hipLaunchKernelGGL(sel_pick_kernel, dim3((unsigned)lt.n), dim3(ST), 0, st, t, lt, workspace, pass);
    }
    hipLaunchKernelGGL(sel_count_kernel, dim3((unsigned)lt.n_emit), dim3(ST), 0, st, scores, t, lt, workspace);
    hipLaunchKernelGGL(sel_scan_kernel, dim3((unsigned)lt.n), dim3(ST), 0, st, lt, workspace);
    hipLaunchKernelGGL(sel_place_kernel, dim3((unsigned)lt.n_emit), dim3(ST), 0, st, scores, t, lt, workspace, kept);
    return hipGetLastError();
}

}  // namespace tg
