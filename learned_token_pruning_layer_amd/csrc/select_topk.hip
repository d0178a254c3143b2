// Step 2 - per-prompt top-K selection over document rows, stable by row id.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (a top-K selector keeps the
// best-scored tokens; only the document part of the prompt may be removed,
// the question never); ai4bro.com post, section on how learned token pruning
// works (same rule). The pages do not say how ties break: here the lower row
// id wins, -0 equals +0 and NaN ranks below every number.
//
// Prompts of up to 32768 rows: 16 workgroups of 1024 threads per prompt,
// each of which finds the threshold on its own and writes one sixteenth of
// the rows.
//  1. Scores map to order-preserving u32 keys (larger key = better rank).
//     Every workgroup of the prompt keeps every key in registers (WU = 16
//     or 32 per lane, read coalesced: wave w, register u, lane l holds row
//     64*WU*w + 64u + l). Rows outside the document hold key 0 and are not
//     counted: while the chosen digits are all zero they fall into bin 0,
//     whose count is corrected by their known number, so the inner loops
//     carry no bounds or document tests. Longer prompts are split into
//     chunks of 16384 rows, one workgroup each, and the per-prompt
//     histograms, the chunks' candidate keys and their counts meet in a
//     workspace (the multi-workgroup kernels at the end of this file).
//  2. A 3-pass MSB radix select (11, 11 and 10-bit digits; LDS histograms
//     with integer atomics; a DPP wave scan over the bins from the top)
//     finds the k-th largest key T and rem = how many keys equal to T are
//     kept. Pass 0 counts each key as its load returns. The steps are
//     integer and see the same keys in every workgroup of the prompt, so
//     all of them reach the same T and rem; none reads another's results.
//     A pass whose chosen bin is kept whole ends the search early (T is
//     then the key just below the bin and rem is 0).
//  3. Emission: a row is "above" (outside the document, or key > T) or
//     "tied" (document key == T). Kept rows are the above rows and the
//     first rem tied rows; a kept row's output slot is (#above before it) +
//     min(#tied before it, rem), so rows land in ascending order without a
//     sort. Workgroup g writes slice g, the 64*WU consecutive rows held by
//     its wave g: every wave's above / tied totals (DPP scans) and wave
//     g's per-lane row masks meet in LDS, and each wave ranks 64 (or 2 x
//     64) of the slice's rows with ballots + mbcnt, from the totals of the
//     slices before g and of the slice's earlier rows.
//     Chunked path: the same ranking per chunk, kept row ids staged in LDS
//     by slot and written out coalesced.
// Replicating the threshold search costs 16 reads of the prompt's scores
// (from L2) instead of the one-workgroup emission's many dependent steps,
// whose instruction count on a single CU set that kernel's time.
// Integer work only: the result is bit-exact and deterministic.
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

constexpr int ST = 1024;               // threads per workgroup (16 waves)
constexpr int NW = ST / 64;
constexpr int NB = 2048;               // histogram bins (11-bit digits)
constexpr int HTOT = 2 * NB + NB / 2;  // the three passes' histograms (11, 11 and 10 bits)

struct PickSmem {
    uint32_t hist[HTOT];  // one histogram per pass, cleared once
    uint32_t wtot[NW][1];  // per-wave bin totals of the current bin search
};

struct RegSmem : PickSmem {
    uint32_t ctot[NW][2];  // per-wave above / tied totals
    uint32_t em[64][2];    // the written slice's per-lane above / tied masks
};

// Padded LDS index of row r in a chunk's key transpose: one spare word per
// 64 rows spreads both the row-order writes and the lane-contiguous reads
// (stride 16 words) over all 64 banks.
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
// Lane slot i (thread i, or lane l of the chosen wave range) covers bins
// dmask - 2i and dmask - 2i - 1. One barrier: each wave publishes its
// range's total, then every wave finds the range holding the rem-th key
// from the totals, re-reads that range's bins and finds the bin itself, so
// all waves reach the same result with no broadcast. sm.wtot is free again
// once every wave has passed the caller's next barrier. Returns the chosen
// bin's count.
__device__ __forceinline__ uint32_t pick_bin(PickSmem& sm, int pass, uint32_t excess, uint32_t& prefix,
                                             uint32_t& mask, uint32_t& rem, int tid, int lane, int wave) {
    const int shift = digit_shift(pass);
    const uint32_t dmask = digit_mask(pass);
    const uint32_t* h = sm.hist + pass * NB;
    auto bins = [&](int i, uint32_t& c0, uint32_t& c1) {
        const int b0 = (int)dmask - 2 * i, b1 = b0 - 1;
        c0 = b0 >= 0 ? h[b0] : 0u;
        c1 = b1 >= 0 ? h[b1] : 0u;
        if (b0 == 0) c0 -= excess;
        if (b1 == 0) c1 -= excess;
    };
    uint32_t c0, c1;
    bins(tid, c0, c1);
    const uint32_t inc = wave_scan(c0 + c1);
    if (lane == 63) sm.wtot[wave][0] = inc;
    __syncthreads();
    // The wave range W holding the rem-th key (rem >= 1 keys are counted).
    const uint32_t wt = lane < NW ? sm.wtot[lane][0] : 0u;
    const uint32_t winc = wave_scan(wt);
    const uint64_t wb = __ballot(lane < NW && winc >= rem);
    const int W = wb ? (int)__builtin_ctzll(wb) : NW - 1;
    const uint32_t wbefore = (uint32_t)__builtin_amdgcn_readlane((int)(winc - wt), W);
    // ... and the lane slot inside it.
    uint32_t d0, d1;
    bins(64 * W + lane, d0, d1);
    const uint32_t dinc = wave_scan(d0 + d1);
    const uint64_t lb = __ballot(wbefore + dinc >= rem);
    const int L = lb ? (int)__builtin_ctzll(lb) : 63;
    const uint32_t before = wbefore + (uint32_t)__builtin_amdgcn_readlane((int)(dinc - d0 - d1), L);
    const uint32_t d0l = (uint32_t)__builtin_amdgcn_readlane((int)d0, L);
    const uint32_t d1l = (uint32_t)__builtin_amdgcn_readlane((int)d1, L);
    const uint32_t top = dmask - 2u * (uint32_t)(64 * W + L);
    const bool first = rem <= before + d0l;
    prefix |= (first ? top : top - 1u) << shift;
    mask |= dmask << shift;
    rem = first ? rem - before : rem - before - d0l;
    return first ? d0l : d1l;
}

// Prompts of at most NW*64*WU rows: every key in registers. Wave w holds
// rows 64*WU*w + 64u + lane (register u), so the rows split into NW slices
// of 64*WU consecutive rows, slice w being exactly wave w's rows. Each of
// the prompt's NW workgroups finds the threshold from every key on its own
// (the same integer steps on the same keys, so every workgroup reaches the
// same T and rem) and writes the kept rows of slice g = its index within
// the prompt; no workgroup waits for or reads from another.
template <int WU>  // WU <= 32
__device__ __forceinline__ void select_registers(RegSmem& sm, const SeqDesc& sd, int g,
                                                 const float* __restrict__ scores,
                                                 int32_t* __restrict__ kept, int tid, int lane,
                                                 int wave) {
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const int32_t k = sd.k_doc;
    const int mode = (k == 0) ? 0 : (k == n_doc ? 1 : 2);  // keep no / all / top-k document rows
    const int32_t wbase = wave * 64 * WU;
    uint32_t key[WU];
    uint32_t thr = 0, rem = 0;
    if (mode == 2) {
        for (int i = tid; i < HTOT; i += ST) sm.hist[i] = 0u;
        float f[WU];
#pragma unroll
        for (int u = 0; u < WU; ++u) {  // clamped into the document: every load is valid
            const int32_t r = wbase + u * 64 + lane;
            f[u] = scores[sd.start + min(max(r, sd.doc_begin), sd.doc_end - 1)];
        }
        // The histograms are clear once every wave passes this barrier; it
        // does not wait for the score loads, which are still in flight.
        ring_barrier();
        // Pass 0 counts every key as its load returns.
#pragma unroll
        for (int u = 0; u < WU; ++u) {
            const int32_t r = wbase + u * 64 + lane;
            key[u] = (r >= sd.doc_begin && r < sd.doc_end) ? score_key(f[u]) : 0u;
            atomicAdd(&sm.hist[key[u] >> 21], 1u);
        }
        __syncthreads();  // pass 0's histogram complete
        // Rows of the register range that are not document rows (key 0).
        const uint32_t npad = (uint32_t)(NW * 64 * WU - n_doc);
        uint32_t prefix = 0, mask = 0;
        rem = (uint32_t)k;
        uint32_t cnt = pick_bin(sm, 0, npad, prefix, mask, rem, tid, lane, wave);
        // When the chosen bin holds exactly rem keys, all of them are kept:
        // the threshold is then the key just below the bin (prefix - 1, the
        // lower digits zero), with no tied row kept, and the later passes
        // are skipped. (A bin with prefix 0 would need T = -1, so it always
        // takes the full passes.) The test is uniform over the workgroup.
        int pass = 1;
#pragma nounroll
        for (; pass < 3 && !(cnt == rem && prefix != 0u); ++pass) {
            const int shift = digit_shift(pass);
            const uint32_t dmask = digit_mask(pass);
            uint32_t* const h = sm.hist + pass * NB;
#pragma unroll
            for (int u = 0; u < WU; ++u)
                if ((key[u] & mask) == prefix) atomicAdd(&h[(key[u] >> shift) & dmask], 1u);
            __syncthreads();
            cnt = pick_bin(sm, pass, prefix == 0 ? npad : 0u, prefix, mask, rem, tid, lane, wave);
        }
        if (pass < 3) {
            thr = prefix - 1u;
            rem = 0u;
        } else {
            thr = prefix;
        }
    } else {
#pragma unroll
        for (int u = 0; u < WU; ++u) key[u] = 0u;
    }

    // A row is "above" (inside the prompt and outside the document, or a
    // document key > T; every document row when all are kept) or "tied" (a
    // document key == T). Kept: the above rows and the first rem tied rows
    // in row order; a kept row's slot is (#above before it) + min(#tied
    // before it, rem).
    // Bit u of the lane's masks describes its row wbase + 64u + lane. The
    // prompt and the document are row ranges, so for each lane they are
    // ranges of u; only the key comparisons are per row.
    auto u_bound = [&](int32_t row) -> int {  // first u whose row is >= row
        return min(max((row - wbase - lane + 63) >> 6, 0), WU);
    };
    auto bits_below = [](int b) -> uint32_t { return b >= 32 ? 0xffffffffu : ((1u << b) - 1u); };
    const uint32_t in_len = bits_below(u_bound(sd.len));
    const uint32_t in_doc = bits_below(u_bound(sd.doc_end)) & ~bits_below(u_bound(sd.doc_begin));
    uint32_t ma_bits, mt_bits;  // above / tied
    if (mode == 2) {
        uint32_t gt_bits = 0u, eq_bits = 0u;
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
    // Every wave's above / tied totals; wave g also leaves its masks for the
    // workgroup, which ranks slice g's rows 64 per wave.
    const uint32_t ia = wave_scan((uint32_t)__popc(ma_bits)), it = wave_scan((uint32_t)__popc(mt_bits));
    if (lane == 63) {
        sm.ctot[wave][0] = ia;
        sm.ctot[wave][1] = it;
    }
    if (wave == g) {
        sm.em[lane][0] = ma_bits;
        sm.em[lane][1] = mt_bits;
    }
    __syncthreads();
    uint32_t pa = 0, pt = 0;  // above / tied rows of the slices before g
    for (int w = 0; w < g; ++w) {
        pa += sm.ctot[w][0];
        pt += sm.ctot[w][1];
    }
    const uint32_t ea = sm.em[lane][0], et = sm.em[lane][1];
    const uint32_t n_kept = (uint32_t)sd.n_kept;
    const int32_t sbase = g * 64 * WU;  // slice g's first row
#pragma unroll
    for (int j = 0; j < WU / NW; ++j) {
        const int u = wave + NW * j;  // this wave ranks the slice's rows 64u .. 64u + 63
        // rows of the slice before row 64u: the bits below u, over all lanes
        const uint32_t lo = bits_below(u);
        const uint32_t sa = wave_scan((uint32_t)__popc(ea & lo)), sti = wave_scan((uint32_t)__popc(et & lo));
        const uint32_t ua = pa + (uint32_t)__builtin_amdgcn_readlane((int)sa, 63);
        const uint32_t ut = pt + (uint32_t)__builtin_amdgcn_readlane((int)sti, 63);
        const bool above = (ea >> u) & 1u, tied = (et >> u) & 1u;
        const uint64_t ba = __ballot(above), bt = __ballot(tied);
        const uint32_t la = __builtin_amdgcn_mbcnt_hi((uint32_t)(ba >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ba, 0u));
        const uint32_t lt = __builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
        const uint32_t tr = ut + lt;  // tied rows before this one
        const uint32_t slot = ua + la + min(tr, rem);
        // slot < n_kept always holds for a kept row when the counts are right
        if ((above || (tied && tr < rem)) && slot < n_kept)
            kept[sd.kept_off + slot] = (int32_t)(sd.start + sbase + u * 64 + lane);
    }
}

// Grid: NW workgroups per prompt (prompt b = blockIdx / NW, slice g =
// blockIdx % NW). Slices past the prompt's end have nothing to write and
// exit at once; prompts above SEL_REG_MAX rows take the kernels below.
__global__ __launch_bounds__(ST) void select_kernel(const float* __restrict__ scores, SeqTable t,
                                                    int32_t* __restrict__ kept) {
    __shared__ RegSmem sm;
    const SeqDesc sd = t.s[blockIdx.x / NW];
    const int g = (int)(blockIdx.x % NW);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave tests stay scalar
    static_assert(ST * 32 == SEL_REG_MAX, "register path bound");
    if (sd.len <= ST * 16) {
        if (g * 64 * 16 < sd.len) select_registers<16>(sm, sd, g, scores, kept, tid, lane, wave);
    } else if (sd.len <= ST * 32) {
        if (g * 64 * 32 < sd.len) select_registers<32>(sm, sd, g, scores, kept, tid, lane, wave);
    }
}

// ---------------------------------------------------------------------------
// Long prompts (more than SEL_REG_MAX rows): the same radix select and
// emission spread over chunks of SEL_CHUNK rows, one 1024-thread workgroup
// per chunk, in six kernels on the stream, three of which read the scores:
//   zero   clears the per-prompt histograms;
//   hist   each chunk of the document builds its histogram of the first
//          (top 11-bit) digit in LDS and adds it into the prompt's
//          histogram (read 1);
//   cand   each chunk of the prompt finds the first digit's bin (the one
//          holding the k-th largest key) from the finished histogram, counts
//          its rows that are kept whatever the rest of the threshold is
//          (rows outside the document, keys in higher bins), copies the keys
//          inside the bin to its own candidate list in the workspace, and
//          adds their second digits into the prompt's second histogram
//          (read 2);
//   cand_hist  each chunk finds the second digit's bin and adds the third
//          digits of its matching candidates into the third histogram;
//   count  each chunk finds the threshold key T and how many keys equal to
//          T are kept, and counts its "above" rows (the rows counted by cand
//          plus its candidates above T) and "tied" rows (candidates equal
//          to T) from its candidate list;
//   place  each chunk adds up the counts of the chunks before it, ranks
//          its rows (block scan of per-thread counts) and writes its kept
//          row ids, staged in LDS: a chunk's kept rows take a contiguous
//          run of output slots, written out coalesced (read 3).
// Each bin search is repeated in every workgroup of the kernel that needs
// it rather than run by a kernel of its own (one launch less per pass); the
// prompt's first chunk records (prefix, mask, rem) for the later kernels.
// Workspace, in 32-bit words: hist [n_long][3][NB], state [n_long][3][4]
// ((prefix, mask, rem) after each pass), counts [n_emit][2] (above, tied),
// ccnt [n_emit][2] (candidates, rows kept by the first digit alone),
// cand [n_emit][SEL_CHUNK] (candidate keys, in no particular order).
// ---------------------------------------------------------------------------

struct SelWs {
    uint32_t* hist;
    uint32_t* state;
    uint32_t* counts;
    uint32_t* ccnt;
    uint32_t* cand;
};

__device__ __forceinline__ SelWs sel_ws(void* base, const LongTable& lt) {
    SelWs w;
    w.hist = (uint32_t*)base;
    w.state = w.hist + (size_t)lt.n * 3 * NB;
    w.counts = w.state + (size_t)lt.n * 12;
    w.ccnt = w.counts + (size_t)lt.n_emit * 2;
    w.cand = w.ccnt + (size_t)lt.n_emit * 2;
    return w;
}

// (prefix, mask, rem) after pass `pass` of long prompt li: this workgroup
// redoes the bin search over the pass's completed histogram, starting from
// the state the previous pass left (pass 0 starts from (0, 0, k)). The
// first chunk's workgroup (`store`) records the result for later kernels.
__device__ __forceinline__ void pick_after(PickSmem& sm, const SelWs& ws, int li, int pass, uint32_t k_doc,
                                           bool store, uint32_t& prefix, uint32_t& mask, uint32_t& rem, int tid,
                                           int lane, int wave) {
    if (pass == 0) {
        prefix = 0u;
        mask = 0u;
        rem = k_doc;
    } else {
        const uint32_t* st = ws.state + (size_t)(li * 3 + pass - 1) * 4;
        prefix = st[0];
        mask = st[1];
        rem = st[2];
    }
    const uint32_t* g = ws.hist + ((size_t)li * 3 + pass) * NB;
    for (int b = tid; b <= (int)digit_mask(pass); b += ST) sm.hist[pass * NB + b] = g[b];
    __syncthreads();
    pick_bin(sm, pass, 0u, prefix, mask, rem, tid, lane, wave);
    if (store && tid == 0) {
        uint32_t* st = ws.state + (size_t)(li * 3 + pass) * 4;
        st[0] = prefix;
        st[1] = mask;
        st[2] = rem;
    }
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
                                                     void* ws_base) {
    constexpr int pass = 0;
    __shared__ uint32_t h[NB];
    int li, chunk;
    long_item(lt, blockIdx.x, false, li, chunk);
    const SeqDesc sd = t.s[lt.s[li].seq];
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    if (!(sd.k_doc > 0 && sd.k_doc < n_doc)) return;  // keep none / all: no threshold needed
    const SelWs ws = sel_ws(ws_base, lt);
    const int tid = threadIdx.x;
    const int64_t dbeg = sd.start + sd.doc_begin;
    const int32_t i0 = chunk * SEL_CHUNK;
    float f[SEL_CHUNK / ST];
#pragma unroll
    for (int u = 0; u < SEL_CHUNK / ST; ++u) f[u] = scores[dbeg + min(i0 + u * ST + tid, n_doc - 1)];
    h[tid] = 0u;
    h[tid + ST] = 0u;
    const int shift = digit_shift(pass);
    const uint32_t dmask = digit_mask(pass);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < SEL_CHUNK / ST; ++u) {
        const uint32_t key = score_key(f[u]);
        if (i0 + u * ST + tid < n_doc) atomicAdd(&h[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    uint32_t* g = ws.hist + ((size_t)li * 3 + pass) * NB;
    for (int b = tid; b < NB; b += ST)
        if (h[b]) atomicAdd(&g[b], h[b]);
}

// Classification of this thread's SEL_CHUNK/ST consecutive rows of chunk
// `chunk` (rows rbase + u): bit u of *ma (above) / *mt (tied). Keys are read
// coalesced and transposed through LDS (padded, conflict-free).
constexpr int CU_ROWS = SEL_CHUNK / ST;  // rows per thread in a chunk
__device__ __forceinline__ void classify_chunk(const float* __restrict__ scores, const SeqDesc& sd, uint32_t thr,
                                               int chunk, uint32_t* stage, uint32_t& ma, uint32_t& mt) {
    const int tid = threadIdx.x;
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const int mode = (sd.k_doc == 0) ? 0 : (sd.k_doc == n_doc ? 1 : 2);
    const int32_t cbase = chunk * SEL_CHUNK;  // first row of the chunk (prompt-relative)
    const int32_t rbase = cbase + tid * CU_ROWS;
    uint32_t key[CU_ROWS];
    if (mode == 2) {
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

// Rows of the chunk kept whatever the threshold's lower digits are, and the
// keys of the first digit's bin, copied to the chunk's candidate list; their
// second digits go into the prompt's second histogram.
__global__ __launch_bounds__(ST) void sel_cand_kernel(const float* __restrict__ scores, SeqTable t, LongTable lt,
                                                     void* ws_base) {
    __shared__ PickSmem sm;
    __shared__ uint32_t h[NB];
    __shared__ uint32_t wtot[NW];
    __shared__ uint32_t n_cand;
    int li, chunk;
    long_item(lt, blockIdx.x, true, li, chunk);
    const SeqDesc sd = t.s[lt.s[li].seq];
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    if (!(sd.k_doc > 0 && sd.k_doc < n_doc)) return;  // keep none / all: counted from the ranges alone
    const SelWs ws = sel_ws(ws_base, lt);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t cbase = chunk * SEL_CHUNK;  // first row of the chunk (prompt-relative)
    float f[CU_ROWS];
#pragma unroll
    for (int u = 0; u < CU_ROWS; ++u)  // clamped into the document: every load is valid
        f[u] = scores[sd.start + min(max(cbase + u * ST + tid, sd.doc_begin), sd.doc_end - 1)];
    h[tid] = 0u;
    h[tid + ST] = 0u;
    if (tid == 0) n_cand = 0u;
    uint32_t prefix, mask, rem;
    pick_after(sm, ws, li, 0, (uint32_t)sd.k_doc, chunk == 0, prefix, mask, rem, tid, lane, wave);
    (void)rem;
    const uint32_t top = prefix | ~mask;  // largest key of the chosen bin
    uint32_t* const cand = ws.cand + (size_t)(lt.s[li].emit_base + chunk) * SEL_CHUNK;
    uint32_t above = 0u;
#pragma unroll
    for (int u = 0; u < CU_ROWS; ++u) {
        const int32_t r = cbase + u * ST + tid;
        const bool in_doc = r >= sd.doc_begin && r < sd.doc_end;
        const uint32_t key = score_key(f[u]);
        if (r < sd.len && (!in_doc || key > top)) {
            ++above;
        } else if (in_doc && (key & mask) == prefix) {
            atomicAdd(&h[(key >> digit_shift(1)) & digit_mask(1)], 1u);
            cand[atomicAdd(&n_cand, 1u)] = key;
        }
    }
    uint32_t total_above;
    block_prefix(above, wtot, total_above);  // its barrier also completes h and n_cand
    uint32_t* g = ws.hist + ((size_t)li * 3 + 1) * NB;
    for (int b = tid; b < NB; b += ST)
        if (h[b]) atomicAdd(&g[b], h[b]);
    if (tid == 0) {
        ws.ccnt[(size_t)(lt.s[li].emit_base + chunk) * 2 + 0] = n_cand;
        ws.ccnt[(size_t)(lt.s[li].emit_base + chunk) * 2 + 1] = total_above;
    }
}

// The third digits of the candidates that match the second digit's bin.
__global__ __launch_bounds__(ST) void sel_cand_hist_kernel(SeqTable t, LongTable lt, void* ws_base) {
    __shared__ PickSmem sm;
    __shared__ uint32_t h[NB];
    int li, chunk;
    long_item(lt, blockIdx.x, true, li, chunk);
    const SeqDesc sd = t.s[lt.s[li].seq];
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    if (!(sd.k_doc > 0 && sd.k_doc < n_doc)) return;
    const SelWs ws = sel_ws(ws_base, lt);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    h[tid] = 0u;
    h[tid + ST] = 0u;
    uint32_t prefix, mask, rem;
    pick_after(sm, ws, li, 1, (uint32_t)sd.k_doc, chunk == 0, prefix, mask, rem, tid, lane, wave);
    (void)rem;
    const size_t ci = (size_t)(lt.s[li].emit_base + chunk);
    const uint32_t n = ws.ccnt[ci * 2];
    const uint32_t* const cand = ws.cand + ci * SEL_CHUNK;
    for (uint32_t i = tid; i < n; i += ST) {
        const uint32_t key = cand[i];
        if ((key & mask) == prefix) atomicAdd(&h[(key >> digit_shift(2)) & digit_mask(2)], 1u);
    }
    __syncthreads();
    uint32_t* g = ws.hist + ((size_t)li * 3 + 2) * NB;
    for (int b = tid; b <= (int)digit_mask(2); b += ST)
        if (h[b]) atomicAdd(&g[b], h[b]);
}

__global__ __launch_bounds__(ST) void sel_count_kernel(const float* __restrict__ scores, SeqTable t, LongTable lt,
                                                      void* ws_base) {
    __shared__ PickSmem sm;
    __shared__ uint32_t stage[SEL_CHUNK + SEL_CHUNK / 64];
    __shared__ uint32_t wtot[2][NW];
    int li, chunk;
    long_item(lt, blockIdx.x, true, li, chunk);
    const SeqDesc sd = t.s[lt.s[li].seq];
    const SelWs ws = sel_ws(ws_base, lt);
    const int tid = threadIdx.x;
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    uint32_t ta, tt;
    if (sd.k_doc > 0 && sd.k_doc < n_doc) {
        // Above: the rows the first digit already keeps plus the candidates
        // above T; tied: the candidates equal to T.
        uint32_t thr, mask, rem;
        pick_after(sm, ws, li, 2, (uint32_t)sd.k_doc, chunk == 0, thr, mask, rem, tid, tid & 63,
                   __builtin_amdgcn_readfirstlane(tid >> 6));
        const size_t ci = (size_t)(lt.s[li].emit_base + chunk);
        const uint32_t n = ws.ccnt[ci * 2];
        const uint32_t* const cand = ws.cand + ci * SEL_CHUNK;
        uint32_t gt = 0u, eq = 0u;
        for (uint32_t i = tid; i < n; i += ST) {
            const uint32_t key = cand[i];
            gt += key > thr ? 1u : 0u;
            eq += key == thr ? 1u : 0u;
        }
        block_prefix(gt, wtot[0], ta);
        block_prefix(eq, wtot[1], tt);
        ta += ws.ccnt[ci * 2 + 1];
    } else {
        uint32_t ma, mt;
        classify_chunk(scores, sd, 0u, chunk, stage, ma, mt);  // no keys read: the ranges decide
        block_prefix((uint32_t)__popc(ma), wtot[0], ta);
        block_prefix((uint32_t)__popc(mt), wtot[1], tt);
    }
    if (tid == 0) {
        ws.counts[(size_t)(lt.s[li].emit_base + chunk) * 2 + 0] = ta;
        ws.counts[(size_t)(lt.s[li].emit_base + chunk) * 2 + 1] = tt;
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
    const int32_t n_doc = sd.doc_end - sd.doc_begin;
    const bool radix = sd.k_doc > 0 && sd.k_doc < n_doc;
    const uint32_t thr = radix ? ws.state[(size_t)(li * 3 + 2) * 4 + 0] : 0u;
    const uint32_t rem = radix ? ws.state[(size_t)(li * 3 + 2) * 4 + 2] : 0u;
    // Above / tied rows of the chunks before this one: their counts from
    // the count kernel, added up here.
    const uint32_t* cnt = ws.counts + (size_t)lt.s[li].emit_base * 2;
    uint32_t ba = 0u, bt = 0u;
    for (int j = threadIdx.x; j < chunk; j += ST) {
        ba += cnt[j * 2 + 0];
        bt += cnt[j * 2 + 1];
    }
    uint32_t oa, ot;
    block_prefix(ba, wtot[0], oa);
    block_prefix(bt, wtot[1], ot);
    __syncthreads();  // wtot is rewritten by the ranking below
    uint32_t ma, mt;
    classify_chunk(scores, sd, thr, chunk, stage, ma, mt);
    uint32_t* const slots = stage;
    const size_t ci = (size_t)(lt.s[li].emit_base + chunk) * 2;
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
    return ((size_t)lt->n * (3 * NB + 12) + (size_t)lt->n_emit * (4 + SEL_CHUNK)) * sizeof(uint32_t);
}

hipError_t launch_select(const float* scores, const SeqTable& t, const LongTable& lt, void* workspace,
                         int32_t* kept, hipStream_t st) {
    bool any_short = false;
    for (int b = 0; b < t.n; ++b) any_short |= t.s[b].len > 0 && t.s[b].len <= SEL_REG_MAX;
    if (any_short) hipLaunchKernelGGL(select_kernel, dim3((unsigned)t.n * NW), dim3(ST), 0, st, scores, t, kept);
    if (lt.n == 0) return hipGetLastError();
    hipLaunchKernelGGL(sel_zero_kernel, dim3((unsigned)lt.n * 6), dim3(256), 0, st, (uint32_t*)workspace,
                       (int64_t)lt.n * 3 * NB);
    if (lt.n_hist)
        hipLaunchKernelGGL(sel_hist_kernel, dim3((unsigned)lt.n_hist), dim3(ST), 0, st, scores, t, lt, workspace);
    hipLaunchKernelGGL(sel_cand_kernel, dim3((unsigned)lt.n_emit), dim3(ST), 0, st, scores, t, lt, workspace);
    hipLaunchKernelGGL(sel_cand_hist_kernel, dim3((unsigned)lt.n_emit), dim3(ST), 0, st, t, lt, workspace);
    hipLaunchKernelGGL(sel_count_kernel, dim3((unsigned)lt.n_emit), dim3(ST), 0, st, scores, t, lt, workspace);
    hipLaunchKernelGGL(sel_place_kernel, dim3((unsigned)lt.n_emit), dim3(ST), 0, st, scores, t, lt, workspace, kept);
    return hipGetLastError();
}

}  // namespace tg
