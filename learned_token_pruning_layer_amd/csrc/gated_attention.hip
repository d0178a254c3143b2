// Step 4 - token-gated causal attention over the kept rows.
//
// Defined by the TokenGate pages: spke.com article, section "Was ist
// token-gated Attention?" (the score of each kept token becomes a bias on
// the attention logits of the layers above the gate, with a learnable gain
// per head and a learnable temperature) and section "Wie wird TokenGate
// implementiert?" (the kernel is a key-bias attention). The bias form used
// on both sides: for kept rows i, j of one prompt and query head h,
//     logit_ij = q_i.k_j / (sqrt(D) tau) + gain[h] * bias[j],  pos_j <= pos_i.
//
// bf16 path (flash-attention style, online softmax, v_mfma_f32_32x32x16_bf16):
//  * Each wave owns 32 query rows of one query head. A workgroup holds the
//    query heads of one KV head that share its K/V (GQA; 2 when Hq/Hkv is
//    even), times query slabs, times key splits; three shapes (see
//    launch_cfg): short prompts take 32 rows x 2 key splits, long prompts 2
//    slabs of 32 rows sharing every K/V tile with one split, and the longest
//    the same at three workgroups per CU.
//  * S^T = K Q^T: K (keys x d) is the A operand read from LDS, Q^T the B
//    operand kept in registers for the whole key loop. The 32x32 result
//    layout puts one query column in each lane (keys down its registers),
//    so the softmax row statistics are per lane, with one exchange between
//    lanes l and l^32.
//  * O^T += V^T P^T: the lane's own S^T registers, rounded to bf16, are
//    exactly the B operand once keys are taken in the order
//    16s + 8(e/4) + 4(l/32) + e%4; V^T operands come from transposing LDS
//    reads (ds_read_b64_tr_b16) of row-major V tiles.
//  * Logits are built in the exp2 domain: the S^T accumulators start from
//    the key's bias term gain[h] * bias[j] / scale (read from LDS into the
//    accumulator registers), and each element takes one FMA with the scale
//    log2 e / (sqrt(D) tau) and the running max before exp2.
//  * Causality compares original positions element-wise (exact for any
//    non-decreasing positions, repeats included); key tiles past the
//    workgroup's last visible key are skipped, and waves whose queries
//    precede a whole tile skip its math.
//  * Work items run longest-first (last query blocks of a prompt first),
//    except that the longest items share their CU with short ones, and when
//    fewer than a CU's worth of items remain after two per CU, the shortest
//    go first (their CUs then take the rest), so the longest items soon run
//    alone.
//
// fp32 path: one thread per query row, K/V tiles in LDS, plain fp32 FMA.
#include "tg_internal.hpp"
#include "tg_device.hpp"

#include <limits.h>
#include <utility>

namespace tg {
namespace {


constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Index of the key tile one past the last tile a query block can see:
// tiles up to the block's last row, extended while the next tile starts at
// a position not after the block's last position (repeated positions).
template <int TB>
__device__ __forceinline__ int key_tile_end(const int32_t* __restrict__ pos, int64_t off, int n,
                                            int q_last) {
    int kt_end = q_last / TB + 1;
    const int32_t pl = pos[off + q_last];
    while (kt_end * TB < n && pos[off + kt_end * TB] <= pl) ++kt_end;
    return kt_end;
}

struct Item {
    int seg, qb, kvh, hg;
};

// f(integral_constant<int, I>) for I = B .. E-1, each index a compile-time constant.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ Item decode_item(const AttnTable& t, int item, int hkv, int ngroups) {
    int s = 0;
    for (int i = 1; i < t.n_seg; ++i)
        if (t.s[i].item_base <= item) s = i;
    const int local = item - t.s[s].item_base;
    const int per_qb = hkv * ngroups;
    Item it;
    it.seg = s;
    it.qb = t.s[s].n_qblk - 1 - local / per_qb;  // longest query blocks first
    const int rest = local % per_qb;
    it.kvh = rest / ngroups;
    it.hg = rest % ngroups;
    return it;
}

// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane
// i receives element i%4 of the 4-element rows addressed by lanes i/4,
// 4+i/4, 8+i/4 and 12+i/4 of its group.
__device__ __forceinline__ v4i16 lds_read_tr16(const LDS_AS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)p);
}

// LDS swizzles of the K and V tiles (row = key within the tile, CH = 16-byte
// chunks per row; 16 for head_dim 128, 8 for 64). The LDS has 64 banks of 4
// bytes. K is read with ds_read_b128, 16 lanes (16 consecutive keys, one
// chunk) per cycle: XOR with the key spreads them over 16 distinct chunk
// positions. V is read with ds_read_b64_tr_b16, 32 lanes (4 keys x 4
// chunks x 2 halves of a chunk) per cycle: XOR the chunk's upper bits with
// the key's low bits so the 16 (key, chunk) pairs again cover all 64 banks.
template <int CH>
__device__ __forceinline__ int swz_k(int row) { return CH == 16 ? (row & 15) : ((row >> 1) & 7); }
template <int CH>
__device__ __forceinline__ int swz_v(int row) { return CH == 16 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }

// Workgroup = HW query heads of one KV head x QS slabs of 32 query rows x SPL
// key splits; each wave owns 32 query rows of one head. Wave w: head slot
// w % HW, slab (w / HW) % QS, split w / (HW QS); split p owns key tiles
// kt = SPL*i + p. Every K/V tile staged in LDS feeds the HW x QS waves of its
// split. K and V tiles (32 keys x D) stream straight from global memory into
// LDS (global_load_lds, 16 bytes per lane, no staging registers) through an
// NSTG-stage ring filled NSTG-1 tiles ahead; 16-byte chunk c of key row r is
// stored at position c ^ swz(r), which keeps both the K operand reads
// (ds_read_b128) and the V^T operand reads (ds_read_b64_tr_b16) free of
// bank conflicts. The splits' (max, sum, O) are merged through LDS at the
// end, in split order.
template <int D, int HW, int QS, int SPL, int NSTG, int OCC, int VA = D / 32>
__global__ __launch_bounds__(64 * HW * QS * SPL, OCC) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ bias, const int32_t* __restrict__ pos, AttnTable t, int hq, int hkv,
    const float* __restrict__ gain, float qk_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
    constexpr int BN = 32;                        // keys per tile
    constexpr int NW = HW * QS * SPL;             // waves
    constexpr int ROWB = D * 2;                   // bytes per K/V row
    constexpr int CH = ROWB / 16;                 // 16-byte chunks per row
    constexpr int TILEB = BN * ROWB;              // bytes per K or V tile
    constexpr int RPI = 1024 / ROWB;              // rows per 1 KB load instruction
    constexpr int IPT = TILEB / 1024;             // load instructions per tile
    constexpr int NTL = 2 * SPL;                  // K and V tiles per stage
    constexpr int TPW = NTL * IPT / NW;           // tile load instructions per wave per stage
    constexpr int NSM = 2 * SPL;                  // small loads per stage: bias and position per split
    // Small loads per wave per stage: every wave issues the same number (a
    // wave past the last small load repeats one, same data to the same place),
    // so every wave's vmcnt bookkeeping is the same.
    constexpr int SPW = NSM >= NW ? NSM / NW : 1;
    constexpr int LPS = TPW + SPW;                // vector-memory instructions per wave per stage
    static_assert((NTL * IPT) % NW == 0 && (NSM < NW || NSM % NW == 0), "loads must split evenly over waves");
    static_assert(NSTG >= 2 && NSTG <= 4 && LPS * (NSTG - 2) < 64, "ring depth and vmcnt range");
    constexpr int KS = D / 16;                    // k-steps of q.k
    constexpr int DB = D / 32;                    // 32-wide d blocks of O
    constexpr int PS = BN / 16;                   // 16-key k-steps of P.V per tile
    static_assert(VA >= 1 && VA <= DB, "V^T blocks read ahead");
    constexpr int SM = 64;                        // bias/pos entries per tile (one dword load)
    constexpr int STAGEB = NTL * TILEB;

    __shared__ __attribute__((aligned(1024))) char ring[NSTG][STAGEB];   // [stage][split][K,V][tile]
    __shared__ __attribute__((aligned(16))) uint32_t smallr[NSTG][SPL][2][SM];  // [stage][split][bias, pos][key]
    // long shape: per wave, this head's bias term of the current tile, in units of q.k
    __shared__ __attribute__((aligned(16))) float sbias[QS == 1 ? 1 : NW][BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: load set-up stays scalar
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int G = hq / hkv;
    const int ngroups = G / HW;
    const int hl = wave % HW;
    const int qs = (wave / HW) % QS;
    const int split = wave / (HW * QS);

    // Work item: consecutive items differ in KV head first, so with 8 KV
    // heads each XCD (items are dealt round-robin to the 8 XCDs) serves one
    // KV head and keeps its K/V in its own L2; query blocks run longest first.
    // Workgroups b and b + C (C = the device's CUs) share a CU, and
    // workgroups from 2C on take the first slots that free up. The mapping
    // below pairs the longest items with short ones (reversed in groups of
    // 8, so each XCD keeps its KV head), so that they soon run alone, at the
    // faster single-workgroup rate, through the tail. With L = N - 2C later
    // workgroups (0 < L < C), the L shortest items go first, to their own
    // CUs: those slots free up first and take the later workgroups, away
    // from the CUs of the longest items.
    int item = blockIdx.x;
    {
        const int C = t.cus, N = t.n_items, L = N - 2 * C, b = item;
        if (C > 0 && L > 0 && L < C && (C & 7) == 0 && (L & 7) == 0) {
            if (b < L) item = N - L + b;                      // CUs 0..L-1: the L shortest items
            else if (b < C + L) item = b - L;                 // CUs L..C-1: the C - L longest items;
                                                              // then the partners on CUs 0..L-1
            else if (b < 2 * C) {                             // partners on CUs L..C-1, reversed
                const int j = b - C - L, g = j >> 3, r = j & 7, G = (C - L) >> 3;
                item = C + L + ((G - 1 - g) << 3) + r;
            } else item = C + (b - 2 * C);                    // the later workgroups
        } else {
            const int n2 = min(2 * C, N);
            if (C > 0 && item >= C && item < n2) {
                const int g = (item - C) >> 3, r = (item - C) & 7, G2 = (n2 - C) >> 3;
                if (g < G2) item = C + ((G2 - 1 - g) << 3) + r;
            }
        }
    }
    int sg = 0;
    for (int i = 1; i < t.n_seg; ++i)
        if (t.s[i].item_base <= item) sg = i;
    const int local = item - t.s[sg].item_base;
    const int per_qb = hkv * ngroups;
    const int qb = t.s[sg].n_qblk - 1 - local / per_qb;
    const int rest = local % per_qb;
    const int kvh = rest % hkv;
    const int hg = rest / hkv;
    const int64_t off = t.s[sg].kept_off;
    const int n = t.s[sg].n;
    const int h = kvh * G + hg * HW + hl;
    const int64_t rowb = (int64_t)hkv * ROWB;  // bytes between consecutive keys of one KV head
    const char* kbase = (const char*)(k + (off * hkv + kvh) * D);
    const char* vbase = (const char*)(v + (off * hkv + kvh) * D);

    // Loads of one stage: wave w issues instructions w*TPW .. w*TPW+TPW-1 of
    // the stage's NTL*IPT 1 KB instructions; instruction `inst` fills row
    // group inst%IPT of tile inst/IPT (split tile/2; K for even, V for odd),
    // at LDS offset inst*1 KB of the stage (tiles are laid out in that
    // order). Inside row group rg a lane loads key row rg*RPI + lane/CH,
    // chunk (lane%CH) ^ swz(row), which is the rg = 0 chunk with bits flipped
    // by the constant swz(rg*RPI).
    //
    // Full stages (every key exists) use loop-invariant per-load lane offsets
    // and one running scalar pointer per tile the wave loads, so a load costs
    // one scalar add (its LDS destination) besides the instruction itself.
    // A stage reaching past the segment's end (only the last one) re-reads
    // the segment's last key for the missing rows (they are masked or
    // skipped, never used) through the general per-lane computation.
    constexpr int NTW = TPW >= IPT ? TPW / IPT : 1;  // tiles one wave loads per stage
    static_assert(TPW % IPT == 0 || IPT % TPW == 0, "a wave's loads cover whole tiles or part of one");
    const int first_tile = __builtin_amdgcn_readfirstlane((wave * TPW) / IPT);
    const int64_t step_b = (int64_t)SPL * BN * rowb;  // bytes between a tile and the same tile one stage later
    const char* tile_ptr0[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int tile = first_tile + j;
        tile_ptr0[j] = ((tile & 1) ? vbase : kbase) + (int64_t)(tile >> 1) * BN * rowb;
    }
    uint32_t voff[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int inst = wave * TPW + i;
        const int rg = inst % IPT, kind = (inst / IPT) & 1;
        const uint32_t lo = (uint32_t)((lane / CH) * rowb + (((lane % CH) ^ (kind ? swz_v<CH>(lane / CH) : swz_k<CH>(lane / CH))) * 16));
        const uint32_t flip = (uint32_t)((kind ? swz_v<CH>(rg * RPI) : swz_k<CH>(rg * RPI)) * 16);
        voff[i] = (lo ^ flip) + (uint32_t)(rg * RPI * rowb);
    }
    const uint32_t ring0 = LDS_ADDR(&ring[0][0]);
    const uint32_t small0 = LDS_ADDR(&smallr[0][0][0][0]);
    constexpr uint32_t SMALL_STAGE = SPL * 2 * SM * 4;
    const uint32_t wave_lds = (uint32_t)(wave * TPW * 1024);
    auto issue = [&](int it) __attribute__((always_inline)) {
        const int st = it % NSTG;
        const uint32_t tl = ring0 + (uint32_t)st * STAGEB;
        const uint32_t sm = small0 + (uint32_t)st * SMALL_STAGE;
        if ((SPL * it + SPL) * BN <= n) {
            const int64_t adv = (int64_t)it * step_b;
            const uint32_t ldsw = tl + wave_lds;
            static_for<0, TPW>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                dma16_so_at<i * 1024>(tile_ptr0[i * NTW / TPW] + adv, voff[i], ldsw);
            });
        } else {
#pragma nounroll
            for (int i = 0; i < TPW; ++i) {
                const int inst = wave * TPW + i;
                const int tile = inst / IPT, rg = inst % IPT;
                const int sp_ = tile >> 1, kind = tile & 1;
                const int key0 = (SPL * it + sp_) * BN;
                const int r0 = min(key0, n - 1);
                const int row = rg * RPI + lane / CH;
                const int chunk = (lane % CH) ^ (kind ? swz_v<CH>(row) : swz_k<CH>(row));
                dma16_so((kind ? vbase : kbase) + (int64_t)r0 * rowb,
                         (uint32_t)((min(key0 + row, n - 1) - r0) * rowb + chunk * 16),
                         tl + (uint32_t)(inst * 1024));
            }
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int sid = (wave * SPW + i) % NSM;  // split sid/2, bias (even) or position (odd)
            const int sp_ = sid >> 1;
            const int key0 = (SPL * it + sp_) * BN;
            const int r0 = min(key0, n - 1);
            const char* base = (sid & 1) ? (const char*)(pos + off + r0) : (const char*)(bias + off + r0);
            // one dword per lane covers SM >= BN keys: always clamp
            const uint32_t vo = (uint32_t)(min(key0 + lane, n - 1) - r0) * 4u;
            dma4_so(base, vo, sm + (uint32_t)((sp_ * 2 + (sid & 1)) * SM * 4));
        }
    };

    // The first stage exists for every block (it covers the block's first
    // rows); its loads go out before the position lookups and the Q loads, so
    // their latencies overlap. Only the wait below, for every load of the
    // wave, separates them from the ring's own counting.
    issue(0);

    const int b0 = qb * 32 * QS;                  // first row of the workgroup's block
    const int i0 = b0 + 32 * qs;                  // first row of this wave's slab
    const bool live = i0 < n;                     // the block's last slabs may lie past the segment
    const int q_last = min(n, i0 + 32) - 1;
    const int n_tiles = live ? key_tile_end<BN>(pos, off, n, q_last) : 0;
    const int n_tiles_wg = key_tile_end<BN>(pos, off, n, min(n, b0 + 32 * QS) - 1);
    const int n_it = (n_tiles_wg + SPL - 1) / SPL;

    const int qi = min(i0 + l32, n - 1);
    const int32_t my_pos = pos[off + qi];
    const float c = qk_scale * LOG2E;
    // The logit in the exp2 domain is c * (q.k + gb * bias): the bias term
    // seeds the S^T accumulators, the scale c is applied inside exp2.
    const float gb = gain[h] / qk_scale;

    bf16x8 qf[KS];
    {
        const uint16_t* qrow = q + ((off + qi) * hq + h) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(qrow + s * 16);
    }
    // The ring's vmcnt bookkeeping counts only its own loads: finish every
    // other vector-memory load (and the first stage) first and keep the
    // compiler from moving any past this point.
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");

    // Per-lane parts of the LDS operand addresses (stage base added per tile).
    // K: key row l32, chunk (2s + hh) ^ swz_k(row), which is the s = 0 chunk
    // with bits flipped by 2s. V^T (transpose reads): lane L of group
    // g = L/16 addresses key 16s + 4(g/2) + (L%16)/4 (+8 for the upper four
    // slots) at d = 32b + 16(g%2) + 4(L%4); the swizzled chunk of d-block b is
    // the b = 0 chunk with bits flipped by 4b.
    const uint32_t k_lane = (uint32_t)(l32 * ROWB + ((hh ^ swz_k<CH>(l32)) * 16));
    uint32_t v_lane;
    {
        const int g = lane >> 4, r16 = lane & 15;
        const int dsub = 16 * (g & 1) + 4 * (r16 & 3);
        const int keyo = 4 * (g >> 1) + (r16 >> 2);
        v_lane = (uint32_t)(keyo * ROWB + (((dsub >> 3) ^ swz_v<CH>(keyo)) * 16) + (dsub & 7) * 2);
    }
    const uint32_t k_split = (uint32_t)(split * 2 * TILEB), v_split = (uint32_t)((split * 2 + 1) * TILEB);

    f32x16 acc_o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc_o[b][j] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // One key tile for this wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
    // Every LDS operand is read ahead of its use so that the read latency
    // overlaps other work: the bias seed and all K operands before the first
    // q.k MFMA, the V^T operands right after the q.k MFMAs (the softmax runs
    // while they arrive). sched_barrier keeps the compiler from sinking the
    // reads back next to their uses.
    // K operands and the bias seed of the tile in stage st: register j of
    // the S^T layout holds key 8(j/4) + 4hh + j%4. The short shape, bound by
    // the latency of its per-tile chain, reads its 16 keys' bias as four
    // 16-byte vectors straight from the stage and scales them by this head's
    // gain in registers. The long shape, closer to its issue rate, scales the
    // tile's 32 bias values once per wave (one multiply per lane) and reads
    // them back through a per-wave array.
    auto read_k = [&](int st, bf16x8 (&kf)[KS], f32x16& seed) __attribute__((always_inline)) {
        const LDS_AS float* bsv = (const LDS_AS float*)(uintptr_t)(small0 + (uint32_t)st * SMALL_STAGE +
                                                                    (uint32_t)(split * 2 * SM * 4));
        // Operand addresses: XOR-swizzled chunks are one XOR away from the
        // per-lane base. The empty asm makes the base opaque per tile, so the
        // compiler keeps one address register instead of hoisting one per
        // read and ring stage out of the loop.
        uint32_t ka = ring0 + (uint32_t)st * STAGEB + k_split + k_lane;
        asm volatile("" : "+v"(ka));
        if constexpr (QS == 1) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 bb = *(const LDS_AS f32x4*)&bsv[8 * g4 + 4 * hh];
#pragma unroll
                for (int e = 0; e < 4; ++e) seed[4 * g4 + e] = bb[e] * gb;
            }
        } else {
            if (lane < BN) sbias[wave][lane] = bsv[lane] * gb;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 bb = *(const LDS_AS f32x4*)&sbias[wave][8 * g4 + 4 * hh];
#pragma unroll
                for (int e = 0; e < 4; ++e) seed[4 * g4 + e] = bb[e];
            }
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[s] = *(const LDS_AS bf16x8*)(uintptr_t)(ka ^ (uint32_t)(s << 5));
    };

    // One key tile for this wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
    // Every LDS operand is read ahead of its use so that the read latency
    // overlaps other work: the bias seed and all K operands before the first
    // q.k MFMA, the V^T operands right after the q.k MFMAs (the softmax runs
    // while they arrive). sched_barrier keeps the compiler from sinking the
    // reads back next to their uses.
    bf16x8 kf[KS];
    f32x16 seed;
    auto compute = [&](int kt, int st) __attribute__((always_inline)) {
        if (kt >= n_tiles) return;  // past the slab's last visible key
        const LDS_AS int32_t* psv = (const LDS_AS int32_t*)(uintptr_t)(small0 + (uint32_t)st * SMALL_STAGE +
                                                                        (uint32_t)((split * 2 + 1) * SM * 4));
        // Positions never decrease along the kept rows, so keys before the
        // slab's first query row are visible to all of its queries: only tiles
        // reaching row i0 (the ragged end among them) are masked element-wise.
        const bool need_mask = (kt + 1) * BN > i0;
        read_k(st, kf, seed);
        uint32_t va = ring0 + (uint32_t)st * STAGEB + v_split + v_lane;
        asm volatile("" : "+v"(va));
        f32x16 acc_s = seed;  // the bias seed starts the accumulation
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s) acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc_s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 vf[DB][PS];
        auto read_v = [&](int b) __attribute__((always_inline)) {
            const uint32_t vb = va ^ (uint32_t)(b << 6);
#pragma unroll
            for (int s = 0; s < PS; ++s) {
                const v4i16 lo = lds_read_tr16((const LDS_AS char*)(uintptr_t)(vb + 16 * s * ROWB));
                const v4i16 hi = lds_read_tr16((const LDS_AS char*)(uintptr_t)(vb + (16 * s + 8) * ROWB));
                vf[b][s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
#pragma unroll
        for (int b = 0; b < VA; ++b) read_v(b);
        __builtin_amdgcn_sched_barrier(0);
        // acc_s now holds q.k + gb * bias; the exp2-domain logit is c times it.
        if (need_mask) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int key0 = 8 * g4 + 4 * hh;
                const i32x4 pp = *(const LDS_AS i32x4*)&psv[key0];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool vis = (kt * BN + key0 + e < n) & (pp[e] <= my_pos);
                    acc_s[4 * g4 + e] = vis ? acc_s[4 * g4 + e] : -INFINITY;
                }
            }
        }
        float mx = acc_s[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, acc_s[j]);
        {   // lanes l and l^32 hold the two halves of one query's keys
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;  // c > 0: max of the exp2-domain logits
        }
        // The reference max only moves when some row's tile max exceeds it by
        // more than 8 (a factor 256): softmax does not depend on the
        // reference, and p <= 256 stays exact enough in fp32 and bf16. This
        // skips almost every rescale of O after the first tiles.
        if (__any(mx > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
            l_run *= corr;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc_o[b][j] *= corr;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
        float lsum = 0.0f;
        // P^T as B operands: k-step s uses S^T registers 8*s .. +8, i.e.
        // keys 16s + 8(e/4) + 4hh + e%4 for slot e.
        bf16x8 pf[PS];
#pragma unroll
        for (int s = 0; s < PS; ++s) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(acc_s[8 * s + 2 * e], c, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(acc_s[8 * s + 2 * e + 1], c, -m_use));
                lsum += p0 + p1;
                w[e] = pack_bf16x2(p0, p1);
            }
            pf[s] = __builtin_bit_cast(bf16x8, w);
        }
        l_run += lsum;
        // With VA < DB only VA d blocks of V^T are read ahead of the softmax;
        // block b + VA's reads go out before block b's MFMAs, so at most
        // VA + 1 blocks of V^T are live (fewer registers).
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            if (b + VA < DB) {
                __builtin_amdgcn_sched_barrier(0);
                read_v(b + VA);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int s = 0; s < PS; ++s) acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[b][s], pf[s], acc_o[b], 0, 0, 0);
        }
    };

    // Ring with one barrier per iteration: stage it%NSTG holds iteration it.
    // After the barrier of iteration it, every wave's loads of stage it have
    // landed and every wave has finished iteration it-1, so the loads of
    // iteration it+NSTG-1 go into that iteration's stage before this
    // iteration's compute.
#pragma unroll
    for (int i = 1; i < NSTG - 1; ++i)
        if (i < n_it) issue(i);
    for (int it = 0; it < n_it; ++it) {
        // every load of iterations <= it has landed (this wave's); the later
        // ones issued so far (at most NSTG-2 stages) may still be in flight
        const int later = min(n_it - 1, it + NSTG - 2) - it;
        if constexpr (NSTG >= 4) {
            if (later >= 2) wait_vmcnt<LPS * 2>();
            else if (later == 1) wait_vmcnt<LPS>();
            else wait_vmcnt<0>();
        } else if constexpr (NSTG == 3) {
            if (later >= 1) wait_vmcnt<LPS>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        ring_barrier();
        if (it + NSTG - 1 < n_it) issue(it + NSTG - 1);
        compute(SPL * it + split, it % NSTG);
    }
    wait_vmcnt<0>();
    ring_barrier();  // the merge below reuses the ring buffers

    // Merge the key splits: splits 1.. hand (m, l, O) to split 0 through LDS
    // (the ring is free now); split 0 combines them in split order.
    constexpr int NH = HW * QS;                        // waves per split
    constexpr int PER = NH * DB * 16 * 64;             // floats of O per handing split
    static_assert((SPL - 1) * (PER + 2 * NH * 64) * 4 <= NSTG * STAGEB, "merge buffer");
    float* const xo = (float*)&ring[0][0];
    float* const xm = xo + (SPL - 1) * PER;            // [SPL-1][NH][64] max, then the same for sums
    constexpr int XL = (SPL - 1) * NH * 64;
    const int wl = wave % NH;                          // this wave's slot within its split
    if (split > 0) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) xo[(split - 1) * PER + ((wl * DB + b) * 16 + j) * 64 + lane] = acc_o[b][j];
        xm[((split - 1) * NH + wl) * 64 + lane] = m_run;
        xm[XL + ((split - 1) * NH + wl) * 64 + lane] = l_run;
    }
    if constexpr (SPL > 1) __syncthreads();
    if (split == 0) {
        float ms[SPL], ls[SPL];
        ms[0] = m_run;
        ls[0] = l_run;
        float m = m_run;
#pragma unroll
        for (int q2 = 1; q2 < SPL; ++q2) {
            ms[q2] = xm[((q2 - 1) * NH + wl) * 64 + lane];
            ls[q2] = xm[XL + ((q2 - 1) * NH + wl) * 64 + lane];
            m = fmaxf(m, ms[q2]);
        }
        const float mu = (m == -INFINITY) ? 0.0f : m;
        float a[SPL];
        float lt = 0.0f;
#pragma unroll
        for (int q2 = 0; q2 < SPL; ++q2) {
            a[q2] = __builtin_amdgcn_exp2f(ms[q2] - mu);
            lt += ls[q2] * a[q2];
        }
        lt += __shfl_xor(lt, 32);
        const float inv = 1.0f / lt;
        const int row = i0 + l32;
        if (row < n) {
            uint16_t* orow = out + ((off + row) * hq + h) * D;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 4 * g4 + e;
                        float acc = acc_o[b][j] * a[0];
#pragma unroll
                        for (int q2 = 1; q2 < SPL; ++q2)
                            acc += xo[(q2 - 1) * PER + ((wl * DB + b) * 16 + j) * 64 + lane] * a[q2];
                        o[e] = acc * inv;
                    }
                    uint2 w;
                    w.x = pack_bf16x2(o[0], o[1]);
                    w.y = pack_bf16x2(o[2], o[3]);
                    *(uint2*)(orow + 32 * b + 8 * g4 + 4 * hh) = w;
                }
            if (lse && hh == 0) lse[(int64_t)h * t.m_total + off + row] = (mu + log2f(lt)) * LN2;
        }
    }
}

// fp32 path: a 64-thread workgroup owns 64 query rows of one head; each
// thread keeps its query row and output accumulators in registers.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ bias, const int32_t* __restrict__ pos, AttnTable t, int hq, int hkv,
    const float* __restrict__ gain, float qk_scale, float* __restrict__ out, float* __restrict__ lse) {
    constexpr int TB = 32;  // keys per tile
    __shared__ float kt_[TB][D];
    __shared__ float vt_[TB][D];
    __shared__ float bs_[TB];
    __shared__ int32_t ps_[TB];

    const int tid = threadIdx.x;
    // item decomposition: ngroups = hq (one head per item), 64 rows per block
    const Item it = decode_item(t, blockIdx.x, 1, hq);
    const int h = it.hg;
    const int kvh = (h * hkv) / hq;
    const int64_t off = t.s[it.seg].kept_off;
    const int n = t.s[it.seg].n;
    const int row = it.qb * 64 + tid;
    const int qi = min(row, n - 1);
    const int q_last_blk = min(n, it.qb * 64 + 64) - 1;
    const int kt_end = (q_last_blk / TB + 1);
    // extend over repeated positions
    int kend = kt_end;
    {
        const int32_t pl = pos[off + q_last_blk];
        while (kend * TB < n && pos[off + kend * TB] <= pl) ++kend;
    }
    const int32_t my_pos = pos[off + qi];
    const float gh = gain[h];

    float qv[D], o[D];
    const float* qrow = q + ((off + qi) * hq + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qv[d] = qrow[d];
        o[d] = 0.0f;
    }
    float m_run = -INFINITY, l_run = 0.0f;
    for (int tile = 0; tile < kend; ++tile) {
        const int j0 = tile * TB;
        for (int u = tid; u < TB * D; u += 64) {
            const int key = u / D, d = u % D;
            const int j = min(j0 + key, n - 1);
            kt_[key][d] = k[((off + j) * hkv + kvh) * D + d];
            vt_[key][d] = v[((off + j) * hkv + kvh) * D + d];
        }
        if (tid < TB) {
            const int j = j0 + tid;
            bs_[tid] = bias[off + min(j, n - 1)];
            ps_[tid] = (j < n) ? pos[off + j] : INT_MAX;
        }
        __syncthreads();
        float lg[TB];
        float mx = -INFINITY;
        for (int key = 0; key < TB; ++key) {
            float dot = 0.0f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = fmaf(qv[d], kt_[key][d], dot);
            float x = fmaf(dot, qk_scale, gh * bs_[key]);
            if (ps_[key] > my_pos) x = -INFINITY;
            lg[key] = x;
            mx = fmaxf(mx, x);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float corr = expf(m_run - m_use);
        l_run *= corr;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= corr;
        for (int key = 0; key < TB; ++key) {
            const float p = expf(lg[key] - m_use);
            l_run += p;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] = fmaf(p, vt_[key][d], o[d]);
        }
        m_run = m_new;
        __syncthreads();
    }
    if (row < n) {
        float* orow = out + ((off + row) * hq + h) * D;
        const float inv = 1.0f / l_run;
#pragma unroll
        for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
        if (lse) lse[(int64_t)h * t.m_total + off + row] = m_run + logf(l_run);
    }
}

int heads_per_wg(int g) { return (g % 2 == 0) ? 2 : 1; }

// Prompts of at least this many kept rows take the long-prompt shape, and
// from ATTN_XL_ROWS on (head_dim 128) its three-workgroups-per-CU form.
constexpr int64_t ATTN_LONG_ROWS = 4096;
constexpr int64_t ATTN_XL_ROWS = 16384;

// The kernel shapes (HW heads per item in all):
//  0 (short prompts): 32 query rows x 2 key splits, 2-stage ring, two
//    workgroups per CU: the splits halve the serial chain of the longest
//    query blocks, which bounds a short causal problem;
//  1 (long prompts): 2 slabs of 32 query rows share every K/V tile (half
//    the loaded bytes per MFMA), one key split, 3-stage ring, two workgroups
//    per CU;
//  2 (the longest prompts, head_dim 128, two query heads per KV head in
//    the workgroup; other heads take shape 1): shape 1 at three workgroups per
//    CU, which the registers allow once only one d block of V^T is read
//    ahead of the softmax (the rest one block ahead of its MFMAs). The third
//    workgroup hides more latency than the later V^T reads expose once
//    there are enough work items to keep it busy.
template <int D, int HW>
void launch_cfg(int cfg, dim3 grid, hipStream_t st, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                const float* bias, const int32_t* pos, const AttnTable& t, int hq, int hkv, const float* gain,
                float qk_scale, uint16_t* out, float* lse) {
    if constexpr (D == 128 && HW == 2) {
        if (cfg == 2) {
            hipLaunchKernelGGL((attn_bf16_kernel<D, HW, 2, 1, 3, 3, 1>), grid, dim3(64 * HW * 2), 0, st, q, k, v, bias,
                               pos, t, hq, hkv, gain, qk_scale, out, lse);
            return;
        }
    }
    if (cfg == 0)
        hipLaunchKernelGGL((attn_bf16_kernel<D, HW, 1, 2, 2, HW == 2 ? 2 : 1>), grid, dim3(64 * HW * 2), 0, st, q, k, v, bias, pos,
                           t, hq, hkv, gain, qk_scale, out, lse);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<D, HW, 2, 1, 3, 2>), grid, dim3(64 * HW * 2), 0, st, q, k, v, bias, pos,
                           t, hq, hkv, gain, qk_scale, out, lse);
}

}  // namespace

AttnConfig attention_config(tg_dtype dt, int hq, int hkv, int64_t max_rows) {
    AttnConfig c;
    if (dt == TG_F32) {
        c.kind = 0;
        c.block_rows = 64;
        c.heads_per_item = 1;
        return c;
    }
    const int cfg = max_rows >= ATTN_XL_ROWS ? 2 : (max_rows >= ATTN_LONG_ROWS ? 1 : 0);
    c.kind = cfg;
    c.block_rows = cfg == 0 ? 32 : 64;
    c.heads_per_item = heads_per_wg(hq / hkv);
    return c;
}

hipError_t launch_attention(tg_dtype dt, const void* q, const void* k, const void* v,
                            const float* bias, const int32_t* pos, const AttnTable& t, int hq,
                            int hkv, int head_dim, const float* gain, float tau, void* out,
                            float* lse, hipStream_t st) {
    if (t.n_items == 0) return hipSuccess;
    const float qk_scale = 1.0f / (sqrtf((float)head_dim) * tau);
    const dim3 grid((unsigned)t.n_items);
    if (dt == TG_BF16) {
        const int hw = heads_per_wg(hq / hkv);
        const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v;
        uint16_t* oo = (uint16_t*)out;
        if (head_dim == 128 && hw == 2)
            launch_cfg<128, 2>(t.cfg, grid, st, qq, kk, vv, bias, pos, t, hq, hkv, gain, qk_scale, oo, lse);
        else if (head_dim == 128)
            launch_cfg<128, 1>(t.cfg, grid, st, qq, kk, vv, bias, pos, t, hq, hkv, gain, qk_scale, oo, lse);
        else if (hw == 2)
            launch_cfg<64, 2>(t.cfg, grid, st, qq, kk, vv, bias, pos, t, hq, hkv, gain, qk_scale, oo, lse);
        else
            launch_cfg<64, 1>(t.cfg, grid, st, qq, kk, vv, bias, pos, t, hq, hkv, gain, qk_scale, oo, lse);
    } else {
        if (head_dim == 128)
            hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, st, (const float*)q,
                               (const float*)k, (const float*)v, bias, pos, t, hq, hkv, gain,
                               qk_scale, (float*)out, lse);
        else
            hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, st, (const float*)q,
                               (const float*)k, (const float*)v, bias, pos, t, hq, hkv, gain,
                               qk_scale, (float*)out, lse);
    }
    return hipGetLastError();
}

}  // namespace tg
