// Backward of token-gated attention: the path by which the gate's scores
// receive a gradient.
//
// Defined by the TokenGate pages: spke.com article, section "Was ist
// token-gated Attention?" (the score of each kept token becomes a bias on
// the attention logits, which gives the gradient a way back to the scorer,
// in the manner of a mixture-of-experts router; per-head gain and a
// temperature) and the ai4bro.com post, section on how learned token pruning
// works (same). With l_ij = c q_i.k_j + g_h b_j (c = 1/(sqrt(D) tau)), p =
// softmax over the visible keys, o = p V and an upstream gradient dO:
//     dV_j = sum_i p_ij dO_i,   dP_ij = dO_i . v_j,
//     dS_ij = p_ij (dP_ij - dO_i . o_i),
//     dQ_i = c sum_j dS_ij k_j,   dK_j = c sum_i dS_ij q_i,
//     db_j = sum_h g_h sum_i dS_ij,   dg_h = sum_ij dS_ij b_j,
//     dtau = -(c / tau) sum_hij dS_ij q_i.k_j,
// and the score of a kept document row gets db_j * sigmoid(-s_j) (the
// derivative of logsigmoid); question and pruned rows get 0.
//
// Three launches (bf16 inputs, fp32 gradients): prep; one grid whose work
// items alternate between the dkdv pass (2) and the dq pass (3), so that the
// two passes share the chip and neither's tail runs alone; one grid for the
// reductions (4).
//  1. prep: Dl[h][i] = dO_i . o_i (the softmax row term).
//  2. dkdv: one wave per (prompt, 32-key block, query head). The key block
//     sits in LDS; the wave walks the query blocks that can see it and
//     forms S = Q K^T and dP = dO V^T on 32x32x16 bf16 MFMA (one key per
//     lane column, 16 queries down its registers), then P and dS, and
//     accumulates dV += P^T dO and dK += dS^T Q with P^T / dS^T taken
//     straight from those registers (the query order inside each 16-wide
//     k-step is permuted the same way on both operands) and dO / Q read
//     transposed from LDS (ds_read_b64_tr_b16). Per-head partial dK, dV and
//     sum_i dS_ij go to a workspace, with the fp32 sum_i dS_ij (q_i . k_j) of
//     the unrounded dS and S registers per key and head (the temperature's
//     gradient: taken from the bf16-rounded products of dK instead, it loses
//     the digits that survive its cancellation). Blocks that every query of
//     the query block can fully see take a path without the causal and
//     ragged masks.
//  3. dq: one wave per (prompt, 32-query block, query head), like the
//     forward kernel: S^T = K Q^T and dP^T = V dO^T with Q and dO in
//     registers, dS^T in registers, dQ^T += K^T dS^T with K^T read
//     transposed from LDS.
//  When the (block, head) items are too few to fill the chip, each item of 2
//  and 3 is split over two waves, each walking half of the blocks; their
//  partials are summed in a fixed order below.
//  4. reduce: sums the per-head partials of each KV head in a fixed order
//     (so the result is deterministic) and applies the gains to db; other
//     workgroups of the same grid reduce dg_h = sum_j b_j sum_i dS_ij per
//     head and dtau from the per-key sums of dS_ij (q_i . k_j), each in a
//     fixed order, and sum the dq parts of split items. The score kernel
//     applies sigmoid(-s).
// LDS tiles are row-major with a 16-byte pad per row (row stride D*2+16
// bytes), which spreads both the row reads and the transpose reads over
// the banks.
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

constexpr float LOG2E = 1.4426950408889634f;

template <int D>
struct Tile {
    static constexpr int RS = D * 2 + 16;  // padded row stride in bytes
    static constexpr int BYTES = 32 * RS;
};

__device__ __forceinline__ v4i16 read_tr16(const LDS_AS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)p);
}

// Copy 32 rows (row r of the tile <- global row min(row0 + r, n_rows - 1))
// of D bf16 into a padded LDS tile; `stride` elements between global rows.
template <int D>
__device__ __forceinline__ void load_tile(LDS_AS char* tile, const uint16_t* __restrict__ src, int64_t stride,
                                          int row0, int n_rows, int lane) {
    constexpr int CH = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int u = 0; u < 32 * CH / 64; ++u) {
        const int idx = u * 64 + lane;
        const int r = idx / CH, ch = idx % CH;
        const int gr = min(row0 + r, n_rows - 1);
        const u32x4 w = *(const u32x4*)(src + gr * stride + ch * 8);
        *(LDS_AS u32x4*)(tile + r * Tile<D>::RS + ch * 16) = w;
    }
}

// The same copy split in two halves, so that the global loads of the next
// tile can be in flight (in registers) while the current tile is used.
template <int D>
struct TileRegs {
    static constexpr int N = 32 * (D / 8) / 64;  // 16-byte chunks per lane
    u32x4 w[N];
};
template <int D>
__device__ __forceinline__ void fetch_tile(TileRegs<D>& r, const uint16_t* __restrict__ src, int64_t stride,
                                           int row0, int n_rows, int lane) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int u = 0; u < TileRegs<D>::N; ++u) {
        const int idx = u * 64 + lane;
        const int gr = min(row0 + idx / CH, n_rows - 1);
        r.w[u] = *(const u32x4*)(src + gr * stride + (idx % CH) * 8);
    }
}
template <int D>
__device__ __forceinline__ void store_tile(LDS_AS char* tile, const TileRegs<D>& r, int lane) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int u = 0; u < TileRegs<D>::N; ++u) {
        const int idx = u * 64 + lane;
        *(LDS_AS u32x4*)(tile + (idx / CH) * Tile<D>::RS + (idx % CH) * 16) = r.w[u];
    }
}

// A/B operand for k-step s of a 32x32x16 MFMA whose rows (A) or columns (B)
// are the tile's columns d = 32b + (lane%32) and whose k-slots (lane/32, e)
// are tile rows 16s + 8(e/4) + 4(lane/32) + e%4: four transpose reads.
template <int D>
__device__ __forceinline__ bf16x8 tile_tr_operand(const LDS_AS char* tile, int b, int s, int lane) {
    const int g = lane >> 4, r16 = lane & 15;
    const int dsub = 16 * (g & 1) + 4 * (r16 & 3);
    const int rowo = 4 * (g >> 1) + (r16 >> 2);
    const int ra = 16 * s + rowo, rb = ra + 8;
    const int dd = 32 * b + dsub;
    const v4i16 lo = read_tr16(tile + ra * Tile<D>::RS + dd * 2);
    const v4i16 hi = read_tr16(tile + rb * Tile<D>::RS + dd * 2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row operand: tile row (lane%32), elements 16s + 8(lane/32) .. +8.
template <int D>
__device__ __forceinline__ bf16x8 tile_row_operand(const LDS_AS char* tile, int s, int lane) {
    return *(const LDS_AS bf16x8*)(tile + (lane & 31) * Tile<D>::RS + (16 * s + 8 * (lane >> 5)) * 2);
}

// When the (block, head) items alone would leave the chip short of waves,
// each is split in two work items over halves of the blocks it walks, so
// the longest chains (the earliest key blocks, the latest query blocks) are
// half as long; the partial results are summed in a fixed order afterwards.
constexpr int BWD_SPLIT_BELOW = 2048;  // (block, head) items under which the split pays

struct BwdSeg {
    int64_t off;     // first kept row
    int32_t n;       // kept rows
    int32_t n_blk;   // 32-row blocks
    int32_t item0;   // first (block, head, part) work item
    int32_t pad;
};
struct BwdTable {
    int32_t n_seg;
    int32_t n_items;  // sum over prompts of n_blk * hq * parts
    int64_t m_total;
    int32_t parts;    // work items per (block, head): 1 or 2
    int32_t pad;
    BwdSeg s[TG_MAX_SEQS];
};

// Work item -> (prompt, block, head, part): item = item0 + (order(block) *
// hq + h) * parts + part, blocks in the order given (the ones with the most
// work first).
__device__ __forceinline__ void bwd_item(const BwdTable& t, int item, int hq, bool last_first, int& sg, int& blk,
                                         int& h, int& part) {
    sg = 0;
    for (int i = 1; i < t.n_seg; ++i)
        if (t.s[i].item0 <= item) sg = i;
    const int local = item - t.s[sg].item0;
    part = local % t.parts;
    const int bh = local / t.parts;
    blk = last_first ? t.s[sg].n_blk - 1 - bh / hq : bh / hq;
    h = bh % hq;
}

// 1. Dl[h][i] = dO_i . o_i (fp32), one thread per (row, head).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ d_out,
                                                      const uint16_t* __restrict__ out, int64_t m, int hq,
                                                      float* __restrict__ dl) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= m * hq) return;
    const int64_t row = idx / hq;
    const int h = (int)(idx % hq);
    const uint16_t* a = d_out + idx * D;
    const uint16_t* b = out + idx * D;
    float acc = 0.0f;
#pragma unroll 4
    for (int c = 0; c < D; c += 8) {
        const uint4 x = *(const uint4*)(a + c), y = *(const uint4*)(b + c);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(__uint_as_float(xs[e] << 16), __uint_as_float(ys[e] << 16), acc);
            acc = fmaf(__uint_as_float(xs[e] & 0xffff0000u), __uint_as_float(ys[e] & 0xffff0000u), acc);
        }
    }
    dl[(int64_t)h * m + row] = acc;
}

// 2. Per (prompt, key block, head): partial dK, dV of that head, and per key
// sum_i dS_ij and sum_i dS_ij (q_i . k_j). ws layout per part (fp32): dk
// [hq][M][D], dv [hq][M][D], db [hq][M], dt [hq][M].
template <int D>
__device__ __forceinline__ void bwd_dkdv_body(
    int item, LDS_AS char* kt, LDS_AS char* vt, LDS_AS char* qt, LDS_AS char* dot, LDS_AS float* s_nlse,
    LDS_AS float* s_dl, LDS_AS int32_t* s_pos,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ d_out, const float* __restrict__ lse, const float* __restrict__ dl,
    const float* __restrict__ bias, const int32_t* __restrict__ pos, BwdTable t, int hq, int hkv,
    const float* __restrict__ gain, float c, float* __restrict__ ws_dk, float* __restrict__ ws_dv,
    float* __restrict__ ws_db, float* __restrict__ ws_dt) {
    constexpr int KS = D / 16, DB = D / 32;
    const int lane = threadIdx.x;
    const int hh = lane >> 5, l32 = lane & 31;
    int sg, jb, h, part;
    bwd_item(t, item, hq, false, sg, jb, h, part);  // early key blocks see the most queries
    const int64_t off = t.s[sg].off, m = t.m_total;
    const int n = t.s[sg].n;
    const int kvh = h / (hq / hkv);
    const int key0 = 32 * jb;
    const float c2 = c * LOG2E, gb2 = gain[h] * LOG2E;

    load_tile<D>((LDS_AS char*)kt, k + (off * hkv + kvh) * D, (int64_t)hkv * D, key0, n, lane);
    load_tile<D>((LDS_AS char*)vt, v + (off * hkv + kvh) * D, (int64_t)hkv * D, key0, n, lane);
    __syncthreads();
    // The key block's row operands (S = Q K^T, dP = dO V^T) stay in registers.
    bf16x8 kop[KS], vop[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        kop[s] = tile_row_operand<D>((const LDS_AS char*)kt, s, lane);
        vop[s] = tile_row_operand<D>((const LDS_AS char*)vt, s, lane);
    }
    const int key = key0 + l32;                       // this lane's key column
    const bool key_ok = key < n;
    const float kterm = gb2 * bias[off + min(key, n - 1)];
    const int32_t p_key = pos[off + min(key, n - 1)];
    const int32_t p_key0 = pos[off + key0];
    // Every query of a full query block at or after this position sees every
    // key of a full key block.
    const int32_t p_key_last = key0 + 32 <= n ? pos[off + key0 + 31] : INT32_MAX;

    // First query block that can see a key of this block (positions never
    // decrease along the kept rows; repeats can reach earlier blocks).
    int i0 = jb;
    while (i0 > 0 && pos[off + 32 * i0 - 1] >= p_key0) --i0;

    f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            acc_dk[b][j] = 0.0f;
            acc_dv[b][j] = 0.0f;
        }
    float db_acc = 0.0f, dt_acc = 0.0f;

    // Q / dO tiles and the per-query scalars of block ib + 1 are fetched into
    // registers while block ib is processed.
    const uint16_t* qsrc = q + (off * hq + h) * D;
    const uint16_t* dsrc = d_out + (off * hq + h) * D;
    TileRegs<D> rq, rd;
    float n_nlse = 0.0f, n_dl = 0.0f;
    int32_t n_pos = 0;
    auto fetch_q = [&](int ib) __attribute__((always_inline)) {
        fetch_tile<D>(rq, qsrc, (int64_t)hq * D, 32 * ib, n, lane);
        fetch_tile<D>(rd, dsrc, (int64_t)hq * D, 32 * ib, n, lane);
        const int qi = min(32 * ib + (lane & 31), n - 1);
        n_nlse = -lse[(int64_t)h * m + off + qi] * LOG2E;
        n_dl = dl[(int64_t)h * m + off + qi];
        n_pos = pos[off + qi];
    };
    // This item's half of the query blocks i0 .. n_blk - 1.
    const int n_blk = t.s[sg].n_blk;
    const int half = t.parts == 1 ? n_blk - i0 : (n_blk - i0 + 1) / 2;
    const int lo = part == 0 ? i0 : i0 + half, hi = part == 0 ? i0 + half : n_blk;
    if (lo < hi) fetch_q(lo);
    for (int ib = lo; ib < hi; ++ib) {
        const int qrow0 = 32 * ib;
        __syncthreads();  // previous iteration's reads of qt / dot are done
        store_tile<D>((LDS_AS char*)qt, rq, lane);
        store_tile<D>((LDS_AS char*)dot, rd, lane);
        if (lane < 32) {
            s_nlse[lane] = n_nlse;
            s_dl[lane] = n_dl;
            s_pos[lane] = n_pos;
        }
        // Lane 0 holds the position of the block's first (lowest) query.
        const bool full = qrow0 + 32 <= n && __builtin_amdgcn_readfirstlane(n_pos) >= p_key_last;
        __syncthreads();
        if (ib + 1 < hi) fetch_q(ib + 1);
        f32x16 sacc, pacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            sacc[j] = 0.0f;
            pacc[j] = 0.0f;
        }
        // Operands are read from LDS ahead of their MFMAs (one batch of row
        // reads, then the transpose reads while the softmax math runs), so the
        // LDS latency is paid once per batch rather than once per MFMA.
        bf16x8 qop[KS], dop[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qop[s] = tile_row_operand<D>((const LDS_AS char*)qt, s, lane);
            dop[s] = tile_row_operand<D>((const LDS_AS char*)dot, s, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[s], kop[s], sacc, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dop[s], vop[s], pacc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 dotr[DB][2], qtr[DB][2];
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                dotr[b][s] = tile_tr_operand<D>((const LDS_AS char*)dot, b, s, lane);
                qtr[b][s] = tile_tr_operand<D>((const LDS_AS char*)qt, b, s, lane);
            }
        __builtin_amdgcn_sched_barrier(0);
        // Register j: query qrow0 + 8(j/4) + 4hh + j%4 of key `key`; the
        // per-query scalars of four consecutive queries come in one read.
        f32x4 nl[4], dlq[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            nl[g4] = *(const LDS_AS f32x4*)(s_nlse + 8 * g4 + 4 * hh);
            dlq[g4] = *(const LDS_AS f32x4*)(s_dl + 8 * g4 + 4 * hh);
        }
        bf16x8 pf[2], dsf[2];
        auto softmax = [&](auto masked) __attribute__((always_inline)) {
            i32x4 pq[4];
            if constexpr (decltype(masked)::value) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) pq[g4] = *(const LDS_AS i32x4*)(s_pos + 8 * g4 + 4 * hh);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 wp, wd;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float pv[2], dv_[2];
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        const int j = 8 * s + 2 * e2 + t2;
                        float p = __builtin_amdgcn_exp2f(fmaf(sacc[j], c2, kterm + nl[j / 4][j % 4]));
                        if constexpr (decltype(masked)::value) {
                            const int qloc = 8 * (j / 4) + 4 * hh + (j % 4);
                            const bool vis = key_ok & (qrow0 + qloc < n) & (p_key <= pq[j / 4][j % 4]);
                            p = vis ? p : 0.0f;
                        }
                        const float ds = p * (pacc[j] - dlq[j / 4][j % 4]);
                        db_acc += ds;
                        dt_acc = fmaf(ds, sacc[j], dt_acc);
                        pv[t2] = p;
                        dv_[t2] = ds;
                    }
                    wp[e2] = pack_bf16x2(pv[0], pv[1]);
                    wd[e2] = pack_bf16x2(dv_[0], dv_[1]);
                }
                pf[s] = __builtin_bit_cast(bf16x8, wp);
                dsf[s] = __builtin_bit_cast(bf16x8, wd);
            }
        };
        if (full)
            softmax(std::false_type{});
        else
            softmax(std::true_type{});
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                acc_dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[s], dotr[b][s], acc_dv[b], 0, 0, 0);
                acc_dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsf[s], qtr[b][s], acc_dk[b], 0, 0, 0);
            }
    }
    // Accumulator j of block b: key key0 + 8(j/4) + 4hh + j%4, d = 32b + l32.
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int kr = key0 + 8 * (j / 4) + 4 * hh + (j % 4);
            if (kr < n) {
                const int64_t o = (((int64_t)part * hq + h) * m + off + kr) * D + 32 * b + l32;
                ws_dk[o] = acc_dk[b][j] * c;
                ws_dv[o] = acc_dv[b][j];
            }
        }
    // sum_i dS_ij of this lane's key, over both query halves (the gain is
    // applied when the heads are summed).
    db_acc += __shfl_xor(db_acc, 32);
    dt_acc += __shfl_xor(dt_acc, 32);
    if (hh == 0 && key_ok) {
        ws_db[((int64_t)part * hq + h) * m + off + key] = db_acc;
        ws_dt[((int64_t)part * hq + h) * m + off + key] = dt_acc;
    }
}

// 3. dQ of one (prompt, query block, head).
template <int D>
__device__ __forceinline__ void bwd_dq_body(int item, LDS_AS char* kt, LDS_AS char* vt, LDS_AS float* s_kb,
                                            LDS_AS int32_t* s_p, const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const uint16_t* __restrict__ d_out, const float* __restrict__ lse,
                                                   const float* __restrict__ dl, const float* __restrict__ bias,
                                                   const int32_t* __restrict__ pos, BwdTable t, int hq, int hkv,
                                                   const float* __restrict__ gain, float c, float* __restrict__ dq) {
    constexpr int KS = D / 16, DB = D / 32;
    const int lane = threadIdx.x;
    const int hh = lane >> 5, l32 = lane & 31;
    int sg, ib, h, part;
    bwd_item(t, item, hq, true, sg, ib, h, part);  // late query blocks see the most keys
    const int64_t off = t.s[sg].off, m = t.m_total;
    const int n = t.s[sg].n;
    const int kvh = h / (hq / hkv);
    const int i0 = 32 * ib;
    const int qi = min(i0 + l32, n - 1);
    const bool q_ok = i0 + l32 < n;
    const float c2 = c * LOG2E, gb2 = gain[h] * LOG2E;
    const float nlse2 = -lse[(int64_t)h * m + off + qi] * LOG2E;
    const float dlq = dl[(int64_t)h * m + off + qi];
    const int32_t my_pos = pos[off + qi];
    const int32_t pos_last = pos[off + min(i0 + 31, n - 1)];
    // Lowest query position of the block, if the block is full: a full key
    // block whose last key is at or before it is visible to every query.
    const int32_t pos_first = i0 + 32 <= n ? pos[off + i0] : INT32_MIN;

    bf16x8 qf[KS], df[KS];
    {
        const uint16_t* qrow = q + ((off + qi) * hq + h) * D + 8 * hh;
        const uint16_t* drow = d_out + ((off + qi) * hq + h) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = *(const bf16x8*)(qrow + 16 * s);
            df[s] = *(const bf16x8*)(drow + 16 * s);
        }
    }
    // Key blocks up to the last one holding a key visible to this block.
    int n_kt = min(n - 1, i0 + 31) / 32 + 1;
    while (n_kt * 32 < n && pos[off + n_kt * 32] <= pos_last) ++n_kt;

    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[b][j] = 0.0f;

    // K / V tiles and the key scalars of block kb + 1 are fetched into
    // registers while block kb is processed.
    const uint16_t* ksrc = k + (off * hkv + kvh) * D;
    const uint16_t* vsrc = v + (off * hkv + kvh) * D;
    TileRegs<D> rk, rv;
    float n_kb = 0.0f;
    int32_t n_p = 0;
    auto fetch_kv = [&](int kb) __attribute__((always_inline)) {
        fetch_tile<D>(rk, ksrc, (int64_t)hkv * D, 32 * kb, n, lane);
        fetch_tile<D>(rv, vsrc, (int64_t)hkv * D, 32 * kb, n, lane);
        const int kr = 32 * kb + (lane & 31);
        n_kb = gb2 * bias[off + min(kr, n - 1)];
        n_p = (kr < n) ? pos[off + kr] : INT32_MAX;
    };
    // This item's half of the key blocks 0 .. n_kt - 1.
    const int half = t.parts == 1 ? n_kt : (n_kt + 1) / 2;
    const int lo = part == 0 ? 0 : half, hi = part == 0 ? half : n_kt;
    if (lo < hi) fetch_kv(lo);
    for (int kb = lo; kb < hi; ++kb) {
        __syncthreads();
        store_tile<D>((LDS_AS char*)kt, rk, lane);
        store_tile<D>((LDS_AS char*)vt, rv, lane);
        if (lane < 32) {
            s_kb[lane] = n_kb;
            s_p[lane] = n_p;
        }
        // Lane 31 holds the position of the block's last key (INT32_MAX past the end).
        const bool full = __builtin_amdgcn_readlane(n_p, 31) <= pos_first;
        __syncthreads();
        if (kb + 1 < hi) fetch_kv(kb + 1);
        f32x16 sacc, pacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            sacc[j] = 0.0f;
            pacc[j] = 0.0f;
        }
        bf16x8 kop[KS], vop[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kop[s] = tile_row_operand<D>((const LDS_AS char*)kt, s, lane);
            vop[s] = tile_row_operand<D>((const LDS_AS char*)vt, s, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s], qf[s], sacc, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[s], df[s], pacc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 ktr[DB][2];
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int s = 0; s < 2; ++s) ktr[b][s] = tile_tr_operand<D>((const LDS_AS char*)kt, b, s, lane);
        __builtin_amdgcn_sched_barrier(0);
        // Register j: key 32kb + 8(j/4) + 4hh + j%4 of query qi; the key
        // scalars of four consecutive keys come in one read.
        f32x4 kb4[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) kb4[g4] = *(const LDS_AS f32x4*)(s_kb + 8 * g4 + 4 * hh);
        bf16x8 dsf[2];
        auto softmax = [&](auto masked) __attribute__((always_inline)) {
            i32x4 pk[4];
            if constexpr (decltype(masked)::value) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) pk[g4] = *(const LDS_AS i32x4*)(s_p + 8 * g4 + 4 * hh);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 w;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float dv_[2];
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        const int j = 8 * s + 2 * e2 + t2;
                        float p = __builtin_amdgcn_exp2f(fmaf(sacc[j], c2, kb4[j / 4][j % 4] + nlse2));
                        if constexpr (decltype(masked)::value) p = (q_ok & (pk[j / 4][j % 4] <= my_pos)) ? p : 0.0f;
                        dv_[t2] = p * (pacc[j] - dlq);
                    }
                    w[e2] = pack_bf16x2(dv_[0], dv_[1]);
                }
                dsf[s] = __builtin_bit_cast(bf16x8, w);
            }
        };
        if (full)
            softmax(std::false_type{});
        else
            softmax(std::true_type{});
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktr[b][s], dsf[s], acc[b], 0, 0, 0);
    }
    // acc[b] register j: d = 32b + 8(j/4) + 4hh + j%4 of query qi.
    if (q_ok) {
        float* row = dq + (((int64_t)part * m + off + i0 + l32) * hq + h) * D;  // this part's partial
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = acc[b][4 * g4 + e] * c;
                *(f32x4*)(row + 32 * b + 8 * g4 + 4 * hh) = o;
            }
    }
}

// 2 + 3 in one launch: work item pairs alternate between the dkdv and dq
// passes (both in their longest-first orders), so one grid keeps the chip
// busy through both and neither pass's tail runs alone. The LDS of a
// workgroup is shared by the two bodies (one runs per workgroup).
template <int D>
__global__ __launch_bounds__(64) void bwd_main_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ d_out, const float* __restrict__ lse, const float* __restrict__ dl,
    const float* __restrict__ bias, const int32_t* __restrict__ pos, BwdTable t, int hq, int hkv,
    const float* __restrict__ gain, float c, float* __restrict__ ws_dk, float* __restrict__ ws_dv,
    float* __restrict__ ws_db, float* __restrict__ ws_dt, float* __restrict__ dq) {
    __shared__ __attribute__((aligned(16))) char tiles[4 * Tile<D>::BYTES];
    __shared__ __attribute__((aligned(16))) float sf[2][32];
    __shared__ __attribute__((aligned(16))) int32_t si[32];
    LDS_AS char* base = (LDS_AS char*)tiles;
    LDS_AS float* f0 = (LDS_AS float*)&sf[0][0];
    LDS_AS float* f1 = (LDS_AS float*)&sf[1][0];
    LDS_AS int32_t* i0 = (LDS_AS int32_t*)&si[0];
    constexpr int TB = Tile<D>::BYTES;
    const int item = (int)(blockIdx.x >> 1);
    if ((blockIdx.x & 1) == 0)
        bwd_dkdv_body<D>(item, base, base + TB, base + 2 * TB, base + 3 * TB, f0, f1, i0, q, k, v, d_out, lse, dl,
                         bias, pos, t, hq, hkv, gain, c, ws_dk, ws_dv, ws_db, ws_dt);
    else
        bwd_dq_body<D>(item, base, base + TB, f0, i0, q, k, v, d_out, lse, dl, bias, pos, t, hq, hkv, gain, c, dq);
}

// 4a. dK, dV = sums of the per-head partials over each KV head's query
// heads (in head order); db = sum over heads of g_h times the head's
// sum_i dS_ij.
template <int D>
__device__ __forceinline__ void bwd_reduce_body(int64_t idx, const float* __restrict__ ws_dk,
                                                        const float* __restrict__ ws_dv,
                                                        const float* __restrict__ ws_db,
                                                        const float* __restrict__ gain, int64_t m, int hq, int hkv,
                                                        int parts, float* __restrict__ dk, float* __restrict__ dv,
                                                        float* __restrict__ db) {
    const int gsz = hq / hkv;
    if (idx < m * hkv * D) {
        const int64_t row = idx / (hkv * D);
        const int kvh = (int)((idx / D) % hkv), d = (int)(idx % D);
        float a = 0.0f, b = 0.0f;
        for (int pt = 0; pt < parts; ++pt)
            for (int hl = 0; hl < gsz; ++hl) {
                const int64_t o = (((int64_t)pt * hq + kvh * gsz + hl) * m + row) * D + d;
                a += ws_dk[o];
                b += ws_dv[o];
            }
        dk[idx] = a;
        dv[idx] = b;
    }
    if (idx < m) {
        float s = 0.0f;
        for (int h = 0; h < hq; ++h) {
            float sh = 0.0f;
            for (int pt = 0; pt < parts; ++pt) sh += ws_db[((int64_t)pt * hq + h) * m + idx];
            s = fmaf(gain[h], sh, s);
        }
        db[idx] = s;
    }
}

// Fixed-order sum of one 1024-thread workgroup's values (a butterfly per
// wave, then the sixteen wave sums in order); valid in thread 0.
__device__ __forceinline__ float block_sum_1024(float v, float* part) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.0f;
    if (threadIdx.x == 0)
        for (int i = 0; i < 16; ++i) s += part[i];
    return s;
}

// dQ = the sum of its parts, in part order.
__device__ __forceinline__ void bwd_dq_sum_body(int64_t i, const float* __restrict__ ws_dq, int64_t n,
                                                float* __restrict__ dq) {
    if (i < n) dq[i] = ws_dq[i] + ws_dq[n + i];
}

// 4b. Workgroup h < hq: dg_h = sum_j b_j sum_i dS_ij over all kept rows.
// Workgroup hq: dtau = -(c/tau) times the sum of the per-key, per-head sums
// of dS_ij (q_i . k_j) over every part. Each thread keeps four loads in
// flight; the summation order is fixed.
__device__ __forceinline__ void bwd_scalars_body(int h, float* part, const float* __restrict__ ws_db,
                                                 const float* __restrict__ bias, int64_t m, int hq, int parts,
                                                 const float* __restrict__ ws_dt, float dtau_scale,
                                                 float* __restrict__ dgain, float* __restrict__ dtau) {
    const bool gain_wg = h < hq;
    const float* x = gain_wg ? ws_db + (int64_t)h * m : ws_dt;
    const int64_t len = gain_wg ? m : (int64_t)parts * hq * m;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t j0 = threadIdx.x; j0 < len; j0 += 4 * 1024) {
        float xv[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = j0 + (int64_t)u * 1024;
            float xs = 0.0f;
            if (j < len) {
                xs = x[j];
                if (gain_wg)  // the other parts of the head's sum_i dS row
                    for (int pt = 1; pt < parts; ++pt) xs += x[(int64_t)pt * hq * m + j];
            }
            xv[u] = xs;
            bv[u] = (gain_wg && j < len) ? bias[j] : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = fmaf(bv[u], xv[u], acc[u]);
    }
    const float tot = block_sum_1024((acc[0] + acc[1]) + (acc[2] + acc[3]), part);
    if (threadIdx.x == 0) {
        if (gain_wg)
            dgain[h] = tot;
        else
            *dtau = dtau_scale * tot;
    }
}

// 4 in one launch of 1024-thread workgroups: workgroups 0 .. hq the
// scalars (the longest, latency-bound sums, first), then the reduction of
// dK / dV / db, then (split items only) the dQ part sums.
template <int D>
__global__ __launch_bounds__(1024) void bwd_post_kernel(const float* __restrict__ ws_dk, const float* __restrict__ ws_dv,
                                                       const float* __restrict__ ws_db, const float* __restrict__ gain,
                                                       int64_t m, int hq, int hkv, int parts, float* __restrict__ dk,
                                                       float* __restrict__ dv, float* __restrict__ db,
                                                       const float* __restrict__ bias, const float* __restrict__ ws_dt,
                                                       float dtau_scale, float* __restrict__ dgain,
                                                       float* __restrict__ dtau, int n_red,
                                                       const float* __restrict__ ws_dq, float* __restrict__ dq) {
    __shared__ float part[16];
    const int b = (int)blockIdx.x;
    if (b <= hq) {
        bwd_scalars_body(b, part, ws_db, bias, m, hq, parts, ws_dt, dtau_scale, dgain, dtau);
    } else if (b <= hq + n_red) {
        bwd_reduce_body<D>((int64_t)(b - hq - 1) * 1024 + threadIdx.x, ws_dk, ws_dv, ws_db, gain, m, hq, hkv, parts,
                           dk, dv, db);
    } else {
        bwd_dq_sum_body((int64_t)(b - hq - 1 - n_red) * 1024 + threadIdx.x, ws_dq, m * hq * D, dq);
    }
}

template <int D>
hipError_t launch_bwd_d(const AttnBwdArgs& a, const BwdTable& t, float c, hipStream_t st) {
    const int64_t m = t.m_total;
    float* ws = (float*)a.workspace;
    float* dl = ws;
    const int np = t.parts;
    float* ws_dk = dl + (int64_t)a.hq * m;
    float* ws_dv = ws_dk + (int64_t)np * a.hq * m * D;
    float* ws_db = ws_dv + (int64_t)np * a.hq * m * D;
    float* ws_dt = ws_db + (int64_t)np * a.hq * m;
    float* ws_dq = ws_dt + (int64_t)np * a.hq * m;  // split: the dq parts; else dq is written directly
    const uint16_t *q = (const uint16_t*)a.q, *k = (const uint16_t*)a.k, *v = (const uint16_t*)a.v;
    const uint16_t *dout = (const uint16_t*)a.d_out, *out = (const uint16_t*)a.out;
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((m * a.hq + 255) / 256)), dim3(256), 0, st, dout, out, m,
                       a.hq, dl);
    hipLaunchKernelGGL((bwd_main_kernel<D>), dim3((unsigned)(2 * t.n_items)), dim3(64), 0, st, q, k, v, dout, a.lse,
                       dl, a.bias, a.pos, t, a.hq, a.hkv, a.gain, c, ws_dk, ws_dv, ws_db, ws_dt,
                       np > 1 ? ws_dq : a.d_q);
    const int n_red = (int)((m * a.hkv * D + 1023) / 1024);
    const int n_sum = np > 1 ? (int)((m * a.hq * D + 1023) / 1024) : 0;
    hipLaunchKernelGGL((bwd_post_kernel<D>), dim3((unsigned)(a.hq + 1 + n_red + n_sum)), dim3(1024), 0, st, ws_dk,
                       ws_dv, ws_db, a.gain, m, a.hq, a.hkv, np, a.d_k, a.d_v, a.d_bias, a.bias, ws_dt, -c / a.tau,
                       a.d_gain, a.d_tau, n_red, ws_dq, a.d_q);
    return hipGetLastError();
}

}  // namespace

size_t attention_backward_plan(const SeqTable& st, int hq, int hkv, int head_dim, void* table_out) {
    BwdTable& t = *(BwdTable*)table_out;
    t = BwdTable{};
    t.n_seg = st.n;
    int64_t blocks = 0;
    for (int b = 0; b < st.n; ++b) blocks += (st.s[b].n_kept + 31) / 32;
    t.parts = blocks * hq < BWD_SPLIT_BELOW ? 2 : 1;
    int64_t items = 0, m = 0;
    for (int b = 0; b < st.n; ++b) {
        t.s[b].off = st.s[b].kept_off;
        t.s[b].n = st.s[b].n_kept;
        t.s[b].n_blk = (st.s[b].n_kept + 31) / 32;
        t.s[b].item0 = (int32_t)items;
        items += (int64_t)t.s[b].n_blk * hq * t.parts;
        m += st.s[b].n_kept;
    }
    t.n_items = (int32_t)items;
    t.m_total = m;
    // Dl [hq][M]; per part: dk and dv partials [hq][M][D], sum_i dS and
    // sum_i dS (q . k) partials [hq][M] each; when split, dq partials
    // [parts][M][hq][D].
    (void)hkv;
    const size_t per_part = (size_t)hq * m * (2 * (size_t)head_dim + 2);
    const size_t dq_parts = t.parts > 1 ? (size_t)t.parts * hq * m * head_dim : 0;
    return ((size_t)hq * m + t.parts * per_part + dq_parts) * sizeof(float);
}

size_t attention_backward_table_bytes() { return sizeof(BwdTable); }

hipError_t launch_attention_backward(const AttnBwdArgs& a, const void* table, hipStream_t st) {
    const BwdTable& t = *(const BwdTable*)table;
    if (t.n_items == 0) return hipSuccess;
    const float c = 1.0f / (sqrtf((float)a.head_dim) * a.tau);
    return a.head_dim == 128 ? launch_bwd_d<128>(a, t, c, st) : launch_bwd_d<64>(a, t, c, st);
}

// Score gradient: zero every row, then d_scores[kept_idx[m]] = d_bias[m] *
// sigmoid(-s) for kept document rows.
namespace {
__global__ __launch_bounds__(256) void score_zero_kernel(float* __restrict__ d, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) d[i] = 0.0f;
}
__global__ __launch_bounds__(256) void score_grad_kernel(const float* __restrict__ d_bias,
                                                        const float* __restrict__ scores,
                                                        const int32_t* __restrict__ kept, SeqTable t,
                                                        float* __restrict__ d_scores) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int b = 0;
    for (int s = 1; s < t.n; ++s)
        if (t.s[s].kept_off <= i) b = s;
    const SeqDesc sd = t.s[b];
    if (i >= sd.kept_off + sd.n_kept) return;  // past the last prompt
    const int32_t row = kept[i];
    const int64_t rel = row - sd.start;
    if (rel >= sd.doc_begin && rel < sd.doc_end) {
        const float s = scores[row];
        // sigmoid(-s), without overflow for large |s|
        const float e = __expf(-fabsf(s));
        d_scores[row] = d_bias[i] * (s >= 0.0f ? e / (1.0f + e) : 1.0f / (1.0f + e));
    }
}
}  // namespace

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st) {
    if (n > 0) hipLaunchKernelGGL(score_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_score_grad(const float* d_bias, const float* scores, const int32_t* kept, const SeqTable& t,
                             int64_t m, int64_t n_rows, float* d_scores, hipStream_t st) {
    if (n_rows > 0)
        hipLaunchKernelGGL(score_zero_kernel, dim3((unsigned)((n_rows + 255) / 256)), dim3(256), 0, st, d_scores,
                           n_rows);
    if (m > 0)
        hipLaunchKernelGGL(score_grad_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, d_bias, scores,
                           kept, t, d_scores);
    return hipGetLastError();
}

}  // namespace tg
