// Gated delta rule over the kept rows: the token mixer of a Gated-DeltaNet
// layer above (or at) the gate, run on the kept tokens only.
//
// Defined by the TokenGate pages: ai4bro.com post, section on
// hybrid-attention models; spke.com article, section on hybrid attention;
// ai.info news, section on hybrid models (the gate also prunes at the
// Gated-DeltaNet layers of the Qwen3.5 hybrid, which the next-best pruning
// method cannot). The gated delta rule, per prompt and head, over the kept
// rows in order:
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
// with a_t = exp(g_t) and the state S [dv, dk].
//
// Chunked form (64 rows per chunk; G_t = sum of g over the chunk up to and
// including t, S_0 the state entering the chunk): with
//     L_ts = b_t exp(G_t - G_s) k_t.k_s (s < t),  T = (I + L)^-1 diag(b),
//     U = T V,  Y = T diag(exp(G)) K,  P_ts = exp(G_t - G_s) q_t.k_s (s <= t),
// the chunk's new values are W = U - Y S_0^T, its outputs
//     O = diag(exp(G)) Q S_0^T + P W,
// and the state after it S = exp(G_last) S_0 + W^T diag(exp(G_last - G)) K.
// (By induction, S_t = exp(G_t) S_0 + sum_{s<=t} exp(G_t - G_s) w_s k_s^T
// with w_t = b_t (v_t - a_t S_{t-1} k_t); substituting gives (I + L) W =
// diag(b) (V - diag(exp(G)) K S_0^T).) Rows past a prompt's end are padded
// with b = g = 0, which makes their w zero.
//
// Kernels:
//  * delta_prep_kernel: one workgroup per (chunk, head), independent of the
//    state, so all chunks run at once: K K^T and Q K^T on bf16 MFMA, L and
//    P, the triangular solve for T in fp32 (one wave, a column per lane),
//    then U = T V and Y = T diag(exp(G)) K on bf16 MFMA; U is kept in fp32,
//    Y and P in bf16 for the MFMAs of the next kernel.
//  * delta_scan_kernel: one workgroup of four waves per (prompt, head, 32
//    state rows), walking the chunks in order on 32x32x16 bf16 MFMA with the
//    state in fp32 registers (32 key columns per wave): W = U - Y S^T,
//    O = diag(exp(G)) Q S^T + P W, and S = exp(G_last) S + (diag(e) W)^T K
//    with K read transposed from LDS; W goes through LDS transposed, read
//    in the permuted row order of the other operand of each product.
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

constexpr int DC = 64;   // rows per chunk
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int DD = 128;  // dk = dv

__device__ __forceinline__ uint16_t f2bf(float x) { return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xffffu); }

// Chunk c of the whole call -> (prompt, first kept row, rows in the chunk).
__device__ __forceinline__ void delta_chunk(const SeqTable& t, int c, int& sg, int64_t& row0, int& len,
                                            int& c_in) {
    int base = 0;
    sg = 0;
    for (int i = 0; i < t.n; ++i) {
        const int nc = (t.s[i].n_kept + DC - 1) / DC;
        if (c < base + nc) {
            sg = i;
            break;
        }
        base += nc;
    }
    c_in = c - base;
    row0 = t.s[sg].kept_off + (int64_t)c_in * DC;
    len = min(DC, t.s[sg].n_kept - c_in * DC);
}

// Per (chunk, head) workspace record.
struct DeltaRec {
    static constexpr size_t U = 0;                          // fp32 [64][128]
    static constexpr size_t Y = U + DC * DD * 4;            // bf16 [64][128]
    static constexpr size_t P = Y + DC * DD * 2;            // bf16 [64][64]
    static constexpr size_t GAM = P + DC * DC * 2;          // fp32 [64]: exp(G_t)
    static constexpr size_t E = GAM + DC * 4;               // fp32 [64]: exp(G_last - G_t)
    static constexpr size_t BYTES = E + DC * 4;
};

__device__ __forceinline__ int sw16(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
__device__ __forceinline__ int sw8(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// B operand from a swizzled 256-byte-row tile (16-byte chunk c of row r at
// c ^ (r % 16)): column 32b + lane%32, k-slots = tile rows 16s + 8(e/4) +
// 4(lane/32) + e%4.
__device__ __forceinline__ bf16x8 k_tr_operand(const LDS_AS char* tile, int b, int s, int lane) {
    const int gq = lane >> 4, r16 = lane & 15;
    const int ra = 16 * s + 4 * (gq >> 1) + (r16 >> 2);
    const int col = 32 * b + 16 * (gq & 1) + 4 * (r16 & 3);  // element; chunk col / 8, half (col % 8) / 4
    const int off = ((col & 7) >> 2) * 8;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(tile + sw16(ra, col >> 3) + off));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(tile + sw16(ra + 8, col >> 3) + off));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Per (chunk, head), 4 waves. K K^T and Q K^T on MFMA (operands straight
// from memory; wave w takes the 32 x 32 tile (w/2, w%2)), then L and P; the
// triangular solve for T in one wave (lane c holds column c in registers);
// U = T V and Y = T diag(exp(G)) K on MFMA (A = T rows in the permuted k
// order of the transpose reads of V and K; wave w takes 32 rows x 64
// columns). Accumulator layout: row 8(r/4) + 4hh + r%4 of the tile, column
// lane%32.
__global__ __launch_bounds__(256) void delta_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, const float* __restrict__ g,
                                                         const float* __restrict__ beta, SeqTable t, int nh,
                                                         char* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) char kt[DC * DD * 2], vt[DC * DD * 2];  // swizzled rows
    __shared__ __attribute__((aligned(16))) float lm[DC][DC + 4], tm[DC][DC + 4];
    __shared__ float gc[DC], bl[DC];
    __shared__ __attribute__((aligned(16))) float gm[DC];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int chunk = blockIdx.x, h = blockIdx.y;
    int sg, len, c_in;
    int64_t row0;
    delta_chunk(t, chunk, sg, row0, len, c_in);
    auto grow = [&](int r) __attribute__((always_inline)) { return ((row0 + min(r, len - 1)) * nh + h) * DD; };
    // K and V tiles (bf16) into LDS; rows past the chunk repeat its last row
    // (their beta is 0, so they never contribute).
    for (int idx = tid; idx < DC * DD / 8; idx += 256) {
        const int r = idx >> 4, cc = idx & 15;
        *(LDS_AS u32x4*)(kt + sw16(r, cc)) = *(const u32x4*)(k + grow(r) + cc * 8);
        *(LDS_AS u32x4*)(vt + sw16(r, cc)) = *(const u32x4*)(v + grow(r) + cc * 8);
    }
    if (tid < DC) {
        const bool in = tid < len;
        const int64_t o = (row0 + min(tid, len - 1)) * nh + h;
        float x = in ? g[o] : 0.0f;
        bl[tid] = in ? beta[o] : 0.0f;
        // inclusive prefix sum of g over the chunk (one wave)
#pragma unroll
        for (int d = 1; d < DC; d <<= 1) {
            const float y = __shfl_up(x, d);
            if (tid >= d) x += y;
        }
        gc[tid] = x;
        gm[tid] = __expf(x);
    }
    // K K^T and Q K^T: tile (tm_, tn_) of wave w.
    const int tm_ = wave >> 1, tn_ = wave & 1;
    f32x16 kk, qk;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        kk[r] = 0.0f;
        qk[r] = 0.0f;
    }
    {
        const uint16_t* ka = k + grow(32 * tm_ + l32) + 8 * hh;
        const uint16_t* qa = q + grow(32 * tm_ + l32) + 8 * hh;
        const uint16_t* kb = k + grow(32 * tn_ + l32) + 8 * hh;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
            const bf16x8 a1 = *(const bf16x8*)(ka + 16 * s2), a2 = *(const bf16x8*)(qa + 16 * s2);
            const bf16x8 b1 = *(const bf16x8*)(kb + 16 * s2);
            kk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, kk, 0, 0, 0);
            qk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b1, qk, 0, 0, 0);
        }
    }
    __syncthreads();  // gc, bl, gm and the tiles are ready
    char* rec = ws + ((size_t)chunk * nh + h) * DeltaRec::BYTES;
    uint16_t* prec = (uint16_t*)(rec + DeltaRec::P);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int rr = 32 * tm_ + 8 * (r >> 2) + 4 * hh + (r & 3), ss = 32 * tn_ + l32;
        const float dec = ss <= rr ? __expf(gc[rr] - gc[ss]) : 0.0f;
        lm[rr][ss] = ss < rr ? bl[rr] * dec * kk[r] : 0.0f;
        prec[rr * DC + ss] = f2bf(dec * qk[r]);
    }
    __syncthreads();
    // T = (I + L)^-1 diag(b), row by row: one wave, lane c holds column c of
    // T in registers (fully unrolled; the row entries of L are the same for
    // every lane, two partial sums shorten the dependence chain).
    if (tid < DC) {
        const int c = tid;
        float tcol[DC];
#pragma unroll
        for (int r = 0; r < DC; ++r) {
            float x0 = r == c ? bl[r] : 0.0f, x1 = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 + 1 < r; s2 += 2) {
                x0 = fmaf(-lm[r][s2], tcol[s2], x0);
                x1 = fmaf(-lm[r][s2 + 1], tcol[s2 + 1], x1);
            }
            if (r & 1) x0 = fmaf(-lm[r][r - 1], tcol[r - 1], x0);
            tcol[r] = x0 + x1;
        }
#pragma unroll
        for (int r = 0; r < DC; ++r) tm[r][c] = tcol[r];
    }
    __syncthreads();
    // U = T V and Y = T diag(exp(G)) K: wave w takes rows 32 (w/2) .. +32 and
    // columns 64 (w%2) .. +64 (two 32-column tiles).
    float* urec = (float*)(rec + DeltaRec::U);
    uint16_t* yrec = (uint16_t*)(rec + DeltaRec::Y);
    const int ur = 32 * (wave >> 1) + l32;  // this lane's A-operand row of T
    bf16x8 ta[4], tg[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        // k-slots (hh, e) <-> T columns 16 s2 + 8(e/4) + 4hh + e%4
        const f32x4 lo = *(const LDS_AS f32x4*)(&tm[ur][16 * s2 + 4 * hh]);
        const f32x4 hi = *(const LDS_AS f32x4*)(&tm[ur][16 * s2 + 8 + 4 * hh]);
        const f32x4 glo = *(const LDS_AS f32x4*)(&gm[16 * s2 + 4 * hh]);
        const f32x4 ghi = *(const LDS_AS f32x4*)(&gm[16 * s2 + 8 + 4 * hh]);
        const u32x4 w1 = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                          pack_bf16x2(hi[2], hi[3])};
        const u32x4 w2 = {pack_bf16x2(lo[0] * glo[0], lo[1] * glo[1]), pack_bf16x2(lo[2] * glo[2], lo[3] * glo[3]),
                          pack_bf16x2(hi[0] * ghi[0], hi[1] * ghi[1]), pack_bf16x2(hi[2] * ghi[2], hi[3] * ghi[3])};
        ta[s2] = __builtin_bit_cast(bf16x8, w1);
        tg[s2] = __builtin_bit_cast(bf16x8, w2);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int ct = 2 * (wave & 1) + cb;  // 32-column tile
        f32x16 ua, ya;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ua[r] = 0.0f;
            ya[r] = 0.0f;
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            ua = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[s2], k_tr_operand((const LDS_AS char*)vt, ct, s2, lane), ua,
                                                         0, 0, 0);
            ya = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tg[s2], k_tr_operand((const LDS_AS char*)kt, ct, s2, lane), ya,
                                                         0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = 32 * (wave >> 1) + 8 * (r >> 2) + 4 * hh + (r & 3);
            urec[rr * DD + 32 * ct + l32] = ua[r];
            yrec[rr * DD + 32 * ct + l32] = f2bf(ya[r]);
        }
    }
    if (tid < DC) {
        ((float*)(rec + DeltaRec::GAM))[tid] = gm[tid];
        ((float*)(rec + DeltaRec::E))[tid] = __expf(gc[DC - 1] - gc[tid]);
    }
}

// LDS stage of one chunk for the scan kernel: Y, Q and K rows (256-byte
// rows, 16-byte chunk c of row r at c ^ (r % 16)), P rows (128-byte rows,
// chunk c at c ^ (r % 8)), the state-row block of U (64 x 32 fp32) and
// exp(G), e (64 fp32 each).
struct DeltaStage {
    static constexpr int Y = 0, Q = Y + DC * DD * 2, K = Q + DC * DD * 2, P = K + DC * DD * 2;
    static constexpr int U = P + DC * DC * 2, GAM = U + DC * 32 * 4, E = GAM + DC * 4, BYTES = E + DC * 4;
};
// One workgroup of four waves per (prompt, head, 32 state rows i0 .. +32):
// the chunks in order, the state rows on the lanes; the next chunk's
// operands stream into the other half of a two-stage LDS ring (direct
// loads, a quarter per wave) while a chunk runs. Per chunk:
//   A: waves 0, 1: W tile tt = U - Y S^T, written transposed to LDS (plain
//      and scaled by e); waves 2, 3: O tile tt = diag(gam) Q S^T.
//   B: waves 2, 3: O += P W, stored; every wave: its 32 key columns of
//      S = e_last S + (diag(e) W)^T K, written back (bf16) for the next A.
// Accumulator layouts: W, O tile tt: chunk row 32tt + 8(r/4) + 4hh + r%4,
// state row i0 + lane%32; S tile jt: state row i0 + 8(r/4) + 4hh + r%4, key
// column 32jt + lane%32. W^T in LDS is read in the permuted chunk-row order
// of the transpose reads of K and of the P column reads.
constexpr int WTS = 72;  // W^T row stride (bf16): 144-byte rows spread 32 rows over the banks

__global__ __launch_bounds__(256) void delta_scan_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k, SeqTable t, int nh,
                                                         const char* __restrict__ ws, const float* __restrict__ state_in,
                                                         uint16_t* __restrict__ out, float* __restrict__ state_out) {
    __shared__ __attribute__((aligned(1024))) char stage[2][DeltaStage::BYTES];
    __shared__ __attribute__((aligned(16))) char st[32 * DD * 2];     // S rows (bf16), row-major
    __shared__ __attribute__((aligned(16))) char wtt[32 * WTS * 2];   // W^T (bf16)
    __shared__ __attribute__((aligned(16))) char wse[32 * WTS * 2];   // (diag(e) W)^T (bf16)
    const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (load bases live in SGPRs)
    const int sg = blockIdx.x, h = blockIdx.y, i0 = 32 * blockIdx.z;
    int c0 = 0;
    for (int i = 0; i < sg; ++i) c0 += (t.s[i].n_kept + DC - 1) / DC;
    const int n_chunks = (t.s[sg].n_kept + DC - 1) / DC;

    // Direct loads of chunk c into stage b, this wave's quarter: loads 4w ..
    // 4w+3 of the Y, Q and K tiles (256-byte rows, 4 rows per load), 2w,
    // 2w+1 of the P and U tiles (128-byte rows, 8 rows per load), and exp(G)
    // (wave 0) or e (wave 1). Each from a wave-uniform base plus a fixed
    // per-lane offset: load ins takes row 4 ins + l/16 and the logical chunk
    // (l%16) ^ (row%16), which depends on ins only through ins % 4 = j.
    uint32_t oy[4], oq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int lc = (lane & 15) ^ ((4 * j + (lane >> 4)) & 15);
        oy[j] = (uint32_t)((lane >> 4) * 256 + lc * 16);
        oq[j] = (uint32_t)((lane >> 4) * nh * 256 + lc * 16);
    }
    const uint32_t op = (uint32_t)((lane >> 3) * 128 + (((lane & 7) ^ ((lane >> 3) & 7)) * 16));
    const uint32_t ou = (uint32_t)((lane >> 3) * DD * 4 + i0 * 4 + (lane & 7) * 16);
    const uint32_t o4 = (uint32_t)(lane * 4);
    auto issue = [&](int c, int b) __attribute__((always_inline)) {
        const int64_t row0 = t.s[sg].kept_off + (int64_t)c * DC;
        const int len = min(DC, t.s[sg].n_kept - c * DC);
        const char* rec = ws + ((size_t)(c0 + c) * nh + h) * DeltaRec::BYTES;
        const uint32_t sb = LDS_ADDR(stage[b]);
        const char* qb = (const char*)(q + (row0 * nh + h) * DD);
        const char* kb = (const char*)(k + (row0 * nh + h) * DD);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ins = 4 * wave + j;
            dma16_so(rec + DeltaRec::Y + ins * 1024, oy[j], sb + DeltaStage::Y + ins * 1024);
            if (len == DC) {
                dma16_so(qb + (size_t)ins * 4 * nh * 256, oq[j], sb + DeltaStage::Q + ins * 1024);
                dma16_so(kb + (size_t)ins * 4 * nh * 256, oq[j], sb + DeltaStage::K + ins * 1024);
            } else {  // the prompt's last, partial chunk: rows past its end repeat its last row
                const int row = ins * 4 + (lane >> 4);
                const int lc = (lane & 15) ^ (row & 15);
                const uint32_t o = (uint32_t)(min(row, len - 1) * nh * 256 + lc * 16);
                dma16_so(qb, o, sb + DeltaStage::Q + ins * 1024);
                dma16_so(kb, o, sb + DeltaStage::K + ins * 1024);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ins = 2 * wave + j;
            dma16_so(rec + DeltaRec::P + ins * 1024, op, sb + DeltaStage::P + ins * 1024);
            dma16_so(rec + DeltaRec::U + ins * 8 * DD * 4, ou, sb + DeltaStage::U + ins * 1024);
        }
        if (wave == 0) dma4_so(rec + DeltaRec::GAM, o4, sb + DeltaStage::GAM);
        if (wave == 1) dma4_so(rec + DeltaRec::E, o4, sb + DeltaStage::E);
    };

    // This wave's 32 key columns of the state (fp32), and their bf16 copy.
    const int jt = wave;
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        sacc[r] = state_in ? state_in[(((int64_t)sg * nh + h) * DD + i) * DD + 32 * jt + l32] : 0.0f;
    }
    auto put_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int il = 8 * (r >> 2) + 4 * hh + (r & 3);
            *(LDS_AS uint16_t*)(st + (il * DD + 32 * jt + l32) * 2) = f2bf(sacc[r]);
        }
    };
    put_state();
    if (n_chunks > 0) issue(0, 0);
    for (int c = 0; c < n_chunks; ++c) {
        const int64_t row0 = t.s[sg].kept_off + (int64_t)c * DC;
        const int len = min(DC, t.s[sg].n_kept - c * DC);
        const LDS_AS char* sb = (const LDS_AS char*)stage[c & 1];
        wait_vmcnt<0>();  // this wave's loads of chunk c (and its earlier stores) are done
        ring_barrier();   // ... every wave's; the other stage and W^T are free again
        if (c + 1 < n_chunks) issue(c + 1, (c + 1) & 1);

        // A: S rows as the B operand (lane = state row, k = key column).
        bf16x8 sop[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
            sop[s2] = *(const LDS_AS bf16x8*)(st + (l32 * DD + 16 * s2 + 8 * hh) * 2);
        const float* gam = (const float*)(sb + DeltaStage::GAM);
        const float* ee = (const float*)(sb + DeltaStage::E);
        const int tt = wave & 1;
        const int rr = 32 * tt + l32;  // this lane's A-operand chunk row
        const int src = wave < 2 ? DeltaStage::Y : DeltaStage::Q;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
            const bf16x8 ab = *(const LDS_AS bf16x8*)(sb + src + sw16(rr, 2 * s2 + hh));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, sop[s2], acc, 0, 0, 0);
        }
        if (wave < 2) {
            // W = U - Y S^T, stored transposed (plain and scaled by e), pairs of rows.
            const float* us = (const float*)(sb + DeltaStage::U);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int tr = 32 * tt + 8 * (r >> 2) + 4 * hh + (r & 3);
                const float w0 = us[tr * 32 + l32] - acc[r], w1 = us[(tr + 1) * 32 + l32] - acc[r + 1];
                *(LDS_AS uint32_t*)(wtt + (l32 * WTS + tr) * 2) = pack_bf16x2(w0, w1);
                *(LDS_AS uint32_t*)(wse + (l32 * WTS + tr) * 2) = pack_bf16x2(w0 * ee[tr], w1 * ee[tr + 1]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] *= gam[32 * tt + 8 * (r >> 2) + 4 * hh + (r & 3)];
        }
        ring_barrier();  // W^T is complete; every wave's reads of the state copy are done

        // B operands from W^T: lane = state row, k-slots (hh, e) = chunk rows
        // 16 s2 + 8(e/4) + 4hh + e%4.
        auto wt_operand = [&](const char* base, int s2) __attribute__((always_inline)) {
            const LDS_AS char* rowp = (const LDS_AS char*)(base) + (l32 * WTS + 16 * s2 + 4 * hh) * 2;
            const u32x2 lo = *(const LDS_AS u32x2*)rowp, hi = *(const LDS_AS u32x2*)(rowp + 16);
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            return __builtin_bit_cast(bf16x8, w);
        };
        if (wave >= 2) {
            // O += P W; store the chunk's own rows.
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int e0 = 16 * s2 + 4 * hh, e1 = e0 + 8;
                const u32x2 lo = *(const LDS_AS u32x2*)(sb + DeltaStage::P + sw8(rr, e0 >> 3) + (e0 & 7) * 2);
                const u32x2 hi = *(const LDS_AS u32x2*)(sb + DeltaStage::P + sw8(rr, e1 >> 3) + (e1 & 7) * 2);
                const u32x4 pw = {lo[0], lo[1], hi[0], hi[1]};
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pw), wt_operand(wtt, s2), acc,
                                                              0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tr = 32 * tt + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (tr < len) out[((row0 + tr) * nh + h) * DD + i0 + l32] = f2bf(acc[r]);
            }
        }
        // S (this wave's key columns) = e_last S + (diag(e) W)^T K.
        const float elast = gam[DC - 1];
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] *= elast;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wt_operand(wse, s2), k_tr_operand(sb + DeltaStage::K, jt, s2, lane),
                                                           sacc, 0, 0, 0);
        put_state();
    }
    wait_vmcnt<0>();
    if (state_out) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            state_out[(((int64_t)sg * nh + h) * DD + i) * DD + 32 * jt + l32] = sacc[r];
        }
    }
}

}  // namespace

size_t delta_scan_workspace_bytes(const SeqTable& t, int nh) {
    int64_t chunks = 0;
    for (int i = 0; i < t.n; ++i) chunks += (t.s[i].n_kept + DC - 1) / DC;
    return (size_t)chunks * nh * DeltaRec::BYTES;
}

hipError_t launch_delta_scan(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const SeqTable& t, int nh, const float* state_in, void* out, float* state_out,
                             void* workspace, hipStream_t st) {
    int64_t chunks = 0;
    for (int i = 0; i < t.n; ++i) chunks += (t.s[i].n_kept + DC - 1) / DC;
    if (chunks > 0)
        hipLaunchKernelGGL(delta_prep_kernel, dim3((unsigned)chunks, (unsigned)nh), dim3(256), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, beta, t, nh,
                           (char*)workspace);
    if (t.n > 0)
        hipLaunchKernelGGL(delta_scan_kernel, dim3((unsigned)t.n, (unsigned)nh, DD / 32), dim3(256), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, t, nh, (const char*)workspace, state_in,
                           (uint16_t*)out, state_out);
    return hipGetLastError();
}

}  // namespace tg
