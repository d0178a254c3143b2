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
//    state, so all chunks run at once: L, the triangular solve for T (one
//    wave, row by row), U, Y and P in fp32; U is kept in fp32, Y and P in
//    bf16 for the MFMAs of the next kernel.
//  * delta_scan_kernel: one wave per (prompt, head, 32 state rows), walking
//    the chunks in order on 32x32x16 bf16 MFMA with the state in fp32
//    registers: W = U - Y S^T, O = diag(exp(G)) Q S^T + P W, and
//    S = exp(G_last) S + (diag(e) W)^T K with K read transposed from LDS.
//    W's registers feed the next two products directly (the row order
//    inside each 16-wide k step is permuted the same way on both operands).
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

constexpr int DC = 64;   // rows per chunk
constexpr int DD = 128;  // dk = dv

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
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

__global__ __launch_bounds__(256) void delta_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, const float* __restrict__ g,
                                                         const float* __restrict__ beta, SeqTable t, int nh,
                                                         char* __restrict__ ws) {
    __shared__ float ks[DC][DD + 1], qs[DC][DD + 1], vs[DC][DD + 1];
    __shared__ float lm[DC][DC + 1], tm[DC][DC + 1];
    __shared__ float gc[DC], bl[DC];
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x, h = blockIdx.y;
    int sg, len, c_in;
    int64_t row0;
    delta_chunk(t, chunk, sg, row0, len, c_in);
    for (int idx = tid; idx < DC * DD; idx += 256) {
        const int r = idx / DD, c = idx % DD;
        const int64_t o = ((row0 + min(r, len - 1)) * nh + h) * DD + c;
        const bool in = r < len;
        ks[r][c] = in ? bf2f(k[o]) : 0.0f;
        qs[r][c] = in ? bf2f(q[o]) : 0.0f;
        vs[r][c] = in ? bf2f(v[o]) : 0.0f;
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
    }
    __syncthreads();
    // L (strictly lower) and P (lower with the diagonal), 16 entries per thread.
    char* rec = ws + ((size_t)chunk * nh + h) * DeltaRec::BYTES;
    uint16_t* prec = (uint16_t*)(rec + DeltaRec::P);
    for (int idx = tid; idx < DC * DC; idx += 256) {
        const int r = idx / DC, s = idx % DC;
        float kk = 0.0f, qk = 0.0f;
        if (s <= r) {
#pragma unroll 8
            for (int c = 0; c < DD; ++c) {
                kk = fmaf(ks[r][c], ks[s][c], kk);
                qk = fmaf(qs[r][c], ks[s][c], qk);
            }
        }
        const float dec = s <= r ? __expf(gc[r] - gc[s]) : 0.0f;
        lm[r][s] = s < r ? bl[r] * dec * kk : 0.0f;
        prec[r * DC + s] = f2bf(dec * qk);
    }
    __syncthreads();
    // T = (I + L)^-1 diag(b), row by row (one wave; lane c holds column c).
    if (tid < DC) {
        const int c = tid;
        for (int r = 0; r < DC; ++r) {
            float x = r == c ? bl[r] : 0.0f;
            for (int s = c; s < r; ++s) x = fmaf(-lm[r][s], tm[s][c], x);
            tm[r][c] = x;  // read back by this wave only, in order
        }
    }
    __syncthreads();
    // U = T V (fp32) and Y = T diag(exp(G)) K (bf16), 32 entries each per thread.
    float* urec = (float*)(rec + DeltaRec::U);
    uint16_t* yrec = (uint16_t*)(rec + DeltaRec::Y);
    for (int idx = tid; idx < DC * DD; idx += 256) {
        const int r = idx / DD, c = idx % DD;
        float u = 0.0f, y = 0.0f;
        for (int s = 0; s <= r; ++s) {
            const float ts = tm[r][s];
            u = fmaf(ts, vs[s][c], u);
            y = fmaf(ts * __expf(gc[s]), ks[s][c], y);
        }
        urec[idx] = u;
        yrec[idx] = f2bf(y);
    }
    if (tid < DC) {
        ((float*)(rec + DeltaRec::GAM))[tid] = __expf(gc[tid]);
        ((float*)(rec + DeltaRec::E))[tid] = __expf(gc[DC - 1] - gc[tid]);
    }
}

// B operand of a 32x32x16 MFMA from an LDS tile of bf16 rows with the given
// byte stride: column 32b + lane%32, k-slots = tile rows 16s + 8(e/4) +
// 4(lane/32) + e%4.
__device__ __forceinline__ bf16x8 tr_operand(const LDS_AS char* tile, int stride, int b, int s, int lane) {
    const int gq = lane >> 4, r16 = lane & 15;
    const int ra = 16 * s + 4 * (gq >> 1) + (r16 >> 2);
    const int col = 32 * b + 16 * (gq & 1) + 4 * (r16 & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(tile + ra * stride + col * 2));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(tile + (ra + 8) * stride + col * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One wave per (prompt, head, 32 state rows i0 .. i0+31): the chunks in
// order, the state rows on the lanes:
//     W (64 x 32)   = U - Y S^T                 (A = Y rows, B = S rows)
//     O (64 x 32)   = diag(gam) Q S^T + P W     (B = W from registers)
//     S (32 x 128)  = e_last S + (diag(e) W)^T K
// Accumulator layouts: W, O tile tt: chunk row 32tt + 8(r/4) + 4hh + r%4,
// state row i0 + lane%32; S tile jt: state row i0 + 8(r/4) + 4hh + r%4,
// key column 32jt + lane%32. The chunk-row order of W's registers inside a
// 16-wide k step is the permuted order of the transpose reads of K and of
// the P column reads.
__global__ __launch_bounds__(64) void delta_scan_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k, SeqTable t, int nh,
                                                        const char* __restrict__ ws, const float* __restrict__ state_in,
                                                        uint16_t* __restrict__ out, float* __restrict__ state_out) {
    __shared__ __attribute__((aligned(16))) char kt[DC * DD * 2];  // K rows of the chunk, bf16
    __shared__ __attribute__((aligned(16))) char st[32 * DD * 2];  // S rows (bf16), row-major
    const int lane = threadIdx.x, hh = lane >> 5, l32 = lane & 31;
    const int sg = blockIdx.x, h = blockIdx.y, i0 = 32 * blockIdx.z;
    int c0 = 0;
    for (int i = 0; i < sg; ++i) c0 += (t.s[i].n_kept + DC - 1) / DC;
    const int n_chunks = (t.s[sg].n_kept + DC - 1) / DC;

    f32x16 sacc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            sacc[jt][r] = state_in ? state_in[(((int64_t)sg * nh + h) * DD + i) * DD + 32 * jt + l32] : 0.0f;
        }

    for (int c = 0; c < n_chunks; ++c) {
        const int64_t row0 = t.s[sg].kept_off + (int64_t)c * DC;
        const int len = min(DC, t.s[sg].n_kept - c * DC);
        const char* rec = ws + ((size_t)(c0 + c) * nh + h) * DeltaRec::BYTES;
        const float* urec = (const float*)(rec + DeltaRec::U);
        const uint16_t* yrec = (const uint16_t*)(rec + DeltaRec::Y);
        const uint16_t* prec = (const uint16_t*)(rec + DeltaRec::P);
        const float* gam = (const float*)(rec + DeltaRec::GAM);
        const float* ee = (const float*)(rec + DeltaRec::E);

        // The state (bf16) and the chunk's K rows into LDS.
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int il = 8 * (r >> 2) + 4 * hh + (r & 3);
                *(LDS_AS uint16_t*)(st + (il * DD + 32 * jt + l32) * 2) = f2bf(sacc[jt][r]);
            }
        for (int idx = lane; idx < DC * DD / 8; idx += 64) {
            const int r = idx / (DD / 8), cc = idx % (DD / 8);
            *(LDS_AS u32x4*)(kt + (r * DD + cc * 8) * 2) =
                *(const u32x4*)(k + ((row0 + min(r, len - 1)) * nh + h) * DD + cc * 8);
        }
        __syncthreads();

        // S rows as the B operand (lane = state row, k = key column).
        bf16x8 sop[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
            sop[s2] = *(const LDS_AS bf16x8*)(st + (l32 * DD + 16 * s2 + 8 * hh) * 2);
        f32x16 wt[2], ot[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int rr = 32 * tt + l32;  // this lane's A-operand chunk row
            const uint16_t* yrow = yrec + rr * DD + 8 * hh;
            const uint16_t* qrow = q + ((row0 + min(rr, len - 1)) * nh + h) * DD + 8 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                wt[tt][r] = 0.0f;
                ot[tt][r] = 0.0f;
            }
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
                const bf16x8 yb = *(const bf16x8*)(yrow + 16 * s2);
                const bf16x8 qb = *(const bf16x8*)(qrow + 16 * s2);
                wt[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yb, sop[s2], wt[tt], 0, 0, 0);
                ot[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb, sop[s2], ot[tt], 0, 0, 0);
            }
            // W = U - Y S^T; O's rows scaled by exp(G).
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tr = 32 * tt + 8 * (r >> 2) + 4 * hh + (r & 3);
                wt[tt][r] = urec[tr * DD + i0 + l32] - wt[tt][r];
                ot[tt][r] *= gam[tr];
            }
        }
        // O += P W: A = P rows (k = chunk rows in the permuted order), B = W
        // from its registers (k-step s2: tile s2/2, registers 8(s2%2) .. +8).
        bf16x8 wop[4], wsc[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            u32x4 w, ws2;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int r0 = 8 * (s2 & 1) + 2 * e2;
                const float x0 = wt[s2 >> 1][r0], x1 = wt[s2 >> 1][r0 + 1];
                const int t0 = 32 * (s2 >> 1) + 8 * (r0 >> 2) + 4 * hh + (r0 & 3);
                w[e2] = pack_bf16x2(x0, x1);
                ws2[e2] = pack_bf16x2(x0 * ee[t0], x1 * ee[t0 + 1]);
            }
            wop[s2] = __builtin_bit_cast(bf16x8, w);
            wsc[s2] = __builtin_bit_cast(bf16x8, ws2);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const uint16_t* prow = prec + (32 * tt + l32) * DC + 4 * hh;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const uint2 lo = *(const uint2*)(prow + 16 * s2), hi = *(const uint2*)(prow + 16 * s2 + 8);
                const u32x4 pw = {lo.x, lo.y, hi.x, hi.y};
                ot[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pw), wop[s2], ot[tt], 0,
                                                                 0, 0);
            }
            // Output rows of the chunk (only the prompt's own rows).
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tr = 32 * tt + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (tr < len) out[((row0 + tr) * nh + h) * DD + i0 + l32] = f2bf(ot[tt][r]);
            }
        }
        // S = e_last S + (diag(e) W)^T K: A = diag(e) W from registers (lane =
        // state row, k = chunk rows), B = K read transposed from LDS.
        const float elast = gam[DC - 1];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[jt][r] *= elast;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    wsc[s2], tr_operand((const LDS_AS char*)kt, DD * 2, jt, s2, lane), sacc[jt], 0, 0, 0);
        }
        __syncthreads();  // LDS tiles are rewritten by the next chunk
    }
    if (state_out) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                state_out[(((int64_t)sg * nh + h) * DD + i) * DD + 32 * jt + l32] = sacc[jt][r];
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
        hipLaunchKernelGGL(delta_scan_kernel, dim3((unsigned)t.n, (unsigned)nh, DD / 32), dim3(64), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, t, nh, (const char*)workspace, state_in,
                           (uint16_t*)out, state_out);
    return hipGetLastError();
}

}  // namespace tg
