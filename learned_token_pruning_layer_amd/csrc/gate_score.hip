// Step 1 - gate score: s_r = w2 . SiLU(W1 x_r + b1) + b2 for every row.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (a small MLP gate scores
// every token from its post-attention residual at gate layer L); ai4bro.com
// post, section on how learned token pruning works (same gate module).
//
// bf16 path: a skinny GEMM H^T = W1 . X^T on v_mfma_f32_32x32x16_bf16 with
// the SiLU, the w2 dot product and the cross-wave reduction fused into the
// epilogue, so the [N, H] hidden activations never leave registers. One
// workgroup owns a tile of 64 or 128 rows and all H hidden units; its 8
// waves split the tile's hidden x row blocks (32 x 32 per MFMA tile).
//
// The kernel streams X from HBM once and W1 (L2-resident: 1 MiB at H=256,
// d=2048) once per tile, and the L2 -> CU path carrying W1 is what bounds
// it: at 64-row tiles W1 is 4x the X bytes a CU receives. Hence
//  * both operands move global -> LDS with direct loads
//    (global_load_lds_dwordx4, no staging registers), the fastest path into
//    LDS on this part, through rings of 64-wide k chunks: 4 stages each for
//    X and W1 at 64-row tiles (all 160 KB of LDS; the epilogue's partial
//    sums reuse the X ring once the k loop is done), 3 each at 128 rows.
//    The W1 ring's depth sets how many chunks ahead its loads are issued,
//    which matters more than the X ring's. Every load instruction covers 8
//    whole 128-byte row segments, so each fetched cache line is used in
//    full;
//  * one barrier per chunk: after it every wave refills the slots of the
//    chunk just finished, its loads spread between the k steps' MFMAs, so
//    load issue and matrix work overlap;
//  * workgroups on one XCD start at different k chunks, spreading the
//    column every CU reads over the L2 channels;
//  * prompts with more than two 64-row tiles per CU take 128-row tiles,
//    halving the W1 bytes per row.
// Both operands are k-contiguous (W1 rows and X rows), so the MFMA lane
// layouts load 16-byte vectors directly. Inside a 64-wide k chunk the
// k-step / lane-half order is permuted (lane half hh, step ks covers k
// hh*32 + ks*8 .. +8): the same permutation on both operands leaves the
// contraction unchanged. X and W1 rows are 128-byte LDS rows whose 16-byte
// chunk c sits at position c ^ ((row / 2) mod 8): 16 consecutive rows read
// one chunk without bank conflicts (the LDS has 64 four-byte banks). Each
// row's score adds the 32-unit hidden tiles' shares in hidden order, the
// same order for either tile height.
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, int64_t i) { return bf2f(p[i]); }

__device__ __forceinline__ float silu(float h) { return h / (1.0f + __expf(-h)); }

constexpr int GBK = 64;  // k per chunk

// WH x WR waves; wave (wh, wr) owns hidden tiles wh*TH .. +TH and row tiles
// wr*TR .. +TR (32 each), so the workgroup covers H = 32*WH*TH hidden units
// and GBM = 32*WR*TR rows. X streams through an NX-stage LDS ring, W1
// through an NW1-stage one (NW1 <= NX). XF: a wave issues its X loads of an
// iteration before its W1 loads (else after). KR: k steps whose operands are
// read from LDS ahead of the MFMAs.
template <int WH, int TH, int WR, int TR, int NX, int NW1, bool XF, int KR>
__global__ __launch_bounds__(64 * WH * WR) void gate_mfma_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                 int d, const uint16_t* __restrict__ w1,
                                                                 const uint16_t* __restrict__ b1,
                                                                 const uint16_t* __restrict__ w2, float b2,
                                                                 float* __restrict__ scores) {
    constexpr int NWV = WH * WR;
    constexpr int H = 32 * WH * TH;
    constexpr int GBM = 32 * WR * TR;
    constexpr int XI = GBM / 8 / NWV;  // 1 KiB X loads per wave per chunk (8 rows of 128 B)
    constexpr int WI = H / 8 / NWV;    // 1 KiB W1 loads per wave per chunk
    constexpr int OPS = XI + WI;
    static_assert(GBM % (8 * NWV) == 0 && H % (8 * NWV) == 0, "loads split evenly over the waves");
    static_assert(NW1 >= 2 && NW1 <= NX, "ring depths");
    // Loads issued after the youngest load of chunk c, counted when iteration
    // c begins (iteration i issues X(i + NX - 1) and W1(i + NW1 - 1)).
    constexpr int WAIT = XF ? (NW1 - 2) * OPS : (NW1 < NX ? XI + (NW1 - 2) * OPS : (NX - 2) * OPS);
    static_assert(WAIT < 64, "vmcnt range");
    constexpr int U = (NX % NW1 == 0) ? NX : NX * NW1;  // unroll: every ring slot a constant
    __shared__ __attribute__((aligned(1024))) char xs[NX][GBM * GBK * 2];
    __shared__ __attribute__((aligned(1024))) char ws[NW1][H * GBK * 2];
    // Partial sums of the epilogue, in the X ring's memory (free after the k loop).
    static_assert((H / 32) * GBM * 4 <= NX * GBM * GBK * 2, "partial sums fit in the X ring");
    float (*part)[GBM] = (float (*)[GBM])(&xs[0][0]);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wh = wave % WH;
    const int wr = wave / WH;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * GBM;
    const int nchunk = d / GBK;
    // Workgroups start at different k chunks, so that the CUs of an XCD
    // (every eighth workgroup) do not all read the same 128-byte column of
    // every row at once.
    const int r0 = (int)((blockIdx.x >> 3) % (unsigned)nchunk);
    auto rot = [&](int c) { const int t = c + r0; return t >= nchunk ? t - nchunk : t; };

    // Load q (0 .. OPS-1) of iteration it (ub = it mod U, a constant), in
    // issue order. Iterations below 0 prime the rings and skip W1 chunks
    // below 0. A chunk past the last one is not needed, but its loads are
    // still issued, every lane reading the same 16 bytes, so that every
    // iteration issues exactly OPS loads and the waits stay exact.
    auto issue = [&](int it, int ub, int q) {
        const bool isx = XF ? q < XI : q >= WI;
        const int i = XF ? (isx ? q : q - XI) : (isx ? q - WI : q);
        const int c = it + (isx ? NX - 1 : NW1 - 1);
        if (c < 0) return;
        const bool dead = c >= nchunk;
        if (isx) {
            const int inst = wave * XI + i;  // rows 8*inst .. +8 of the X tile
            const int row = inst * 8 + (lane >> 3);
            const int ch = (lane & 7) ^ ((row >> 1) & 7);
            int64_t gr = row0 + row;
            if (gr > n - 1) gr = n - 1;  // ragged tail: re-read the last row, never stored
            const uint16_t* src = dead ? x : x + gr * d + rot(c) * GBK + ch * 8;
            dma16(src, (const LDS_AS void*)&xs[(ub + NX - 1) % NX][inst * 1024]);
        } else {
            const int inst = wave * WI + i;
            const int row = inst * 8 + (lane >> 3);
            const int ch = (lane & 7) ^ ((row >> 1) & 7);
            const uint16_t* src = dead ? w1 : w1 + (int64_t)row * d + rot(c) * GBK + ch * 8;
            dma16(src, (const LDS_AS void*)&ws[(ub + NW1 - 1) % NW1][inst * 1024]);
        }
    };

    f32x16 acc[TH][TR];
#pragma unroll
    for (int th = 0; th < TH; ++th)
#pragma unroll
        for (int tr = 0; tr < TR; ++tr)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[th][tr][j] = 0.0f;

#pragma unroll
    for (int p = -(NX - 1); p < 0; ++p)
#pragma unroll
        for (int q = 0; q < OPS; ++q) issue(p, p + U, q);

    for (int cb = 0; cb < nchunk; cb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cb + u;
            if (c >= nchunk) break;
            // This wave's loads of chunk c have landed; after the barrier so
            // have every other wave's, and every wave is done with chunk c-1,
            // whose ring slots this iteration's loads refill.
            wait_vmcnt<WAIT>();
            ring_barrier();
            const LDS_AS char* xt = (const LDS_AS char*)xs[u % NX];
            const LDS_AS char* wt = (const LDS_AS char*)ws[u % NW1];
            bf16x8 a[4][TH], bx[4][TR];
            auto read = [&](int ks) {
#pragma unroll
                for (int th = 0; th < TH; ++th) {
                    const int r = (wh * TH + th) * 32 + l32;
                    const int ch = (hh * 4 + ks) ^ ((r >> 1) & 7);
                    a[ks][th] = *(const LDS_AS bf16x8*)(wt + r * 128 + ch * 16);
                }
#pragma unroll
                for (int tr = 0; tr < TR; ++tr) {
                    const int r = (wr * TR + tr) * 32 + l32;
                    const int ch = (hh * 4 + ks) ^ ((r >> 1) & 7);
                    bx[ks][tr] = *(const LDS_AS bf16x8*)(xt + r * 128 + ch * 16);
                }
            };
#pragma unroll
            for (int ks = 0; ks < KR; ++ks) read(ks);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                // This iteration's loads go out between the k steps, and the
                // operands of k step ks + KR are read ahead of its MFMAs.
#pragma unroll
                for (int q = ks * OPS / 4; q < (ks + 1) * OPS / 4; ++q) issue(c, u, q);
                if (ks + KR < 4) read(ks + KR);
#pragma unroll
                for (int th = 0; th < TH; ++th)
#pragma unroll
                    for (int tr = 0; tr < TR; ++tr)
                        acc[th][tr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][th], bx[ks][tr], acc[th][tr], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave's loads have landed and its LDS reads are done

    // Epilogue. acc[th][tr] register j holds hidden unit 32*(wh*TH + th) +
    // 8*(j/4) + 4*hh + j%4 of token 32*(wr*TR + tr) + l32. Each 32-unit
    // hidden tile's share of w2 . SiLU(.) is summed on its own and the tiles
    // are added in hidden order, so the rounding is that of one fixed order
    // whatever the wave tiling.
#pragma unroll
    for (int th = 0; th < TH; ++th) {
        const int tile = wh * TH + th;
        float ps[TR];
#pragma unroll
        for (int tr = 0; tr < TR; ++tr) ps[tr] = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int hid = tile * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            const float bias = b1 ? bf2f(b1[hid]) : 0.0f;
            const float wo = bf2f(w2[hid]);
#pragma unroll
            for (int tr = 0; tr < TR; ++tr) ps[tr] += wo * silu(acc[th][tr][j] + bias);
        }
#pragma unroll
        for (int tr = 0; tr < TR; ++tr) {
            ps[tr] += __shfl_xor(ps[tr], 32);
            if (hh == 0) part[tile][(wr * TR + tr) * 32 + l32] = ps[tr];
        }
    }
    __syncthreads();
    for (int r = tid; r < GBM; r += 64 * NWV) {
        if (row0 + r < n) {
            float sum = 0.0f;
#pragma unroll
            for (int t = 0; t < H / 32; ++t) sum += part[t][r];
            scores[row0 + r] = sum + b2;
        }
    }
}

// Plain path (fp32, or bf16 shapes the MFMA kernel does not take): one wave
// per row; lanes split d; hidden units in order; fp32 FMA.
template <typename T>
__global__ __launch_bounds__(256) void gate_simple_kernel(const T* __restrict__ x, int64_t n, int d,
                                                          const T* __restrict__ w1,
                                                          const T* __restrict__ b1, int h,
                                                          const T* __restrict__ w2, float b2,
                                                          float* __restrict__ scores) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const T* xr = x + row * d;
    float s = 0.0f;
    for (int j = 0; j < h; ++j) {
        const T* wr = w1 + (int64_t)j * d;
        float a = 0.0f;
        for (int c = lane; c < d; c += 64) a = fmaf(load_f(xr, c), load_f(wr, c), a);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off);
        if (b1) a += load_f(b1, j);
        s = fmaf(load_f(w2, j), silu(a), s);
    }
    if (lane == 0) scores[row] = s + b2;
}

}  // namespace

hipError_t launch_gate_mfma_bf16(const void* x, int64_t n, int d, const void* w1, const void* b1,
                                 int h, const void* w2, float b2, float* scores, hipStream_t st) {
    auto go = [&](auto kern, int rows, int threads) {
        hipLaunchKernelGGL(kern, dim3((unsigned)((n + rows - 1) / rows)), dim3(threads), 0, st, (const uint16_t*)x, n, d,
                           (const uint16_t*)w1, (const uint16_t*)b1, (const uint16_t*)w2, b2, scores);
    };
    // H = 256: up to two 64-row tiles per CU, 64 rows per workgroup (every
    // CU busy); longer prompts take 128-row tiles, which halve the W1 bytes
    // each row costs (W1 streams from L2 once per tile).
    if (h == 256) {
        if (n <= 2 * 256 * 64) go(gate_mfma_kernel<8, 1, 1, 2, 4, 4, false, 2>, 64, 512);
        else go(gate_mfma_kernel<4, 2, 2, 2, 3, 3, false, 2>, 128, 512);
    } else if (h == 128) {
        go(gate_mfma_kernel<4, 1, 2, 1, 6, 3, false, 2>, 64, 512);
    } else if (h == 192) {
        // 8 waves of 3 hidden tiles x 1 row tile: 192 units x 128 rows
        go(gate_mfma_kernel<2, 3, 4, 1, 3, 3, false, 2>, 128, 512);
    } else {
        // h == 64: 8 waves of 1 hidden tile x 1 row tile: 64 units x 128 rows
        go(gate_mfma_kernel<2, 1, 4, 1, 4, 4, false, 2>, 128, 512);
    }
    return hipGetLastError();
}

hipError_t launch_gate_simple(tg_dtype dt, const void* x, int64_t n, int d, const void* w1,
                              const void* b1, int h, const void* w2, float b2, float* scores,
                              hipStream_t st) {
    const dim3 grid((unsigned)((n + 3) / 4)), block(256);
    if (dt == TG_F32)
        hipLaunchKernelGGL(gate_simple_kernel<float>, grid, block, 0, st, (const float*)x, n, d,
                           (const float*)w1, (const float*)b1, h, (const float*)w2, b2, scores);
    else
        hipLaunchKernelGGL(gate_simple_kernel<uint16_t>, grid, block, 0, st, (const uint16_t*)x, n,
                           d, (const uint16_t*)w1, (const uint16_t*)b1, h, (const uint16_t*)w2, b2,
                           scores);
    return hipGetLastError();
}

}  // namespace tg
