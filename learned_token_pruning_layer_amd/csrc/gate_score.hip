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
// workgroup owns 64 rows and all H hidden units, one wave per 32 hidden
// units (8 waves at H = 256).
//
// The kernel streams X from HBM once and W1 (L2-resident: 1 MiB at H=256,
// d=2048) once per 64 rows; it keeps enough of both in flight per CU:
//  * both move global -> LDS with direct loads (global_load_lds_dwordx4,
//    no staging registers): X through a 6-stage ring of 64-wide k chunks
//    (5 chunks ahead of the MFMAs), W1 through a 3-stage ring (2 ahead; it
//    comes from L2). Every W1 load instruction covers 8 whole 128-byte row
//    segments, so each fetched cache line is used in full;
//  * the chunk loop is unrolled by 6, so every ring slot is a compile-time
//    constant, and all loads are counted explicitly (wait_vmcnt).
// Both operands are k-contiguous (W1 rows and X rows), so the MFMA lane
// layouts load 16-byte vectors directly. Inside a 64-wide k chunk the
// k-step / lane-half order is permuted (lane half hh, step ks covers k
// hh*32 + ks*8 .. +8): the same permutation on both operands leaves the
// contraction unchanged and lets every lane read 64 contiguous bytes of its
// W1 row per chunk. X and W1 rows are 128-byte LDS rows whose 16-byte chunk
// c sits at position c ^ ((row / 2) mod 8): 16 consecutive rows read one
// chunk without bank conflicts (the LDS has 64 four-byte banks).
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

constexpr int GBM = 64;  // rows per workgroup
constexpr int GBK = 64;  // k per chunk
constexpr int GNX = 6;   // X ring depth (chunks)
constexpr int GNW = 3;   // W1 ring depth (chunks)

template <int NWV>  // waves per workgroup = H / 32
__global__ __launch_bounds__(64 * NWV) void gate_mfma_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                             int d, const uint16_t* __restrict__ w1,
                                                             const uint16_t* __restrict__ b1,
                                                             const uint16_t* __restrict__ w2, float b2,
                                                             float* __restrict__ scores) {
    constexpr int XI = 8 / NWV;       // 1 KB X load instructions per wave per chunk
    constexpr int WI = 4;             // 1 KB W1 load instructions per wave per chunk (32 rows)
    constexpr int OPS = XI + WI;      // loads per wave per chunk
    constexpr int WTILE = NWV * 32 * GBK * 2;
    __shared__ __attribute__((aligned(1024))) char xs[GNX][GBM * GBK * 2];
    __shared__ __attribute__((aligned(1024))) char ws[GNW][WTILE];
    __shared__ float part[NWV][GBM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * GBM;
    const int nchunk = d / GBK;

    // Iteration it loads X for chunk it + GNX - 1 and W1 for chunk it + GNW - 1
    // (past the end the last chunk is re-read, so every wave issues exactly
    // OPS loads per iteration; iterations below 0 only prime the X ring).
    auto issue = [&](int it, int xslot, int wslot) {
        {
            const int c = it + GNX - 1;
            const int k0 = (c < nchunk ? c : nchunk - 1) * GBK;
#pragma unroll
            for (int i = 0; i < XI; ++i) {
                const int inst = wave * XI + i;  // rows 8*inst .. +8 of the X tile
                const int row = inst * 8 + (lane >> 3);
                const int ch = (lane & 7) ^ ((row >> 1) & 7);
                int64_t gr = row0 + row;
                if (gr > n - 1) gr = n - 1;  // ragged tail: re-read the last row, never stored
                dma16(x + gr * d + k0 + ch * 8, (const LDS_AS void*)&xs[xslot][inst * 1024]);
            }
        }
        const int c = it + GNW - 1;
        if (c >= 0) {
            const int k0 = (c < nchunk ? c : nchunk - 1) * GBK;
#pragma unroll
            for (int i = 0; i < WI; ++i) {
                const int row = wave * 32 + i * 8 + (lane >> 3);  // this wave's own W1 rows
                const int ch = (lane & 7) ^ ((row >> 1) & 7);
                dma16(w1 + (int64_t)row * d + k0 + ch * 8, (const LDS_AS void*)&ws[wslot][row * 128 - (lane >> 3) * 128]);
            }
        }
    };

    f32x16 acc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[tb][j] = 0.0f;

    // Prime: iterations -(GNX-1) .. -1.
#pragma unroll
    for (int p = -(GNX - 1); p < 0; ++p) issue(p, (p + GNX - 1) % GNX, ((p + GNW - 1) % GNW + GNW) % GNW);

    for (int cb = 0; cb < nchunk; cb += GNX) {
#pragma unroll
        for (int u = 0; u < GNX; ++u) {
            const int c = cb + u;
            ring_barrier();  // every wave is done with chunk c-1's slots
            issue(c, (u + GNX - 1) % GNX, (u + GNW - 1) % GNW);
            // W1(c) is this wave's youngest needed load; 2 iterations of OPS
            // loads were issued after it (and X(c) is older still).
            wait_vmcnt<OPS * (GNW - 1)>();
            ring_barrier();  // ... and every other wave's loads of chunk c landed
            if (c < nchunk) {
                const LDS_AS char* xt = (const LDS_AS char*)xs[u];
                const LDS_AS char* wt = (const LDS_AS char*)ws[u % GNW];
                const int wr = wave * 32 + l32;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cw = (hh * 4 + ks) ^ ((wr >> 1) & 7);
                    const bf16x8 a = *(const LDS_AS bf16x8*)(wt + wr * 128 + cw * 16);
                    bf16x8 xb[2];
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        const int row = tb * 32 + l32;
                        const int ch = (hh * 4 + ks) ^ ((row >> 1) & 7);
                        xb[tb] = *(const LDS_AS bf16x8*)(xt + row * 128 + ch * 16);
                    }
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
                        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb[tb], acc[tb], 0, 0, 0);
                }
            }
        }
    }
    wait_vmcnt<0>();

    // Epilogue. acc[tb] register j holds hidden unit wave*32 + 8*(j/4) +
    // 4*hh + j%4 of token tb*32 + l32.
    float ps[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int hid = wave * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
        const float bias = b1 ? bf2f(b1[hid]) : 0.0f;
        const float wo = bf2f(w2[hid]);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) ps[tb] += wo * silu(acc[tb][j] + bias);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        ps[tb] += __shfl_xor(ps[tb], 32);
        if (hh == 0) part[wave][tb * 32 + l32] = ps[tb];
    }
    __syncthreads();
    if (tid < GBM && row0 + tid < n) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) sum += part[w][tid];
        scores[row0 + tid] = sum + b2;
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
    const dim3 grid((unsigned)((n + GBM - 1) / GBM));
    if (h == 256)
        hipLaunchKernelGGL(gate_mfma_kernel<8>, grid, dim3(512), 0, st, (const uint16_t*)x, n, d,
                           (const uint16_t*)w1, (const uint16_t*)b1, (const uint16_t*)w2, b2, scores);
    else
        hipLaunchKernelGGL(gate_mfma_kernel<4>, grid, dim3(256), 0, st, (const uint16_t*)x, n, d,
                           (const uint16_t*)w1, (const uint16_t*)b1, (const uint16_t*)w2, b2, scores);
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
