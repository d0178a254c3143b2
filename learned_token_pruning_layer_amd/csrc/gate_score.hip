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
// workgroup (4 waves) owns 64 rows and all H hidden units (each wave H/4 of
// them). The 64-row X tile is shared by the 4 waves through LDS; each wave
// streams its own slice of W1 (L2-resident: 1 MiB at H=256, d=2048) straight
// into MFMA operand registers.
//
// Both operands are k-contiguous (W1 rows and X rows), so the MFMA lane
// layouts load 16-byte vectors directly. Inside a 64-wide k chunk the
// k-step / lane-half order is permuted (lane half hh, step ks covers k
// hh*32 + ks*8 .. +8): the same permutation on both operands leaves the
// contraction unchanged and lets every lane read 64 contiguous bytes of its
// W1 row per chunk.
#include "tg_internal.hpp"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, int64_t i) { return bf2f(p[i]); }

__device__ __forceinline__ float silu(float h) { return h / (1.0f + __expf(-h)); }

constexpr int GBM = 64;            // rows per workgroup
constexpr int GBK = 64;            // k per chunk
constexpr int GLDS = GBK + 8;      // LDS row stride in bf16 (144 bytes: conflict-free b128 reads)

template <int HW>  // hidden units per wave (32 or 64); H = 4 * HW
__global__ __launch_bounds__(256) void gate_mfma_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                        int d, const uint16_t* __restrict__ w1,
                                                        const uint16_t* __restrict__ b1,
                                                        const uint16_t* __restrict__ w2, float b2,
                                                        float* __restrict__ scores) {
    constexpr int HB = HW / 32;  // 32-row hidden blocks per wave
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][GBM * GLDS];
    __shared__ float part[4][GBM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * GBM;
    const int nchunk = d / GBK;

    // X tile loader: 64 rows x 8 sixteen-byte units = 512 units, 2 per thread.
    int64_t xrow[2];
    int xcol[2], xlds[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i;
        const int r = u >> 3;
        const int c = (u & 7) * 8;
        int64_t gr = row0 + r;
        if (gr > n - 1) gr = n - 1;  // ragged tail: re-read the last row, never stored
        xrow[i] = gr * (int64_t)d;
        xcol[i] = c;
        xlds[i] = r * GLDS + c;
    }
    // W1 rows of this lane (one per hidden block).
    const uint16_t* wrow[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
        wrow[hb] = w1 + (int64_t)(wave * HW + hb * 32 + l32) * d + hh * 32;

    uint4 xr[2];
    bf16x8 wr[HB][4], wn[HB][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) xr[i] = *(const uint4*)(x + xrow[i] + xcol[i]);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) wr[hb][ks] = *(const bf16x8*)(wrow[hb] + ks * 8);
#pragma unroll
    for (int i = 0; i < 2; ++i) *(uint4*)&xs[0][xlds[i]] = xr[i];
    __syncthreads();

    f32x16 acc[HB][2];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[hb][tb][j] = 0.0f;

    for (int c = 0; c < nchunk; ++c) {
        const int buf = c & 1;
        // Prefetch the next chunk (the last iteration re-reads its own chunk,
        // which keeps the loads unconditional and the registers in place).
        const int k1 = (c + 1 < nchunk ? c + 1 : c) * GBK;
#pragma unroll
        for (int i = 0; i < 2; ++i) xr[i] = *(const uint4*)(x + xrow[i] + k1 + xcol[i]);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) wn[hb][ks] = *(const bf16x8*)(wrow[hb] + k1 + ks * 8);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 xb[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                xb[tb] = *(const bf16x8*)&xs[buf][(tb * 32 + l32) * GLDS + hh * 32 + ks * 8];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc[hb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[hb][ks], xb[tb],
                                                                          acc[hb][tb], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) *(uint4*)&xs[buf ^ 1][xlds[i]] = xr[i];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) wr[hb][ks] = wn[hb][ks];
        __syncthreads();
    }

    // Epilogue. acc[hb][tb] register j holds hidden unit
    // wave*HW + hb*32 + 8*(j/4) + 4*hh + j%4 of token tb*32 + l32.
    float ps[2] = {0.0f, 0.0f};
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int hid = wave * HW + hb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            const float bias = b1 ? bf2f(b1[hid]) : 0.0f;
            const float wo = bf2f(w2[hid]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) ps[tb] += wo * silu(acc[hb][tb][j] + bias);
        }
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        ps[tb] += __shfl_xor(ps[tb], 32);
        if (hh == 0) part[wave][tb * 32 + l32] = ps[tb];
    }
    __syncthreads();
    if (tid < GBM && row0 + tid < n)
        scores[row0 + tid] = ((part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid])) + b2;
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
    const dim3 grid((unsigned)((n + GBM - 1) / GBM)), block(256);
    if (h == 256)
        hipLaunchKernelGGL(gate_mfma_kernel<64>, grid, block, 0, st, (const uint16_t*)x, n, d,
                           (const uint16_t*)w1, (const uint16_t*)b1, (const uint16_t*)w2, b2, scores);
    else
        hipLaunchKernelGGL(gate_mfma_kernel<32>, grid, block, 0, st, (const uint16_t*)x, n, d,
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
