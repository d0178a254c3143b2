// Backward of the gate MLP: the last link of the path from the attention
// bias back to the scorer.
//
// Defined by the TokenGate pages: spke.com article, section "Was ist
// token-gated Attention?" (the kept tokens' scores enter the logits as a
// bias, which gives the gradient a way back to the scorer, like a
// mixture-of-experts router) and section "Wie hat TokenGate das Pruning von
// Tokens verstanden?" (the scorer is a small MLP over the residual at the
// gate layer). With z_r = W1 x_r + b1, s_r = w2 . SiLU(z_r) + b2 and the
// score gradient ds_r of the listed rows:
//     dz_r = ds_r * w2 * SiLU'(z_r),  SiLU'(z) = sig(z) (1 + z (1 - sig(z))),
//     dW1 = sum_r dz_r x_r^T,  db1 = sum_r dz_r,  dw2 = sum_r ds_r SiLU(z_r),
//     db2 = sum_r ds_r,  dx_r += W1^T dz_r.
//
// Kernels (bf16 inputs, fp32 accumulation and gradients):
//  A. dz: one workgroup per (32 listed rows, 32 hidden units) recomputes z
//     on 32x32x16 bf16 MFMA from the gathered x rows and W1 rows (both
//     k-contiguous, so operands load straight from global memory, the next
//     64-wide k chunk in flight while the current one is used; the four
//     waves split the k range); the epilogue forms dz and the tile's
//     partial sums of dw2 and db1, and stores dz twice in bf16: dZ
//     [rows][H] and dZ^T [H][rows].
//  B. dx: dX = dZ W1 per (128 rows, 32 columns of d) workgroup; W1's
//     column slice is staged in LDS and read transposed
//     (ds_read_b64_tr_b16); results are added to the listed rows of dx.
//  C. dW1 partials: dZ^T X per (64 columns of d, 256-row chunk of the
//     list) workgroup, one wave per 32 hidden units; the chunk's gathered
//     x columns are staged in LDS and read transposed.
//  D. reductions of the partials in a fixed order (deterministic).
// Launches: A; then B, C and the small reductions of D (which read only
// what A wrote) in one grid, so none of them runs alone; then dW1's
// reduction.
// Inside each 16-wide k step the transpose read hands lane half hh the k
// indices 8(e/4) + 4hh + e%4 (e = 0..7); dZ and dZ^T are stored with bits
// 2 and 3 of the index inside each 16-group swapped, so a plain 16-byte
// load of 8 consecutive entries gives the matching operand.
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Position inside a 16-group with bits 2 and 3 exchanged (an involution).
__device__ __forceinline__ int swap23(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// Gathered row of list entry i (entries past the list end repeat the last).
__device__ __forceinline__ int64_t list_row(const int32_t* __restrict__ rows, int64_t i, int64_t n_list,
                                            int64_t n_rows) {
    const int64_t li = min(i, n_list - 1);
    int64_t r = rows ? (int64_t)rows[li] : li;
    return r < 0 ? 0 : (r >= n_rows ? n_rows - 1 : r);
}

// B operand of a 32x32x16 MFMA from an LDS tile of 64-byte rows (32 bf16
// columns): column (lane%32), k-slots = tile rows r0 + 8(e/4) + 4(lane/32) +
// e%4. Four consecutive rows of one read cover disjoint 16-bank spans.
__device__ __forceinline__ bf16x8 tr_operand64(const LDS_AS char* tile, int r0, int lane) {
    const int g = lane >> 4, r16 = lane & 15;
    const int ra = r0 + 4 * (g >> 1) + (r16 >> 2);
    const int col = 16 * (g & 1) + 4 * (r16 & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(tile + ra * 64 + col * 2));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(tile + (ra + 8) * 64 + col * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A. z = X_list W1^T for 32 listed rows x 32 hidden units, then dz and the
// partial sums. The four waves of a workgroup take interleaved 64-wide k
// chunks (chunk c goes to wave c % 4) and add their partial sums through LDS
// in wave order; wave 0 runs the epilogue. acc register j: list row m0 +
// 8(j/4) + 4hh + j%4, hidden unit h0 + lane%32.
__global__ __launch_bounds__(256) void gbwd_dz_kernel(const uint16_t* __restrict__ x, int d,
                                                      const uint16_t* __restrict__ w1,
                                                      const uint16_t* __restrict__ b1,
                                                      const uint16_t* __restrict__ w2,
                                                      const float* __restrict__ d_scores,
                                                      const int32_t* __restrict__ rows, int64_t n_list,
                                                      int64_t n_rows, int hdim, int64_t n_pad,
                                                      uint16_t* __restrict__ dz, uint16_t* __restrict__ dzt,
                                                      float* __restrict__ pw2, float* __restrict__ pb1) {
    __shared__ __attribute__((aligned(16))) f32x4 part[3][4][64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int64_t m0 = 32LL * blockIdx.x;
    const int h0 = 32 * blockIdx.y;
    const uint16_t* arow = x + list_row(rows, m0 + l32, n_list, n_rows) * d + 8 * hh;
    const uint16_t* brow = w1 + (int64_t)(h0 + l32) * d + 8 * hh;

    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
    // Two register stages of one 64-wide k chunk (4 k-steps) each.
    bf16x8 a0[4], b0[4], a1[4], b1v[4];
    auto load = [&](bf16x8* a, bf16x8* b, int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a[s] = *(const bf16x8*)(arow + k0 + 16 * s);
            b[s] = *(const bf16x8*)(brow + k0 + 16 * s);
        }
    };
    auto mma = [&](const bf16x8* a, const bf16x8* b) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc, 0, 0, 0);
    };
    const int kstep = 4 * 64;
    int k0 = 64 * wave;
    if (k0 < d) load(a0, b0, k0);
    for (; k0 < d; k0 += 2 * kstep) {
        if (k0 + kstep < d) load(a1, b1v, k0 + kstep);
        mma(a0, b0);
        if (k0 + kstep >= d) break;
        if (k0 + 2 * kstep < d) load(a0, b0, k0 + 2 * kstep);
        mma(a1, b1v);
    }
    if (wave > 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            part[wave - 1][q][lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = part[w][q][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * q + e] += v[e];
        }

    const int h = h0 + l32;
    const float bias = b1 ? bf2f(b1[h]) : 0.0f, wo = bf2f(w2[h]);
    float sw2 = 0.0f, sb1 = 0.0f;
    uint32_t packed[8];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int64_t m = m0 + 8 * (j >> 2) + 4 * hh + (j & 3);
        const float ds = m < n_list ? d_scores[list_row(rows, m, n_list, n_rows)] : 0.0f;
        const float z = acc[j] + bias;
        const float sg = 1.0f / (1.0f + __expf(-z));
        const float g = ds * wo * sg * (1.0f + z * (1.0f - sg));
        sw2 = fmaf(ds, z * sg, sw2);
        sb1 += g;
        const uint32_t bits = pack_bf16x2(g, 0.0f) & 0xffffu;
        // dZ [m][h]: hidden units in swapped order inside each 16-group.
        dz[m * hdim + h0 + (l32 & 16) + swap23(l32 & 15)] = (uint16_t)bits;
        if (j & 1)
            packed[j >> 1] |= bits << 16;
        else
            packed[j >> 1] = bits;
    }
    // dZ^T [h][m]: registers 8g .. 8g+7 are list rows m0 + 16g + swap23(8hh + e),
    // i.e. stored positions m0 + 16g + 8hh .. +8: one 16-byte store each.
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const u32x4 w = {packed[4 * g], packed[4 * g + 1], packed[4 * g + 2], packed[4 * g + 3]};
        *(u32x4*)(dzt + (int64_t)h * n_pad + m0 + 16 * g + 8 * hh) = w;
    }
    sw2 += __shfl_xor(sw2, 32);
    sb1 += __shfl_xor(sb1, 32);
    if (hh == 0) {
        pw2[(int64_t)blockIdx.x * hdim + h] = sw2;
        pb1[(int64_t)blockIdx.x * hdim + h] = sb1;
    }
}

// B. dx[rows[m]] += dZ[m] W1 for 128 list rows x 32 columns of d (one wave
// per 32 rows). acc register j: list row m0 + 8(j/4) + 4hh + j%4, column
// d0 + lane%32.
// Runs on 256 threads (tid 0..255) with a 16 KB LDS slice; `live` false:
// only the barrier (the other half of the workgroup may need it).
__device__ __forceinline__ void gbwd_dx_body(bool live, int bx, int by, int tid, LDS_AS char* wt,
                                             const uint16_t* __restrict__ dz, const uint16_t* __restrict__ w1,
                                             int d, int hdim, const int32_t* __restrict__ rows, int64_t n_list,
                                             int64_t n_rows, float* __restrict__ d_x) {
    const int lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int d0 = 32 * by;
    const int64_t m0 = 128LL * bx + 32 * (tid >> 6);
    if (live)
        for (int idx = tid; idx < hdim * 4; idx += 256)
            *(LDS_AS u32x4*)(wt + idx * 16) = *(const u32x4*)(w1 + (int64_t)(idx >> 2) * d + d0 + (idx & 3) * 8);
    __syncthreads();
    if (!live || m0 >= n_list) return;
    const uint16_t* arow = dz + (m0 + l32) * hdim + 8 * hh;
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
    for (int s0 = 0; s0 < hdim; s0 += 64) {
        bf16x8 a[4], b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a[s] = *(const bf16x8*)(arow + s0 + 16 * s);
            b[s] = tr_operand64((const LDS_AS char*)wt, s0 + 16 * s, lane);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int64_t m = m0 + 8 * (j >> 2) + 4 * hh + (j & 3);
        if (m < n_list) {
            float* p = d_x + list_row(rows, m, n_list, n_rows) * d + d0 + l32;
            *p += acc[j];
        }
    }
}

constexpr int GKC = 256;  // list rows per dW1 chunk

// C. Partial dW1 of one 256-row chunk of the list: dZ^T X for all H hidden
// units (one wave per 32) x 64 columns of d (two 32-column blocks sharing
// the wave's dZ^T operands, which are loaded before any MFMA). acc
// register j: hidden unit 32 wave + 8(j/4) + 4hh + j%4, column d0 + 32cb +
// lane%32.
// Runs on all 512 threads; waves from hdim / 32 on only help stage x.
__device__ __forceinline__ void gbwd_dw1_body(int bx, int by, int tid, LDS_AS char* xt0, LDS_AS char* xt1,
                                              const uint16_t* __restrict__ x, int d,
                                              const uint16_t* __restrict__ dzt, int hdim,
                                              const int32_t* __restrict__ rows, int64_t n_list, int64_t n_rows,
                                              int64_t n_pad, float* __restrict__ pw1) {
    const int lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const bool mw = (tid >> 6) < hdim / 32;  // this wave owns 32 hidden units
    const int d0 = 64 * bx;
    const int64_t c0 = (int64_t)GKC * by;
    const int n_steps = (int)(min((int64_t)GKC, n_pad - c0) / 16);
    const int hrow = 32 * (tid >> 6) + l32;
    const uint16_t* arow = dzt + (int64_t)hrow * n_pad + c0 + 8 * hh;
    bf16x8 a[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (mw && s < n_steps) a[s] = *(const bf16x8*)(arow + 16 * s);
    for (int idx = tid; idx < GKC * 8; idx += 512)
        *(LDS_AS u32x4*)((((idx >> 2) & 1) ? xt1 : xt0) + (idx >> 3) * 64 + (idx & 3) * 16) =
            *(const u32x4*)(x + list_row(rows, c0 + (idx >> 3), n_list, n_rows) * d + d0 + (idx & 7) * 8);
    __syncthreads();
    if (!mw) return;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        f32x16 acc;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int s = 0; s < 16; ++s)
            if (s < n_steps)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    a[s], tr_operand64((const LDS_AS char*)(cb ? xt1 : xt0), 16 * s, lane), acc, 0, 0, 0);
        float* out = pw1 + ((int64_t)by * hdim + 32 * (tid >> 6)) * d + d0 + 32 * cb + l32;
#pragma unroll
        for (int j = 0; j < 16; ++j) out[(int64_t)(8 * (j >> 2) + 4 * hh + (j & 3)) * d] = acc[j];
    }
}

// D1. dW1 = sum of the chunk partials, in chunk order.
__global__ __launch_bounds__(256) void gbwd_reduce_w1_kernel(const float* __restrict__ pw1, int n_kc, int64_t hd,
                                                             float* __restrict__ d_w1) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= hd) return;
    float s = 0.0f;
    for (int c = 0; c < n_kc; ++c) s += pw1[(int64_t)c * hd + i];
    d_w1[i] = s;
}

// D2. Workgroup h < H: dw2[h] and db1[h], the sums of the per-tile
// partials (each lane a strided share, then a butterfly). Workgroup H: db2,
// the sum of the listed score gradients (four loads in flight per thread,
// then a fixed-order tree). Summation orders are fixed.
// Runs on 256 threads (tid 0..255); h > hdim: only the barrier.
__device__ __forceinline__ void gbwd_reduce_small_body(int h, int tid, float (*part)[4],
                                                       const float* __restrict__ pw2,
                                                       const float* __restrict__ pb1, int n_mt, int hdim,
                                                       const float* __restrict__ d_scores,
                                                       const int32_t* __restrict__ rows, int64_t n_list,
                                                       int64_t n_rows, float* __restrict__ d_w2,
                                                       float* __restrict__ d_b1, float* __restrict__ d_b2) {
    float sw = 0.0f, sb = 0.0f;
    if (h < hdim) {
        for (int t = tid; t < n_mt; t += 256) {
            sw += pw2[(int64_t)t * hdim + h];
            sb += pb1[(int64_t)t * hdim + h];
        }
    } else if (h == hdim) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t i0 = tid; i0 < n_list; i0 += 4 * 256) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + (int64_t)u * 256;
                v[u] = i < n_list ? d_scores[list_row(rows, i, n_list, n_rows)] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] += v[u];
        }
        sw = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        sw += __shfl_xor(sw, o);
        sb += __shfl_xor(sb, o);
    }
    if ((tid & 63) == 0) {
        part[0][tid >> 6] = sw;
        part[1][tid >> 6] = sb;
    }
    __syncthreads();
    if (tid == 0 && h <= hdim) {
        const float tw = (part[0][0] + part[0][1]) + (part[0][2] + part[0][3]);
        const float tb = (part[1][0] + part[1][1]) + (part[1][2] + part[1][3]);
        if (h < hdim) {
            d_w2[h] = tw;
            d_b1[h] = tb;
        } else {
            *d_b2 = tw;
        }
    }
}

// B + C + D2 in one launch of 512-thread workgroups (all three read only
// what A wrote): first the small reductions (two hidden units per
// workgroup, one per half), then the dW1 partials, then dx (two of its
// 128-row x 32-column tiles per workgroup, one per half).
__global__ __launch_bounds__(512) void gbwd_mid_kernel(
    const uint16_t* __restrict__ x, int d, const uint16_t* __restrict__ w1, int hdim,
    const uint16_t* __restrict__ dz, const uint16_t* __restrict__ dzt, const float* __restrict__ pw2,
    const float* __restrict__ pb1, int n_mt, const float* __restrict__ d_scores, const int32_t* __restrict__ rows,
    int64_t n_list, int64_t n_rows, int64_t n_pad, float* __restrict__ pw1, float* __restrict__ d_x,
    float* __restrict__ d_w2, float* __restrict__ d_b1, float* __restrict__ d_b2, int n_small, int dw1_x,
    int n_dw1, int dx_x, int n_dx_tiles) {
    __shared__ __attribute__((aligned(16))) char lds[2 * GKC * 64];  // 32 KB: x chunk, or two W1 slices
    __shared__ float part[2][2][4];
    LDS_AS char* base = (LDS_AS char*)lds;
    const int tid = threadIdx.x, half = tid >> 8;
    int b = (int)blockIdx.x;
    if (b < n_small) {
        gbwd_reduce_small_body(2 * b + half, tid & 255, part[half], pw2, pb1, n_mt, hdim, d_scores, rows, n_list,
                               n_rows, d_w2, d_b1, d_b2);
        return;
    }
    b -= n_small;
    if (b < n_dw1) {
        gbwd_dw1_body(b % dw1_x, b / dw1_x, tid, base, base + GKC * 64, x, d, dzt, hdim, rows, n_list, n_rows,
                      n_pad, pw1);
        return;
    }
    b -= n_dw1;
    const int kt = 2 * b + half;
    gbwd_dx_body(kt < n_dx_tiles, kt % dx_x, kt / dx_x, tid & 255, base + half * (256 * 64), dz, w1, d, hdim, rows,
                 n_list, n_rows, d_x);
}

__global__ __launch_bounds__(256) void gbwd_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

struct GateBwdLayout {
    int64_t n_pad, n_mt, n_kc;
    size_t dz, dzt, pw2, pb1, pw1, total;  // byte offsets
};

GateBwdLayout gate_bwd_layout(int64_t n_list, int d, int hdim) {
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    GateBwdLayout l{};
    l.n_pad = (n_list + 63) / 64 * 64;
    l.n_mt = l.n_pad / 32;
    l.n_kc = (l.n_pad + GKC - 1) / GKC;
    l.dz = 0;
    l.dzt = l.dz + up((size_t)l.n_pad * hdim * 2);
    l.pw2 = l.dzt + up((size_t)l.n_pad * hdim * 2);
    l.pb1 = l.pw2 + up((size_t)l.n_mt * hdim * 4);
    l.pw1 = l.pb1 + up((size_t)l.n_mt * hdim * 4);
    l.total = l.pw1 + up((size_t)l.n_kc * hdim * d * 4);
    return l;
}

}  // namespace

size_t gate_backward_workspace_bytes(int64_t n_list, int d_model, int d_hidden) {
    return n_list > 0 ? gate_bwd_layout(n_list, d_model, d_hidden).total : 0;
}

hipError_t launch_gate_backward(const void* x, int64_t n_rows, int d, const void* w1, const void* b1,
                                const void* w2, int hdim, const float* d_scores, const int32_t* rows,
                                int64_t n_list, float* d_x, float* d_w1, float* d_b1, float* d_w2, float* d_b2,
                                void* workspace, hipStream_t st) {
    const int64_t hd = (int64_t)hdim * d;
    if (n_list == 0) {
        hipLaunchKernelGGL(gbwd_zero_kernel, dim3((unsigned)((hd + 255) / 256)), dim3(256), 0, st, d_w1, hd);
        hipLaunchKernelGGL(gbwd_zero_kernel, dim3(1), dim3(256), 0, st, d_b1, (int64_t)hdim);
        hipLaunchKernelGGL(gbwd_zero_kernel, dim3(1), dim3(256), 0, st, d_w2, (int64_t)hdim);
        hipLaunchKernelGGL(gbwd_zero_kernel, dim3(1), dim3(256), 0, st, d_b2, (int64_t)1);
        return hipGetLastError();
    }
    const GateBwdLayout l = gate_bwd_layout(n_list, d, hdim);
    char* ws = (char*)workspace;
    uint16_t* dz = (uint16_t*)(ws + l.dz);
    uint16_t* dzt = (uint16_t*)(ws + l.dzt);
    float* pw2 = (float*)(ws + l.pw2);
    float* pb1 = (float*)(ws + l.pb1);
    float* pw1 = (float*)(ws + l.pw1);
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* w1b = (const uint16_t*)w1;
    hipLaunchKernelGGL(gbwd_dz_kernel, dim3((unsigned)l.n_mt, (unsigned)(hdim / 32)), dim3(256), 0, st, xb, d, w1b,
                       (const uint16_t*)b1, (const uint16_t*)w2, d_scores, rows, n_list, n_rows, hdim, l.n_pad, dz,
                       dzt, pw2, pb1);
    const int dw1_x = d / 64, n_dw1 = dw1_x * (int)l.n_kc;
    const int dx_x = (int)((l.n_pad + 127) / 128), n_dx_tiles = d_x ? dx_x * (d / 32) : 0;
    const int n_small = (hdim + 2) / 2;  // hdim + 1 reductions, two per workgroup
    hipLaunchKernelGGL(gbwd_mid_kernel, dim3((unsigned)(n_small + n_dw1 + (n_dx_tiles + 1) / 2)), dim3(512), 0, st, xb,
                       d, w1b, hdim, dz, dzt, pw2, pb1, (int)l.n_mt, d_scores, rows, n_list, n_rows, l.n_pad, pw1, d_x,
                       d_w2, d_b1, d_b2, n_small, dw1_x, n_dw1, dx_x, n_dx_tiles);
    hipLaunchKernelGGL(gbwd_reduce_w1_kernel, dim3((unsigned)((hd + 255) / 256)), dim3(256), 0, st, pw1,
                       (int)l.n_kc, hd, d_w1);
    return hipGetLastError();
}

}  // namespace tg
