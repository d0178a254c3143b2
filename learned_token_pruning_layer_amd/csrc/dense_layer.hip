// The full above-gate decoder layer over the kept rows: the model's own
// layer (Qwen3 family) run on the compacted rows at their original positions.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (the layers above the gate
// process only the kept tokens and build no KV entries for the others) and
// section "Was ist token-gated Attention?" (their attention carries the
// kept tokens' bias); ai.info news, section "TokenGate impara quali token
// mantenere" (only the kept tokens' representations go up). The layer:
//     a   = RMSNorm(h) * ln1
//     qkv = a Wqkv^T;  q, k = rotary(RMSNorm_head(q|k) * q_norm|k_norm, pos)
//     h2  = h + TokenGatedAttention(q, k, v) Wo^T
//     out = h2 + (SiLU(a2 Wg^T) * (a2 Wu^T)) Wd^T,   a2 = RMSNorm(h2) * ln2
// bf16 storage between the steps, fp32 arithmetic inside each.
//
// Kernels:
//  * rmsnorm_kernel: one wave per row, sum of squares in fp32.
//  * qk_norm_rope_kernel: one workgroup per row; a wave normalises one head
//    at a time (lane i holds the rotary pair (i, i + D/2)), rotates it by
//    the row's original position (angle reduced in fp64, sin/cos in fp32)
//    and writes q, k and v as separate [M, heads, D] tensors.
//  * linear_kernel<EPI, ...>: C = A W^T on 32x32x16 bf16 MFMA: 256 x 256
//    per workgroup of 8 waves of 128 weight rows x 64 activation rows when
//    that makes at least 128 tiles (half the loads per MFMA of the next
//    size), else 256 x 128 of 8 waves of 64 x 64 (one workgroup per CU), or
//    128 x 128 of 4 such waves (two per CU) for narrow outputs; 64-wide k
//    chunks streamed global -> LDS with direct loads through a two-stage
//    ring (swizzled 128-byte LDS rows, permuted k-step order), tiles ordered
//    so the workgroups of one XCD share weight tiles. The weights are the
//    MFMA A operand, so each lane's accumulators hold 4 consecutive output
//    columns of one row (8-byte stores). Epilogues: plain store, residual
//    add, and SwiGLU (a tile's weight rows are gate rows and the matching up
//    rows; a wave holds both halves of its columns).
#include "tg_internal.hpp"
#include "tg_device.hpp"

namespace tg {
namespace {

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// ------------------------------------------------------------------ RMSNorm

// out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w, rows of d (d % 512 == 0 not
// required: d % 8 == 0). One wave per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int64_t m, int d,
                                                      const uint16_t* __restrict__ w, float eps,
                                                      uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= m) return;
    const uint16_t* xr = x + row * d;
    float ss = 0.0f;
    for (int c = lane * 8; c < d; c += 512) {
        const u32x4 v = *(const u32x4*)(xr + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xffff0000u);
            ss = fmaf(lo, lo, fmaf(hi, hi, ss));
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = rsqrtf(ss / (float)d + eps);
    uint16_t* orow = out + row * d;
    for (int c = lane * 8; c < d; c += 512) {
        const u32x4 v = *(const u32x4*)(xr + c);
        const u32x4 g = *(const u32x4*)(w + c);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(v[e] << 16) * r * __uint_as_float(g[e] << 16);
            const float hi = __uint_as_float(v[e] & 0xffff0000u) * r * __uint_as_float(g[e] & 0xffff0000u);
            o[e] = pack_bf16x2(lo, hi);
        }
        *(u32x4*)(orow + c) = o;
    }
}

// ------------------------------------------------- Q/K RMSNorm + rotary

// One workgroup (4 waves) per kept row. qkv [m, (hq + 2 hkv) D]: q heads,
// then k heads, then v heads. Lane i of a head's lane group holds elements
// i and i + D/2 (D/2 lanes per head, 64 / (D/2) heads per wave pass).
template <int D>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(const uint16_t* __restrict__ qkv, int64_t m, int hq,
                                                           int hkv, const uint16_t* __restrict__ qn,
                                                           const uint16_t* __restrict__ kn,
                                                           const int32_t* __restrict__ pos, float eps,
                                                           float log2_theta, uint16_t* __restrict__ q,
                                                           uint16_t* __restrict__ k, uint16_t* __restrict__ v) {
    constexpr int HALF = D / 2, HPW = 64 / HALF;  // heads per wave pass
    const int64_t row = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane % HALF, sub = lane / HALF;
    const int width = (hq + 2 * hkv) * D;
    const uint16_t* src = qkv + row * width;
    // Rotary angle of pair i at this row's position: pos * theta^(-2i/D),
    // formed and reduced modulo 2 pi in fp64, then sin / cos in fp32.
    const double inv = exp2(-2.0 * (double)i / (double)D * (double)log2_theta);
    double ang = (double)pos[row] * inv;
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    for (int h0 = wave * HPW; h0 < hq + hkv; h0 += 4 * HPW) {
        const int head = h0 + sub;
        const bool on = head < hq + hkv;
        const int hc = on ? head : hq + hkv - 1;
        const float x1 = bf2f(src[hc * D + i]), x2 = bf2f(src[hc * D + i + HALF]);
        float ss = x1 * x1 + x2 * x2;
#pragma unroll
        for (int o = HALF / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        const float r = rsqrtf(ss / (float)D + eps);
        const uint16_t* nw = hc < hq ? qn : kn;
        const float y1 = x1 * r * bf2f(nw[i]), y2 = x2 * r * bf2f(nw[i + HALF]);
        const float o1 = y1 * cs - y2 * sn, o2 = y2 * cs + y1 * sn;
        if (on) {
            uint16_t* dst = hc < hq ? q + (row * hq + hc) * D : k + (row * hkv + (hc - hq)) * D;
            dst[i] = (uint16_t)(pack_bf16x2(o1, 0.0f) & 0xffffu);
            dst[i + HALF] = (uint16_t)(pack_bf16x2(o2, 0.0f) & 0xffffu);
        }
    }
    // v: a plain copy into its own [m, hkv, D] tensor.
    const uint16_t* vs = src + (hq + hkv) * D;
    uint16_t* vd = v + row * hkv * D;
    for (int c = threadIdx.x * 8; c < hkv * D; c += 256 * 8) *(u32x4*)(vd + c) = *(const u32x4*)(vs + c);
}

// ------------------------------------------------------------------- GEMM

enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };
constexpr int LBK = 64;   // k per chunk
constexpr int LNS = 2;    // ring stages

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// out[m, n] = sum_k a[m, k] w[n, k] (+ resid[m, n]); SwiGLU: out[m, n] =
// SiLU(a . wg[n]) * (a . wu[n]). a [m, k], weights [*, k] row-major, k % 64
// == 0. Workgroup: WN x WM waves, each wave SN x SM sub-tiles of 32 x 32
// (weight rows x activation rows), so TN = 32 SN WN weight rows and TM =
// 32 SM WM activation rows per tile; SwiGLU: the first TN/2 weight rows are gate
// rows and the rest the matching up rows, so a tile makes TN/2 output
// columns. Tile t = (m tile, n tile), m tile fastest; the 8 XCDs each take
// a contiguous range of tiles.
template <int EPI, int SN, int SM, int WN, int WM>
__global__ __launch_bounds__(64 * WN * WM) void linear_kernel(const uint16_t* __restrict__ a, int64_t m, int k,
                                                     const uint16_t* __restrict__ w,
                                                     const uint16_t* __restrict__ w_up, int n_out,
                                                     const uint16_t* __restrict__ resid, uint16_t* __restrict__ out,
                                                     int n_mt, int n_nt) {
    constexpr int NW = WN * WM;                    // waves
    constexpr int TN = 32 * SN * WN, TM = 32 * SM * WM;
    constexpr int AI = TM / (8 * NW), WI = TN / (8 * NW);  // direct loads per wave per chunk (8 rows each)
    static_assert(AI * 8 * NW == TM && WI * 8 * NW == TN, "tile rows must split evenly over the waves");
    constexpr int OPS = AI + WI;
    constexpr int NPT = EPI == EPI_SWIGLU ? TN / 2 : TN;  // output columns per tile
    __shared__ __attribute__((aligned(1024))) char as_[LNS][TM * 128];
    __shared__ __attribute__((aligned(1024))) char ws_[LNS][TN * 128];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int n_tiles = n_mt * n_nt;
    int t = blockIdx.x;
    if ((n_tiles & 7) == 0) t = (t & 7) * (n_tiles >> 3) + (t >> 3);
    const int mt = t % n_mt, nt = t / n_mt;
    const int64_t m0 = (int64_t)mt * TM;
    const int n0 = nt * NPT;
    const int nchunk = k / LBK;

    // Per-lane load rows (fixed across chunks): load instruction i of this
    // wave moves 8 rows x 128 bytes; lane >> 3 picks the row, lane & 7 its
    // 16-byte chunk.
    const uint16_t* asrc[AI];
    const uint16_t* wsrc[WI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int row = (wave * AI + i) * 8 + (lane >> 3);
        asrc[i] = a + min(m0 + row, m - 1) * k + ((lane & 7) ^ swz(row)) * 8;
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
        const int row = (wave * WI + i) * 8 + (lane >> 3);
        const uint16_t* wb = (EPI == EPI_SWIGLU && row >= TN / 2) ? w_up : w;
        const int wr = EPI == EPI_SWIGLU ? n0 + (row % (TN / 2)) : n0 + row;
        wsrc[i] = wb + (int64_t)wr * k + ((lane & 7) ^ swz(row)) * 8;
    }
    auto issue = [&](int c, int slot) __attribute__((always_inline)) {
        const int k0 = (c < nchunk ? c : nchunk - 1) * LBK;
#pragma unroll
        for (int i = 0; i < AI; ++i) dma16(asrc[i] + k0, (const LDS_AS void*)&as_[slot][(wave * AI + i) * 1024]);
#pragma unroll
        for (int i = 0; i < WI; ++i) dma16(wsrc[i] + k0, (const LDS_AS void*)&ws_[slot][(wave * WI + i) * 1024]);
    };

    // Wave tile: weight sub-tiles i (rows 32 SN wn + 32 i; SwiGLU: gate rows
    // 16 SN wn + 32 i for i < SN/2 and the matching up rows TN/2 + ...), and
    // activation sub-tiles j (rows 32 SM wm + 32 j).
    const int wn = wave % WN, wm = wave / WN;
    int wrow[SN], arow[SM];
#pragma unroll
    for (int i = 0; i < SN; ++i)
        wrow[i] = (EPI == EPI_SWIGLU ? (i < SN / 2 ? 16 * SN * wn + 32 * i : TN / 2 + 16 * SN * wn + 32 * (i - SN / 2))
                                     : 32 * SN * wn + 32 * i) + l32;  // (TN / 2 = 16 SN WN)
#pragma unroll
    for (int j = 0; j < SM; ++j) arow[j] = 32 * SM * wm + 32 * j + l32;
    f32x16 acc[SN][SM];
#pragma unroll
    for (int i = 0; i < SN; ++i)
#pragma unroll
        for (int j = 0; j < SM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    issue(0, 0);
    for (int c = 0; c < nchunk; ++c) {
        const int slot = c & 1;
        ring_barrier();  // every wave is done with chunk c - 1's slot
        issue(c + 1, slot ^ 1);
        wait_vmcnt<OPS>();  // this wave's loads of chunk c have landed
        ring_barrier();     // ... and every other wave's
        const LDS_AS char* at = (const LDS_AS char*)as_[slot];
        const LDS_AS char* wt = (const LDS_AS char*)ws_[slot];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 wa[SN], xa[SM];
#pragma unroll
            for (int i = 0; i < SN; ++i)
                wa[i] = *(const LDS_AS bf16x8*)(wt + wrow[i] * 128 + (((hh * 4 + ks) ^ swz(wrow[i])) << 4));
#pragma unroll
            for (int j = 0; j < SM; ++j)
                xa[j] = *(const LDS_AS bf16x8*)(at + arow[j] * 128 + (((hh * 4 + ks) ^ swz(arow[j])) << 4));
#pragma unroll
            for (int i = 0; i < SN; ++i)
#pragma unroll
                for (int j = 0; j < SM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[i], xa[j], acc[i][j], 0, 0, 0);
        }
    }
    wait_vmcnt<0>();

    // acc[i][j] register r: weight row wrow[i] - l32 + 8(r/4) + 4hh + r%4 of
    // activation row m0 + arow[j]: 4 consecutive output columns per group.
#pragma unroll
    for (int j = 0; j < SM; ++j) {
        const int64_t mr = m0 + arow[j];
        if (mr >= m) continue;
        uint16_t* orow = out + mr * n_out;
#pragma unroll
        for (int i = 0; i < (EPI == EPI_SWIGLU ? SN / 2 : SN); ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float o[4];
                int col;
                if (EPI == EPI_SWIGLU) {
                    col = n0 + 16 * SN * wn + 32 * i + 8 * g + 4 * hh;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float gt = acc[i][j][4 * g + e], up = acc[i + SN / 2][j][4 * g + e];
                        o[e] = gt / (1.0f + __expf(-gt)) * up;
                    }
                } else {
                    col = n0 + 32 * SN * wn + 32 * i + 8 * g + 4 * hh;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * g + e];
                    if (EPI == EPI_RESID) {
                        const uint2 rv = *(const uint2*)(resid + mr * n_out + col);
                        o[0] += __uint_as_float(rv.x << 16);
                        o[1] += __uint_as_float(rv.x & 0xffff0000u);
                        o[2] += __uint_as_float(rv.y << 16);
                        o[3] += __uint_as_float(rv.y & 0xffff0000u);
                    }
                }
                uint2 st = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                *(uint2*)(orow + col) = st;
            }
    }
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, int64_t m, int d, const void* w, float eps, void* out, hipStream_t st) {
    if (m > 0)
        hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((m + 3) / 4)), dim3(256), 0, st, (const uint16_t*)x, m, d,
                           (const uint16_t*)w, eps, (uint16_t*)out);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const void* qkv, int64_t m, int hq, int hkv, int head_dim, const void* qn,
                               const void* kn, const int32_t* pos, float eps, float theta, void* q, void* k, void* v,
                               hipStream_t st) {
    if (m == 0) return hipSuccess;
    const float l2t = log2f(theta);
    if (head_dim == 128)
        hipLaunchKernelGGL(qk_norm_rope_kernel<128>, dim3((unsigned)m), dim3(256), 0, st, (const uint16_t*)qkv, m, hq,
                           hkv, (const uint16_t*)qn, (const uint16_t*)kn, pos, eps, l2t, (uint16_t*)q, (uint16_t*)k,
                           (uint16_t*)v);
    else
        hipLaunchKernelGGL(qk_norm_rope_kernel<64>, dim3((unsigned)m), dim3(256), 0, st, (const uint16_t*)qkv, m, hq,
                           hkv, (const uint16_t*)qn, (const uint16_t*)kn, pos, eps, l2t, (uint16_t*)q, (uint16_t*)k,
                           (uint16_t*)v);
    return hipGetLastError();
}

template <int SN, int SM, int WN, int WM>
hipError_t launch_linear_t(int epi, const void* a, int64_t m, int k, const void* w, const void* w_up, int n_out,
                           const void* resid, void* out, hipStream_t st) {
    const int tm = 32 * SM * WM, npt = (epi == EPI_SWIGLU ? 16 : 32) * SN * WN;
    const int n_mt = (int)((m + tm - 1) / tm);
    const int n_nt = n_out / npt;
    const dim3 grid((unsigned)(n_mt * n_nt)), block(64 * WN * WM);
    const uint16_t *ab = (const uint16_t*)a, *wb = (const uint16_t*)w, *ub = (const uint16_t*)w_up;
    const uint16_t* rb = (const uint16_t*)resid;
    uint16_t* ob = (uint16_t*)out;
    if (epi == EPI_SWIGLU)
        hipLaunchKernelGGL((linear_kernel<EPI_SWIGLU, SN, SM, WN, WM>), grid, block, 0, st, ab, m, k, wb, ub, n_out,
                           rb, ob, n_mt, n_nt);
    else if (epi == EPI_RESID)
        hipLaunchKernelGGL((linear_kernel<EPI_RESID, SN, SM, WN, WM>), grid, block, 0, st, ab, m, k, wb, ub, n_out, rb,
                           ob, n_mt, n_nt);
    else
        hipLaunchKernelGGL((linear_kernel<EPI_STORE, SN, SM, WN, WM>), grid, block, 0, st, ab, m, k, wb, ub, n_out, rb,
                           ob, n_mt, n_nt);
    return hipGetLastError();
}

hipError_t launch_linear(int epi, const void* a, int64_t m, int k, const void* w, const void* w_up, int n_out,
                         const void* resid, void* out, hipStream_t st) {
    if (m == 0) return hipSuccess;
    // 256 weight rows x 128 activation rows per workgroup (8 waves, one
    // workgroup per CU, shared loads) where the output width allows it;
    // 128 x 128 (4 waves, two workgroups per CU) otherwise.
    const int wide = epi == EPI_SWIGLU ? 128 : 256;
    // 256 x 256 tiles (8 waves of 128 weight rows x 64 activation rows) halve
    // the loads per MFMA; measured faster than twice as many 256 x 128 tiles
    // once there are at least 128 of them (half the CUs).
    if (n_out % wide == 0 && ((m + 255) / 256) * (n_out / wide) >= 128)
        return launch_linear_t<4, 2, 2, 4>(epi, a, m, k, w, w_up, n_out, resid, out, st);
    if (n_out % wide == 0) return launch_linear_t<2, 2, 4, 2>(epi, a, m, k, w, w_up, n_out, resid, out, st);
    return launch_linear_t<2, 2, 2, 2>(epi, a, m, k, w, w_up, n_out, resid, out, st);
}

}  // namespace tg
