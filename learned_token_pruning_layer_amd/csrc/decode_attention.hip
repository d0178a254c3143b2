// Decode over the pruned KV cache: attention of newly generated tokens over
// the kept rows that the layers above the gate cached during the pruned
// prefill.
//
// Defined by the TokenGate pages: spke.com article, section "Wie hat
// TokenGate das Pruning von Tokens verstanden?" (the layers above the gate
// build no KV entries for pruned tokens, so their cache holds only the kept
// rows), section "Was ist token-gated Attention?" (each kept token's score
// sits as a bias on the attention logits of those layers) and section "Wie
// wird TokenGate implementiert?" (generation after a pruned prefill). The
// bias stays on the cached keys while generating; the new tokens, not being
// document tokens, carry bias 0 (the caller appends them to the cache with
// their bias and position). For new token t of a sequence (cache row i) and
// query head h:
//     logit_j = q . k_j / (sqrt(D) tau) + gain[h] * bias[j],  pos[j] <= pos[i].
//
// The step reads every cached K/V row of the sequence once per KV head and
// does a few flops per byte: HBM-bound. Split-KV: each wave takes a range
// of keys of one (sequence, KV head) for all G x n_new queries that share
// that KV head, and leaves an unnormalised partial (max, sum, O) in the
// workspace; a second kernel merges the partials of each query in key
// order, so the result does not depend on scheduling.
//
// Inside a wave a K or V row (D elements, 16 bytes per lane) is spread over
// LPK lanes: a group of LPK lanes owns one key at a time, NG = 64/LPK groups
// work on NG keys side by side. Per block of KB keys a group loads its KB
// K and V slices (KB x 2 loads of 16 bytes in flight per lane), forms the
// q.k partial sums of its slice, adds them across the group with DPP lane
// moves, and updates an online softmax per query. The groups' partials
// are merged with lane shuffles at the end.
#include "tg_internal.hpp"
#include "tg_device.hpp"

#include <atomic>
#include <mutex>

namespace tg {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int DEC_WAVES = 4;  // waves per workgroup (independent key ranges)
constexpr int DEC_KB = 8;     // keys per group per block

template <typename E>
struct Slice;  // 16 bytes of a row as floats
template <>
struct Slice<uint16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void get(const uint4& w, float* f) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
};
template <>
struct Slice<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void get(const uint4& w, float* f) {
        f[0] = __uint_as_float(w.x);
        f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z);
        f[3] = __uint_as_float(w.w);
    }
};

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over each aligned group of LPK lanes (every lane receives its group's sum).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
    x = dpp_add<0xB1>(x);  // quad_perm [1,0,3,2]: lane ^ 1
    x = dpp_add<0x4E>(x);  // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPK >= 8) x = dpp_add<0x141>(x);   // row_half_mirror: the other quad of each 8
    if constexpr (LPK >= 16) x = dpp_add<0x140>(x);  // row_mirror: the other half of each 16
    if constexpr (LPK >= 32) x += __shfl_xor(x, 16);
    return x;
}

template <typename E, int D, int NQ>
__global__ __launch_bounds__(64 * DEC_WAVES) void decode_partial_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ bias,
    const int32_t* __restrict__ pos, DecTable t, int hq, int hkv, const float* __restrict__ gain, float c,
    float* __restrict__ ws) {
    constexpr int EPL = Slice<E>::N;        // elements per 16-byte lane slice
    constexpr int LPK = D / EPL;            // lanes per key row
    constexpr int NG = 64 / LPK;            // key groups per wave
    static_assert(LPK >= 4 && LPK <= 32 && D % EPL == 0, "row split");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w_all = blockIdx.x * DEC_WAVES + wave;
    if (w_all >= t.n_waves) return;  // whole waves only; no barrier in this kernel
    const int kvh = w_all % hkv;
    const int gs = w_all / hkv;  // global split id
    int b = 0;
    for (int i = 1; i < t.n; ++i)
        if (t.s[i].split_base <= gs) b = i;
    const DecSeq sq = t.s[b];
    const int split = gs - sq.split_base;
    const int k0 = split * t.kpw, k1 = min(sq.len, k0 + t.kpw);
    const int G = hq / hkv;
    const int nq = G * sq.n_new;  // queries of this wave (<= NQ)
    const int g = lane / LPK, r = lane % LPK;
    const int64_t rowe = (int64_t)hkv * D;  // elements between consecutive cache rows

    // This wave's queries: slot qi = h_local * n_new + t (head kvh*G + h_local,
    // new token t), scaled into the exp2 domain.
    float qv[NQ][EPL], gb[NQ];
    int32_t qpos[NQ];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        const int qq = min(qi, nq - 1);
        const int hl = qq / sq.n_new, tt = qq % sq.n_new;
        const int h = kvh * G + hl;
        const uint4 w = *(const uint4*)(q + ((int64_t)(sq.q_row0 + tt) * hq + h) * D + r * EPL);
        Slice<E>::get(w, qv[qi]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[qi][e] *= c;
        gb[qi] = gain[h] * LOG2E;
        qpos[qi] = pos[sq.start + sq.len - sq.n_new + tt];
    }
    float m[NQ], l[NQ], acc[NQ][EPL];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        m[qi] = -INFINITY;
        l[qi] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[qi][e] = 0.0f;
    }

    const E* kb_ = k + (sq.start * hkv + kvh) * (int64_t)D + r * EPL;
    const E* vb_ = v + (sq.start * hkv + kvh) * (int64_t)D + r * EPL;
    // Block loads, double-buffered: block n+1's K/V slices are in flight while
    // block n is scored and accumulated.
    uint4 kw[DEC_KB], vw[DEC_KB], kn[DEC_KB], vn[DEC_KB];
    float bj[DEC_KB], bn[DEC_KB];
    int32_t pj[DEC_KB], pn[DEC_KB];
    auto load_block = [&](int base, uint4 (&kx)[DEC_KB], uint4 (&vx)[DEC_KB], float (&bx)[DEC_KB],
                          int32_t (&px)[DEC_KB]) __attribute__((always_inline)) {
        const int kg = base + g * DEC_KB;
#pragma unroll
        for (int i = 0; i < DEC_KB; ++i) {
            const int j = min(kg + i, k1 - 1);  // past the range: re-read its last key, masked below
            kx[i] = *(const uint4*)(kb_ + j * rowe);
            vx[i] = *(const uint4*)(vb_ + j * rowe);
            bx[i] = bias[sq.start + j];
            px[i] = pos[sq.start + j];
        }
    };
    load_block(k0, kw, vw, bj, pj);
    for (int base = k0; base < k1; base += NG * DEC_KB) {
        const int kg = base + g * DEC_KB;  // this group's first key of the block
        const bool more = base + NG * DEC_KB < k1;  // wave-uniform
        if (more) load_block(base + NG * DEC_KB, kn, vn, bn, pn);
        // Scores: each K slice is unpacked once and used for every query.
        float sc[NQ][DEC_KB];
#pragma unroll
        for (int i = 0; i < DEC_KB; ++i) {
            float kf[EPL];
            Slice<E>::get(kw[i], kf);
            const bool in_range = kg + i < k1;
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                float d = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d = fmaf(qv[qi][e], kf[e], d);
                d = group_sum<LPK>(d);
                sc[qi][i] = (in_range & (pj[i] <= qpos[qi])) ? fmaf(gb[qi], bj[i], d) : -INFINITY;
            }
        }
        // Online softmax per query over the block's keys.
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            float mb = -INFINITY;
#pragma unroll
            for (int i = 0; i < DEC_KB; ++i) mb = fmaxf(mb, sc[qi][i]);
            const float mn = fmaxf(m[qi], mb);
            const float mu = (mn == -INFINITY) ? 0.0f : mn;
            const float corr = __builtin_amdgcn_exp2f(m[qi] - mu);
            float ls = 0.0f;
#pragma unroll
            for (int i = 0; i < DEC_KB; ++i) {
                sc[qi][i] = __builtin_amdgcn_exp2f(sc[qi][i] - mu);  // now p
                ls += sc[qi][i];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[qi][e] *= corr;
            l[qi] = fmaf(l[qi], corr, ls);
            m[qi] = mn;
        }
        // P.V: each V slice is unpacked once and used for every query.
#pragma unroll
        for (int i = 0; i < DEC_KB; ++i) {
            float vf[EPL];
            Slice<E>::get(vw[i], vf);
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[qi][e] = fmaf(sc[qi][i], vf[e], acc[qi][e]);
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < DEC_KB; ++i) {
                kw[i] = kn[i];
                vw[i] = vn[i];
                bj[i] = bn[i];
                pj[i] = pn[i];
            }
        }
    }

    // Merge the NG groups (lanes r, r + LPK, ... hold the same d-slice).
#pragma unroll
    for (int step = LPK; step < 64; step *= 2) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            const float mo = __shfl_xor(m[qi], step), lo = __shfl_xor(l[qi], step);
            const float mn = fmaxf(m[qi], mo);
            const float mu = (mn == -INFINITY) ? 0.0f : mn;
            const float a = __builtin_amdgcn_exp2f(m[qi] - mu), bo = __builtin_amdgcn_exp2f(mo - mu);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float xo = __shfl_xor(acc[qi][e], step);
                acc[qi][e] = acc[qi][e] * a + xo * bo;
            }
            l[qi] = l[qi] * a + lo * bo;
            m[qi] = mn;
        }
    }
    // Partial of this wave: m, l [NQ] then O [NQ][D] (unnormalised, exp2 domain).
    float* pm = ws + (int64_t)w_all * NQ * (D + 2);
    float* pl = pm + NQ;
    float* po = pl + NQ;
    if (g == 0) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (r == 0) {
                pm[qi] = m[qi];
                pl[qi] = l[qi];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) po[qi * D + r * EPL + e] = acc[qi][e];
        }
    }
}

// One workgroup per (new token, query head): merges the partials of every
// split of the sequence in split order. Threads (d, part): part p takes
// splits p, p + P, ... (loads for CU_UNROLL of them in flight); the P part
// results are then merged in part order.
constexpr int CB_THREADS = 1024;
constexpr int CB_UNROLL = 4;

__device__ __forceinline__ void merge_into(float& M, float& L, float& A, float ms, float ls, float os) {
    const float mn = fmaxf(M, ms);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    const float a = __builtin_amdgcn_exp2f(M - mu), bs = __builtin_amdgcn_exp2f(ms - mu);
    A = A * a + os * bs;
    L = L * a + ls * bs;
    M = mn;
}

template <typename E, int D, int NQ>
__global__ __launch_bounds__(CB_THREADS) void decode_combine_kernel(DecTable t, int hq, int hkv,
                                                                    const float* __restrict__ ws,
                                                                    E* __restrict__ out, float* __restrict__ lse,
                                                                    int64_t r_total) {
    constexpr int P = CB_THREADS / D;
    __shared__ float sm[P], sl[P], so[P][D];
    const int row = t.row0 + (int)(blockIdx.x / hq), h = blockIdx.x % hq;
    int b = 0;
    for (int i = 1; i < t.n; ++i)
        if (t.s[i].q_row0 <= row) b = i;
    const DecSeq sq = t.s[b];
    const int tt = row - sq.q_row0;
    const int G = hq / hkv, kvh = h / G, hl = h % G;
    const int qi = hl * sq.n_new + tt;
    const int n_split = (sq.len + t.kpw - 1) / t.kpw;
    const int d = threadIdx.x % D, part = threadIdx.x / D;
    constexpr int64_t WSTRIDE = (int64_t)NQ * (D + 2);  // floats per wave partial
    const int64_t hstride = (int64_t)hkv * WSTRIDE;     // between consecutive splits
    const float* base = ws + ((int64_t)sq.split_base * hkv + kvh) * WSTRIDE;
    float M = -INFINITY, L = 0.0f, A = 0.0f;
    int s = part;
    for (; s + (CB_UNROLL - 1) * P < n_split; s += CB_UNROLL * P) {
        float ms[CB_UNROLL], ls[CB_UNROLL], os[CB_UNROLL];
#pragma unroll
        for (int u = 0; u < CB_UNROLL; ++u) {
            const float* pm = base + (int64_t)(s + u * P) * hstride;
            ms[u] = pm[qi];
            ls[u] = pm[NQ + qi];
            os[u] = pm[2 * NQ + qi * D + d];
        }
#pragma unroll
        for (int u = 0; u < CB_UNROLL; ++u) merge_into(M, L, A, ms[u], ls[u], os[u]);
    }
    for (; s < n_split; s += P) {
        const float* pm = base + (int64_t)s * hstride;
        merge_into(M, L, A, pm[qi], pm[NQ + qi], pm[2 * NQ + qi * D + d]);
    }
    if (d == 0) {
        sm[part] = M;
        sl[part] = L;
    }
    so[part][d] = A;
    __syncthreads();
    if (part == 0) {
        for (int p = 1; p < P; ++p) merge_into(M, L, A, sm[p], sl[p], so[p][d]);
        const float o = A / L;
        const int64_t oi = ((int64_t)row * hq + h) * D + d;
        if constexpr (sizeof(E) == 2) {
            out[oi] = (E)(pack_bf16x2(o, 0.0f) & 0xffffu);  // round to nearest even
        } else {
            out[oi] = o;
        }
        if (lse && d == 0) lse[(int64_t)h * r_total + row] = (M + __log2f(L)) * LN2;
    }
}

template <typename E, int D, int NQ>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* bias, const int32_t* pos,
                           const DecTable& t, int hq, int hkv, const float* gain, float c, void* out, float* lse,
                           int64_t r_total, void* ws, hipStream_t st) {
    const unsigned g1 = (unsigned)((t.n_waves + DEC_WAVES - 1) / DEC_WAVES);
    hipLaunchKernelGGL((decode_partial_kernel<E, D, NQ>), dim3(g1), dim3(64 * DEC_WAVES), 0, st, (const E*)q,
                       (const E*)k, (const E*)v, bias, pos, t, hq, hkv, gain, c, (float*)ws);
    hipLaunchKernelGGL((decode_combine_kernel<E, D, NQ>), dim3((unsigned)(t.n_rows * hq)), dim3(CB_THREADS), 0, st, t, hq,
                       hkv, (const float*)ws, (E*)out, lse, r_total);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_decode_d(int nq, const void* q, const void* k, const void* v, const float* bias,
                           const int32_t* pos, const DecTable& t, int hq, int hkv, const float* gain, float c,
                           void* out, float* lse, int64_t r_total, void* ws, hipStream_t st) {
    if (nq <= 1) return launch_decode_t<E, D, 1>(q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st);
    if (nq <= 2) return launch_decode_t<E, D, 2>(q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st);
    if (nq <= 4) return launch_decode_t<E, D, 4>(q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st);
    return launch_decode_t<E, D, 8>(q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st);
}

}  // namespace

int decode_query_slots(int nq) { return nq <= 1 ? 1 : nq <= 2 ? 2 : nq <= 4 ? 4 : nq <= 8 ? 8 : 0; }

// Scratch of the allocation-free decode entry point: the split-KV partials
// live in this file-scope device array instead of a caller workspace. Each
// GPU the library runs on holds its own copy until the process ends. Host
// code never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and cached here.
static __device__ __align__(256) unsigned char scratch[TG_DECODE_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::atomic<void*> g_scratch_ptr[SCRATCH_MAX_DEVICES];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_decode(tg_dtype dt, const void* q, const void* k, const void* v, const float* bias,
                         const int32_t* pos, const DecTable& t, int hq, int hkv, int head_dim, const float* gain,
                         float tau, void* out, float* lse, int64_t r_total, void* ws, hipStream_t st) {
    if (t.n_waves == 0) return hipSuccess;
    const float c = LOG2E / (sqrtf((float)head_dim) * tau);
    if (dt == TG_BF16)
        return head_dim == 128 ? launch_decode_d<uint16_t, 128>(t.nq_max, q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st)
                               : launch_decode_d<uint16_t, 64>(t.nq_max, q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st);
    return head_dim == 128 ? launch_decode_d<float, 128>(t.nq_max, q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st)
                           : launch_decode_d<float, 64>(t.nq_max, q, k, v, bias, pos, t, hq, hkv, gain, c, out, lse, r_total, ws, st);
}

}  // namespace tg
