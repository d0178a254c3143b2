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
//  * A workgroup is 4 waves; each wave owns 32 query rows of one query head.
//    The 4 waves of a workgroup share one KV head (GQA): with G = Hq/Hkv
//    query heads per KV head, a workgroup holds gcd(G,4) heads x (4/gcd)
//    32-row slabs, so each K/V tile staged in LDS feeds 4 waves.
//  * S^T = K Q^T: K (keys x d) is the A operand read from LDS, Q^T the B
//    operand kept in registers for the whole key loop. The 32x32 result
//    layout puts one query column in each lane (keys down its registers),
//    so the softmax row statistics are per lane, with one exchange between
//    lanes l and l^32.
//  * O^T += V^T P^T: the lane's own S^T registers, rounded to bf16, are
//    exactly the B operand once keys are taken in the order
//    16s + 8(e/4) + 4(l/32) + e%4. V is written to LDS transposed with the
//    same key order (bits 2 and 3 of the key index swapped), so each A
//    operand is one 16-byte LDS read.
//  * Logits are built in the exp2 domain with one FMA per element:
//    x = acc * (log2 e / (sqrt(D) tau)) + gain[h] log2 e * bias[j].
//  * Causality compares original positions element-wise (exact for any
//    non-decreasing positions, repeats included); key tiles past the
//    workgroup's last visible key are skipped, and waves whose queries
//    precede a whole tile skip its math.
//  * Work items run longest-first (last query blocks of a prompt first).
//
// fp32 path: one thread per query row, K/V tiles in LDS, plain fp32 FMA.
#include "tg_internal.hpp"

#include <limits.h>

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int BN = 64;  // keys per tile

__device__ __forceinline__ uint16_t f2bf(float f) {
    // round to nearest even (inputs are finite)
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Index of the key tile one past the last tile a query block can see:
// tiles up to the block's last row, extended while the next tile starts at
// a position not after the block's last position (repeated positions).
__device__ __forceinline__ int key_tile_end(const int32_t* __restrict__ pos, int64_t off, int n,
                                            int q_last) {
    int kt_end = q_last / BN + 1;
    const int32_t pl = pos[off + q_last];
    while (kt_end * BN < n && pos[off + kt_end * BN] <= pl) ++kt_end;
    return kt_end;
}

struct Item {
    int seg, qb, kvh, hg;
};

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

template <int D>
__global__ __launch_bounds__(256) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ bias, const int32_t* __restrict__ pos, AttnTable t, int hq, int hkv,
    int hw, const float* __restrict__ gain, float qk_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
    constexpr int KST = D + 8;    // K tile row stride (bf16)
    constexpr int VST = BN + 8;   // V^T tile row stride (bf16)
    constexpr int KS = D / 16;    // k-steps of the QK^T contraction
    constexpr int DB = D / 32;    // 32-wide d blocks of the output
    constexpr int KU = (BN * D / 8) / 256;        // K 16-byte units per thread
    constexpr int VU = (BN / 2) * (D / 8) / 256;  // V key-pair units per thread
    __shared__ __attribute__((aligned(16))) uint16_t ks_[BN * KST];
    __shared__ __attribute__((aligned(16))) uint16_t vt_[D * VST];
    __shared__ float bs_[BN];
    __shared__ int32_t ps_[BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int G = hq / hkv;
    const int ngroups = G / hw;
    const int rw = 4 / hw;  // 32-row slabs per workgroup
    const int bm = 32 * rw;

    const Item it = decode_item(t, blockIdx.x, hkv, ngroups);
    const int64_t off = t.s[it.seg].kept_off;
    const int n = t.s[it.seg].n;
    const int slab = wave / hw;
    const int h = it.kvh * G + it.hg * hw + (wave % hw);
    const int i0 = it.qb * bm + slab * 32;  // first query row of this wave (segment-relative)
    const int q_last_blk = min(n, it.qb * bm + bm) - 1;
    const int kt_end = key_tile_end(pos, off, n, q_last_blk);

    // This lane's query row (clamped for the ragged tail; never stored).
    const int qi = min(i0 + l32, n - 1);
    const int32_t my_pos = pos[off + qi];
    const int32_t wave_pos_lo = pos[off + min(i0, n - 1)];
    const int32_t wave_pos_hi = pos[off + min(i0 + 31, n - 1)];
    const float c = qk_scale * LOG2E;
    const float gl2 = gain[h] * LOG2E;

    bf16x8 qf[KS];
    {
        const uint16_t* qrow = q + ((off + qi) * hq + h) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(qrow + s * 16);
    }

    // Cooperative tile loader (registers -> LDS).
    const int64_t kv_row_stride = (int64_t)hkv * D;
    const uint16_t* kbase = k + (off * hkv + it.kvh) * D;
    const uint16_t* vbase = v + (off * hkv + it.kvh) * D;
    uint4 kr[KU], vr[VU][2];
    float br = 0.0f;
    int32_t pr = 0;
    auto load_tile = [&](int kt) {
        const int j0 = kt * BN;
#pragma unroll
        for (int i = 0; i < KU; ++i) {
            const int u = tid + 256 * i;
            const int key = u / (D / 8), dc = u % (D / 8);
            const int j = min(j0 + key, n - 1);
            kr[i] = *(const uint4*)(kbase + (int64_t)j * kv_row_stride + dc * 8);
        }
#pragma unroll
        for (int i = 0; i < VU; ++i) {
            const int u = tid + 256 * i;
            const int p = u % (BN / 2), dc = u / (BN / 2);
            const int ja = min(j0 + 2 * p, n - 1), jb = min(j0 + 2 * p + 1, n - 1);
            vr[i][0] = *(const uint4*)(vbase + (int64_t)ja * kv_row_stride + dc * 8);
            vr[i][1] = *(const uint4*)(vbase + (int64_t)jb * kv_row_stride + dc * 8);
        }
        if (tid < BN) {
            const int j = j0 + tid;
            br = bias[off + min(j, n - 1)];
            pr = (j < n) ? pos[off + j] : INT_MAX;
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < KU; ++i) {
            const int u = tid + 256 * i;
            const int key = u / (D / 8), dc = u % (D / 8);
            *(uint4*)&ks_[key * KST + dc * 8] = kr[i];
        }
#pragma unroll
        for (int i = 0; i < VU; ++i) {
            const int u = tid + 256 * i;
            const int p = u % (BN / 2), dc = u / (BN / 2);
            const int key = 2 * p;
            const int slot = (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
            const uint32_t a[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
            const uint32_t b[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // d = dc*8 + 2e and dc*8 + 2e + 1: pair (key, key+1) per row
                const uint32_t lo = (a[e] & 0xffffu) | (b[e] << 16);
                const uint32_t hi = (a[e] >> 16) | (b[e] & 0xffff0000u);
                *(uint32_t*)&vt_[(dc * 8 + 2 * e) * VST + slot] = lo;
                *(uint32_t*)&vt_[(dc * 8 + 2 * e + 1) * VST + slot] = hi;
            }
        }
        if (tid < BN) {
            bs_[tid] = br;
            ps_[tid] = pr;
        }
    };

    f32x16 acc_o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc_o[b][j] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    load_tile(0);
    store_tile();
    __syncthreads();

    for (int kt = 0; kt < kt_end; ++kt) {
        const bool more = kt + 1 < kt_end;
        // Prefetch the next tile into registers (unconditional: the last
        // iteration re-reads its own tile, keeping the registers in place).
        load_tile(more ? kt + 1 : kt);

        // A wave whose every query precedes the whole tile skips it.
        if (ps_[0] <= wave_pos_hi) {
            f32x16 acc_s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) acc_s[kb][j] = 0.0f;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 a = *(const bf16x8*)&ks_[(kb * 32 + l32) * KST + s * 16 + 8 * hh];
                    acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc_s[kb], 0, 0, 0);
                }
            }
            const bool need_mask = ps_[BN - 1] > wave_pos_lo;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
                    float x = fmaf(acc_s[kb][j], c, gl2 * bs_[key]);
                    if (need_mask && ps_[key] > my_pos) x = -INFINITY;
                    acc_s[kb][j] = x;
                    mx = fmaxf(mx, x);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            const float corr = exp2f(m_run - m_use);
            float lsum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float p = exp2f(acc_s[kb][j] - m_use);
                    acc_s[kb][j] = p;
                    lsum += p;
                }
            l_run = l_run * corr + lsum;
            m_run = m_new;
            // Rescale O only when some row's running max moved (corr == 1
            // exactly otherwise, so skipping the multiply changes nothing).
            if (__any(corr != 1.0f)) {
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc_o[b][j] *= corr;
            }

            // P^T as B operands: k-step s uses S^T registers 8*(s%2) .. +8 of block s/2.
            bf16x8 pf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf2(acc_s[s >> 1][8 * (s & 1) + 2 * e], acc_s[s >> 1][8 * (s & 1) + 2 * e + 1]);
                pf[s] = __builtin_bit_cast(bf16x8, w);
            }
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 a = *(const bf16x8*)&vt_[(b * 32 + l32) * VST + s * 16 + 8 * hh];
                    acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s], acc_o[b], 0, 0, 0);
                }
        }
        __syncthreads();
        if (more) {
            store_tile();
            __syncthreads();
        }
    }

    // Epilogue: normalise, round, store. Register j of d-block b holds
    // d = 32b + 8(j/4) + 4hh + j%4 of query row i0 + l32.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    const int row = i0 + l32;
    if (row < n) {
        uint16_t* orow = out + ((off + row) * hq + h) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * b + 8 * g4 + 4 * hh;
                uint2 w;
                w.x = pack_bf2(acc_o[b][4 * g4 + 0] * inv, acc_o[b][4 * g4 + 1] * inv);
                w.y = pack_bf2(acc_o[b][4 * g4 + 2] * inv, acc_o[b][4 * g4 + 3] * inv);
                *(uint2*)(orow + d) = w;
            }
        if (lse && hh == 0) lse[(int64_t)h * t.m_total + off + row] = (m_run + log2f(l_tot)) * LN2;
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

int gcd4(int g) { return (g % 4 == 0) ? 4 : ((g % 2 == 0) ? 2 : 1); }

}  // namespace

int attention_heads_per_item(tg_dtype dt, int hq, int hkv) {
    return dt == TG_F32 ? 1 : gcd4(hq / hkv);
}

int attention_block_rows(tg_dtype dt, int hq, int hkv) {
    return dt == TG_F32 ? 64 : 32 * (4 / gcd4(hq / hkv));
}

hipError_t launch_attention(tg_dtype dt, const void* q, const void* k, const void* v,
                            const float* bias, const int32_t* pos, const AttnTable& t, int hq,
                            int hkv, int head_dim, const float* gain, float tau, void* out,
                            float* lse, hipStream_t st) {
    if (t.n_items == 0) return hipSuccess;
    const float qk_scale = 1.0f / (sqrtf((float)head_dim) * tau);
    const dim3 grid((unsigned)t.n_items);
    if (dt == TG_BF16) {
        const int hw = gcd4(hq / hkv);
        if (head_dim == 128)
            hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, st, (const uint16_t*)q,
                               (const uint16_t*)k, (const uint16_t*)v, bias, pos, t, hq, hkv, hw,
                               gain, qk_scale, (uint16_t*)out, lse);
        else
            hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, st, (const uint16_t*)q,
                               (const uint16_t*)k, (const uint16_t*)v, bias, pos, t, hq, hkv, hw,
                               gain, qk_scale, (uint16_t*)out, lse);
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
