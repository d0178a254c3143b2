// Device-side helpers shared by the HIP kernels: MFMA operand types,
// direct global->LDS loads, explicit vector-memory waits and a workgroup
// barrier that does not drain in-flight prefetches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global->LDS loads (global_load_lds_dwordx4 / _dword): lane l's 16
// (or 4) bytes land at LDS address m0 + 16*l (or 4*l); nothing is written to
// VGPRs. Issued from inline asm so that the compiler's conservative LDS-DMA
// tracking (which makes every LDS read wait for all DMA in flight, including
// a ring's next-stage prefetch) stays out of the pipelines; those order
// themselves with explicit wait_vmcnt. The compiler's own waits can only get
// stronger from this, since it undercounts the loads in flight.
// The compiler reserves m0 and may keep a value of its own there, so every
// block saves m0 into a scratch SGPR, sets it for the load and restores it
// before returning control: m0 is unchanged across each statement, which is
// what the compiler assumes of an inline asm that does not list it.
__device__ __forceinline__ void dma16(const void* g, const LDS_AS void* l) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(m0), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, const LDS_AS void* l) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(m0), "v"(g) : "memory");
}
// The same with a wave-uniform 64-bit base (SGPR pair), a per-lane 32-bit
// byte offset and the LDS destination as a plain LDS byte address.
__device__ __forceinline__ void dma16_so(const void* sbase, uint32_t voff, uint32_t lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma4_so(const void* sbase, uint32_t voff, uint32_t lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
}
// The same with m0 = lds_base + IMM (one scalar add, no separate move).
template <int IMM>
__device__ __forceinline__ void dma16_so_at(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %1, %4\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(lds_base), "v"(voff), "s"(sbase), "n"(IMM) : "memory", "scc");
}
template <int IMM>
__device__ __forceinline__ void dma4_so_at(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %1, %4\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(lds_base), "v"(voff), "s"(sbase), "n"(IMM) : "memory", "scc");
}

// LDS byte address of a __shared__ object (the cast of a variable's address
// needs no null check, unlike a cast of an arbitrary generic pointer).
#define LDS_ADDR(obj) ((uint32_t)(uintptr_t)(LDS_AS const char*)(obj))

// Workgroup barrier for LDS rings. __syncthreads() would also wait for every
// outstanding global->LDS load (including prefetches of later stages); here
// each wave waits for exactly the loads it needs (wait_vmcnt) and for its
// own LDS reads, and the compiler is kept from moving memory accesses
// across the barrier.
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

}  // namespace tg
