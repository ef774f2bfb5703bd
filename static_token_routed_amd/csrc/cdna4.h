// Small gfx950 (CDNA4) device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace l3 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline uint32_t f2bf(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ inline uint32_t pack2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// not for its outstanding global loads (HIP's __syncthreads also drains those,
// which would cap every prefetch at one barrier).  The empty asm statements
// keep the compiler from moving memory operations across it.
__device__ inline void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// LDS byte offset of a __shared__ object.
template <typename T>
__device__ inline uint32_t lds_addr(T *p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void *)p);
}

// Asynchronous 16-byte copy global -> LDS (global_load_lds_dwordx4): lane l's
// 16 bytes land at lds_base + 16 * l; lds_base must be uniform across the wave.
// Completion is tracked by vmcnt only; callers wait with wait_vmcnt<N>() before
// a barrier.  Written as asm so the compiler does not treat later LDS reads as
// depending on every copy still in flight.
__device__ inline void async_ld16(const void *gptr, uint32_t lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(m0v), "v"(gptr)
                     : "memory");
}

// Asynchronous 4-byte copy global -> LDS (global_load_lds_dword): lane l's 4 bytes
// land at lds_base + 4 * l; otherwise as async_ld16.
__device__ inline void async_ld4(const void *gptr, uint32_t lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                     :
                     : "s"(m0v), "v"(gptr)
                     : "memory");
}

// Two wave-uniform 32-bit loads through the scalar cache, waited for in the same
// statement: unlike a vector load they leave vmcnt alone, so a loop that keeps
// asynchronous copies in flight can look up addresses without draining them.
__device__ inline void scalar_ld2(const int32_t *p0, const int32_t *p1, int &v0, int &v1) {
    const uint64_t b0 = (uint64_t)(uintptr_t)p0, b1 = (uint64_t)(uintptr_t)p1;
    const uint64_t s0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b0 >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b0);
    const uint64_t s1 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b1 >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b1);
    __asm__ volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
                     : "=&s"(v0), "=&s"(v1)
                     : "s"(s0), "s"(s1)
                     : "memory");
}

// The same copy addressed as a wave-uniform 64-bit base plus a 32-bit per-lane
// byte offset (the scalar-base form of the instruction).
__device__ inline void async_ld16_sb(const void *sbase, uint32_t voff, uint32_t lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    // readfirstlane returns int: widen through uint32_t so the low half is not sign-extended
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(m0v), "v"(voff), "s"(sb)
                     : "memory");
}

// Both copies with the LDS destination given as a wave-uniform base plus the
// compile-time byte offset OFF (added to M0 inside the asm, so a run of copies
// needs one scalar register for its destinations, not one per copy).
template <uint32_t OFF>
__device__ inline void async_ld16_o(const void *gptr, uint32_t lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    __asm__ volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(m0v), "v"(gptr), "i"(OFF)
                     : "memory", "scc");
}

// async_ld16_o with the non-temporal hint (nt): for rows read once per call (cold
// table rows, the tokens' x rows), so they do not push out of L2 the rows that other
// workgroups are about to read again.
template <uint32_t OFF>
__device__ inline void async_ld16_o_nt(const void *gptr, uint32_t lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    __asm__ volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                     :
                     : "s"(m0v), "v"(gptr), "i"(OFF)
                     : "memory", "scc");
}

template <uint32_t OFF>
__device__ inline void async_ld16_sbo(const void *sbase, uint32_t voff, uint32_t lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    __asm__ volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(m0v), "v"(voff), "s"(sb), "i"(OFF)
                     : "memory", "scc");
}

// Raw buffer resource (gfx9 layout): base address, no stride, num_records bytes;
// loads at offsets >= num_records return zeros instead of touching memory.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ inline i32x4_t make_rsrc(const void *base, uint32_t num_records) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    i32x4_t r;
    r.x = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    r.y = (int32_t)(__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffff);
    r.z = (int32_t)__builtin_amdgcn_readfirstlane(num_records);
    r.w = 0x00020000;
    return r;
}

// Asynchronous 16-byte copy global -> LDS through a buffer resource
// (buffer_load_dwordx4 ... offen lds): lane l reads rsrc base + voff + soff and its
// 16 bytes land at lds_base + 16 * l (lds_base uniform).  Lanes whose voff is past
// num_records deliver zeros.  Completion is tracked by vmcnt only, as for async_ld16.
__device__ inline void async_buf16(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(m0v), "v"(voff), "s"(rsrc), "s"(so)
                     : "memory");
}

// This lane's index in its wavefront, computed afresh (v_mbcnt) and hidden from the
// optimiser, so values derived from it are recomputed where they are needed instead
// of being kept live (or spilled) across long stretches of a kernel.
__device__ inline uint32_t fresh_lane_id() {
    uint32_t l;
    __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// compile-time loop: f(std::integral_constant<int, I>) for I in [0, N)
template <int N, int I = 0, typename F>
__device__ inline void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// s_waitcnt vmcnt(N) (N <= 63), other counters untouched.
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace l3
