// Helpers for LDS rings fed by direct-to-LDS loads (gfx950): the load
// itself, explicit load-counter waits, the ring barrier and the row swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

#define LDS_AS __attribute__((address_space(3)))

// s_waitcnt with a run-time vector-memory count (the other counters left
// unconstrained); the instruction takes an immediate, hence the switch.
__device__ __forceinline__ void wait_vmcnt(int n)
{
#define MOE_VMCNT(N)                                                                       \
    case N:                                                                                \
        __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8)); \
        break;
    switch (n) {
        MOE_VMCNT(0) MOE_VMCNT(1) MOE_VMCNT(2) MOE_VMCNT(3) MOE_VMCNT(4) MOE_VMCNT(5)
        MOE_VMCNT(6) MOE_VMCNT(7) MOE_VMCNT(8) MOE_VMCNT(9) MOE_VMCNT(10) MOE_VMCNT(11)
        MOE_VMCNT(12) MOE_VMCNT(13) MOE_VMCNT(14) MOE_VMCNT(15) MOE_VMCNT(16) MOE_VMCNT(17)
        MOE_VMCNT(18) MOE_VMCNT(19) MOE_VMCNT(20) MOE_VMCNT(21) MOE_VMCNT(22) MOE_VMCNT(23)
        MOE_VMCNT(24) MOE_VMCNT(25) MOE_VMCNT(26) MOE_VMCNT(27) MOE_VMCNT(28) MOE_VMCNT(29)
        MOE_VMCNT(30) MOE_VMCNT(31) MOE_VMCNT(32) MOE_VMCNT(33) MOE_VMCNT(34) MOE_VMCNT(35)
        MOE_VMCNT(36) MOE_VMCNT(37) MOE_VMCNT(38) MOE_VMCNT(39) MOE_VMCNT(40) MOE_VMCNT(41)
        MOE_VMCNT(42) MOE_VMCNT(43) MOE_VMCNT(44) MOE_VMCNT(45) MOE_VMCNT(46) MOE_VMCNT(47)
        MOE_VMCNT(48) MOE_VMCNT(49) MOE_VMCNT(50) MOE_VMCNT(51) MOE_VMCNT(52) MOE_VMCNT(53)
        MOE_VMCNT(54) MOE_VMCNT(55) MOE_VMCNT(56) MOE_VMCNT(57) MOE_VMCNT(58) MOE_VMCNT(59)
        MOE_VMCNT(60) MOE_VMCNT(61) MOE_VMCNT(62)
    default:
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (15 << 8));
        break;
    }
#undef MOE_VMCNT
}

// Workgroup barrier for the LDS ring.  The wave's own LDS reads are drained
// first (the slot they read is refilled right after the barrier), and the
// empty asm statements keep the compiler from moving memory accesses across
// it.  No fence: the load counter is managed explicitly with wait_vmcnt.
__device__ __forceinline__ void ring_barrier()
{
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8)); // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One wave-wide direct-to-LDS load: every lane fetches 16 bytes from its own
// global address and the wave's 64 pieces land contiguously at LDS byte
// address lds_addr (wave-uniform, passed in M0).  Written as inline asm so
// that the compiler, which cannot tell the ring's slots apart, does not drain
// the whole load counter before every LDS read; the ring's waits are the
// explicit wait_vmcnt calls.  M0 is restored afterwards.  NT marks the load
// non-temporal, so the L2 keeps the line only briefly (for data that the
// launch reads once and that would otherwise push out data it re-reads).
template <bool NT = false>
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr)
{
    uint32_t saved;
    if constexpr (NT)
        asm volatile("s_mov_b32 %0, m0\n\t"
                     "s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %1, off nt\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(gptr), "s"(lds_addr)
                     : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\t"
                     "s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %1, off\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(gptr), "s"(lds_addr)
                     : "memory");
}

// 16-byte piece p of row r is stored at piece p ^ swz(r) of that row.
template <int RC>
__device__ __forceinline__ int swz(int r)
{
    static_assert(RC == 4 || RC == 8, "rows of 64 or 128 bytes");
    return RC == 8 ? (r & 7) : ((r >> 1) & 3);
}

} // namespace moe
