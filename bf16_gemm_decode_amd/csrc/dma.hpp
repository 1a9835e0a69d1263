// dma.hpp -- buffer descriptors, direct HBM -> LDS loads and the vector
// memory counter wait, shared by the kernels that stage tiles with them.
#pragma once

#include "common.hpp"

namespace migemm {

// Raw buffer descriptor words over [base, base + nbytes), wave-uniform:
// loads past nbytes return zero and never fault.  Word 3 selects 32-bit data
// format, no swizzle; the stride is zero (raw byte offsets).
__device__ inline u32x4 make_desc(const void *base, uint32_t nbytes)
{
    uint64_t a = (uint64_t)base;
    u32x4 d;
    d[0] = (uint32_t)uniform((int)(uint32_t)a);
    d[1] = (uint32_t)uniform((int)((uint32_t)(a >> 32) & 0xffffu));
    d[2] = (uint32_t)uniform((int)nbytes);
    d[3] = 0x00020000u;
    return d;
}

// Direct HBM -> LDS load of BYTES per lane: lane l's bytes land at LDS address
// lds + l*BYTES (M0 holds the wave-uniform base).  Only the 4- and 16-byte
// forms are used; their lane-linear placement and zero fill past the
// descriptor's records are what the kernel relies on.  Issued as inline
// assembly so that the compiler does not make every later LDS read wait for
// these loads: the kernel orders them itself with explicit vmcnt waits and a
// barrier before any wave reads the stage they fill.
template <int BYTES>
__device__ inline void dma_to_lds(u32x4 desc, uint32_t lds, uint32_t voff)
{
    static_assert(BYTES == 16 || BYTES == 4, "LDS load size");
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                     :: "v"(voff), "s"(lds), "s"(desc) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds"
                     :: "v"(voff), "s"(lds), "s"(desc) : "memory", "m0");
}

// The 16-byte form with the non-temporal hint, for data read exactly once
// (a weight matrix streamed past operands that are re-read from L2).
__device__ inline void dma16_to_lds_nt(u32x4 desc, uint32_t lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen nt lds"
                 :: "v"(voff), "s"(lds), "s"(desc) : "memory", "m0");
}

// The global-address form: lane l's 16 bytes at base + voff (base in SGPRs,
// voff a 32-bit lane offset) into LDS at `lds` + 16 l.  No range check, so
// only for loads known to lie inside their operand; it issues faster than
// the buffer form when the data comes from L2 (measured: 71-72 against 62-64
// GB/s per CU with 8 waves, 50-51 against 42 with 4; the same from HBM).
__device__ inline void gdma16_to_lds(const void *base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                 :: "v"(voff), "s"(lds), "s"(base) : "memory", "m0");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace migemm
