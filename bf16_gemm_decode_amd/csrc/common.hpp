// common.hpp -- shared types and small device helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace migemm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned short u16x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

#define MIGEMM_LDS __attribute__((address_space(3)))

// Element types: 16-bit (in and out), and 8-bit inputs (OCP FP8 E4M3, OCP
// FP8 E5M2, INT8) whose GEMMs write BF16 of scale x accumulator.
enum { DT_F16 = 0, DT_BF16 = 1, DT_F8E4M3 = 2, DT_F8E5M2 = 3, DT_I8 = 4 };
constexpr bool dt_is_8bit(int dt) { return dt >= DT_F8E4M3; }

// Offsets at or beyond a buffer descriptor's record count read as zero; this
// value is beyond every record count the library builds (they are < 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int64_t kMaxRecords = 0x7fffffff;

// Raw buffer descriptor over [base, base + nbytes): loads past nbytes return
// zero and never fault.  Word 3 selects 32-bit data format, no swizzle.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int)nbytes, 0x00020000);
}

__device__ inline uint32_t clamp_records(int64_t nbytes)
{
    return (uint32_t)(nbytes < 0 ? 0 : (nbytes > kMaxRecords ? kMaxRecords : nbytes));
}

// FP32 -> 16-bit output, round to nearest even (the hardware converts in the
// default rounding mode; v_cvt_f16_f32 and v_cvt_pk_bf16_f32).
template <int DT>
__device__ inline unsigned short to_out(float x)
{
    if constexpr (DT == DT_F16) {
        _Float16 h = (_Float16)x;
        return __builtin_bit_cast(unsigned short, h);
    } else {
        __bf16 h = (__bf16)x;
        return __builtin_bit_cast(unsigned short, h);
    }
}

// The 16-bit output of one accumulator: 16-bit inputs round it to their own
// format; 8-bit inputs write BF16 of scale x accumulator (an INT8
// accumulator holds the bits of an int32; it is converted to FP32 first).
template <int DT>
__device__ inline unsigned short out16(float acc, float scale)
{
    if constexpr (!dt_is_8bit(DT)) {
        return to_out<DT>(acc);
    } else if constexpr (DT == DT_I8) {
        return to_out<DT_BF16>((float)__builtin_bit_cast(int, acc) * scale);
    } else {
        return to_out<DT_BF16>(acc * scale);
    }
}

// 16-bit input element -> FP32 (exact)
template <int DT>
__device__ inline float from16(unsigned short v)
{
    if constexpr (DT == DT_F16)
        return (float)__builtin_bit_cast(_Float16, v);
    else
        return __builtin_bit_cast(float, (unsigned)v << 16);
}

// Wave-uniform value in a scalar register.
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace migemm
