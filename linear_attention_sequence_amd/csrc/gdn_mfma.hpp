// MFMA helpers for gfx950 (CDNA4, wave64).
//
// v_mfma_f32_16x16x32_f16: D[16x16] += A[16x32] * B[32x16], fp16 operands, fp32
// accumulation. Operand layout per lane l (g = l / 16):
//   A: row l % 16, eight k values (k slot 8g + e, e = 0..7)
//   B: column l % 16, the same eight k slots
//   C/D: column l % 16, rows 4g + e (e = 0..3)
// Any one-to-one assignment of logical k indices to the 32 k slots gives the
// same product as long as A and B use the same assignment; the kernels use
// that freedom to feed an accumulator tile straight back in as a B operand.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma16x16x32(const f16x8& a, const f16x8& b, const f32x4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// max over the wave of non-negative values, returned wave-uniform. Non-negative
// IEEE floats order like their bit patterns, so the reduction runs on integers:
// DPP within quads (lanes ^1, ^2) and rows (rotate by 4, 8), then the four row
// results are read out to scalars.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    int v = __float_as_int(x);
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));  // row_ror:4
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));  // row_ror:8
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return __int_as_float(max(max(r0, r1), max(r2, r3)));
}

// Power-of-two scale that brings max|x| into [2^14, 2^15): inside fp16's range
// with room to spare. Returns the exponent e; values are stored as x * 2^-e and
// results multiplied back by 2^e (both exact). The exponent is kept >= -100 so
// that 2^-e stays finite when max|x| is far below fp32's normal range (a state
// map that has decayed for many chunks): values under 2^-124 then flush to zero
// in fp16, which is at most 2^-39 of the largest one.
__device__ __forceinline__ int pow2_exponent(float maxabs) {
    if (!(maxabs > 0.f) || !isfinite(maxabs)) return 0;
    int ex;
    frexpf(maxabs, &ex);  // maxabs = m * 2^ex, m in [0.5, 1)
    return ex - 15 < -100 ? -100 : ex - 15;
}

}  // namespace gdn
