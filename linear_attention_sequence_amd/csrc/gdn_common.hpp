// Device-side helpers shared by the Gated DeltaNet kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kConvK = 4;   // conv taps supported by the kernels
constexpr int kWave = 64;   // CDNA wavefront width

// Native 4 x fp32 vector (the form the nontemporal builtins accept).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Input storage types. bf16 is carried as raw bits; widening to fp32 is exact.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// Sum over the 64 lanes of a wavefront; every lane receives the total. The
// butterfly order is fixed, so the result does not depend on which wave runs it.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Depthwise causal conv of one channel at one position followed by SiLU:
// silu(sum_j w[j] * win[j]) where win[K-1] is the current token. The sum is
// taken in tap order with explicit fused multiply-adds.
__device__ __forceinline__ float conv_silu(const float* w, const float* win) {
    float acc = w[0] * win[0];
#pragma unroll
    for (int j = 1; j < kConvK; ++j) acc = __fmaf_rn(w[j], win[j], acc);
    return acc / (1.0f + expf(-acc));
}

// Sequence n of a launch: row, first token and length. With cu_seqlens the
// entries are clamped into [0, L] and a decreasing pair is an empty sequence.
struct Seg { int row, start, len; };
__device__ __forceinline__ Seg segment_of(int n, int L, const int32_t* cu) {
    Seg s;
    if (cu == nullptr) { s.row = n; s.start = 0; s.len = L; return s; }
    int a = cu[n], b = cu[n + 1];
    a = a < 0 ? 0 : (a > L ? L : a);
    b = b < 0 ? 0 : (b > L ? L : b);
    s.row = 0; s.start = a; s.len = b > a ? b - a : 0;
    return s;
}

}  // namespace gdn
