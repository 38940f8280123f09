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

// Sum over the 64 lanes of a wavefront, returned wave-uniform (in scalar
// registers): DPP adds within quads (lanes ^1, ^2) and rows of 16 (rotate by 4,
// then 8), then the four row totals are read out and added in row order.
__device__ __forceinline__ float wave_sum_uniform(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
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

// Short-sequence transcendental forms for the fusion prologue/epilogue, built on
// the hardware exp2/log2/rcp/rsqrt instructions (about 1 ulp each), so that the
// fused kernels keep the register budget of the plain ones.
__device__ __forceinline__ float exp_hw(float x) {
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);   // e^x = 2^(x log2 e)
}

// log(1 + y) for y >= 0 with the compensated form log(u) * y / (u - 1), u = 1 + y
// (Goldberg, "What every computer scientist should know about floating-point
// arithmetic", Theorem 4): the rounding of 1 + y cancels out of the ratio.
__device__ __forceinline__ float log1p_hw(float y) {
    const float u = 1.0f + y;
    if (u == 1.0f) return y;
    return __builtin_amdgcn_logf(u) * 0.693147180559945309f * (y * __builtin_amdgcn_rcpf(u - 1.0f));
}

// softplus(x) = max(x, 0) + log(1 + e^-|x|)
__device__ __forceinline__ float softplus_hw(float x) {
    return fmaxf(x, 0.f) + log1p_hw(exp_hw(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_hw(float x) {
    return __builtin_amdgcn_rcpf(1.0f + exp_hw(-x));
}

// gate and beta of V head h at flat index idx, with the optional prologue
// gate = -exp(A_log[h]) softplus(a + dt_bias[h]), beta = sigmoid(b) when A_log is set
// (then `gate`/`beta` hold the raw a/b).
// The same map from values already loaded: raw a, b and the head's A_log, dt_bias.
__device__ __forceinline__ void gate_beta_of(float a, float b, float A_log, float dt_bias, float* g, float* bt) {
    *g = -exp_hw(A_log) * softplus_hw(a + dt_bias);
    *bt = sigmoid_hw(b);
}

template <typename Tin>
__device__ __forceinline__ void gate_beta_at(const void* gate, const void* beta, const void* A_log,
                                             const void* dt_bias, size_t idx, int h, float* g, float* b) {
    float gv = to_f32(static_cast<const Tin*>(gate)[idx]);
    float bv = to_f32(static_cast<const Tin*>(beta)[idx]);
    if (A_log != nullptr) {
        gate_beta_of(gv, bv, to_f32(static_cast<const Tin*>(A_log)[h]), to_f32(static_cast<const Tin*>(dt_bias)[h]),
                     &gv, &bv);
    }
    *g = gv;
    *b = bv;
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

// Sequence that owns token p of row 0 under cu_seqlens (clamped entries), or -1.
__device__ __forceinline__ int token_owner(int p, int L, int N, const int32_t* cu) {
    int lo = 0, hi = N - 1, n = -1;
    while (lo <= hi) {  // last n whose clamped start is <= p
        const int mid = (lo + hi) >> 1;
        int st = cu[mid];
        st = st < 0 ? 0 : (st > L ? L : st);
        if (st <= p) { n = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    if (n < 0) return -1;
    const Seg sg = segment_of(n, L, cu);
    return p < sg.start + sg.len ? n : -1;
}

}  // namespace gdn
