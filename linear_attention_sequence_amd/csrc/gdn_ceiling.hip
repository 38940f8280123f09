// Measurement kernels: achievable HBM read / write / copy rates and the MFMA
// throughput of the device (see include/gdn_ceiling.h). Each is a simple form that
// keeps the unit under test saturated: 16-byte accesses, grid-stride or in blocks with
// up to 16 in flight per thread, for memory; eight independent accumulator chains per
// wave for MFMA.
#include "gdn_ceiling.h"

#include <hip/hip_runtime.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

// Plain grid-stride loops: consecutive lanes read consecutive 16-byte granules, each
// wave streams contiguous memory (an unrolled form that kept four strided granules in
// flight per thread measured slower).
__global__ __launch_bounds__(kThreads) void read_kernel(const f32x4* __restrict__ src, size_t n, float* sink) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) acc += src[i];
    if (acc.x == -1.2345e30f) sink[blockIdx.x] = acc.y + acc.z + acc.w;   // never true for the data read
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void write_kernel(f32x4* __restrict__ dst, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) {
        if constexpr (NT) __builtin_nontemporal_store(z, dst + i);
        else dst[i] = z;
    }
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) {
        if constexpr (NT) __builtin_nontemporal_store(src[i], dst + i);
        else dst[i] = src[i];
    }
}

// Blocked forms: workgroup b moves the contiguous block of U * 256 granules starting at
// granule b * U * 256, each thread's U granules 256 apart (every load instruction of a
// wave covers 1 KB of consecutive memory), all of a thread's loads issued before any of
// its stores (the pattern of the layer's commit kernel).
template <int U>
__global__ __launch_bounds__(kThreads) void read_blocked(const f32x4* __restrict__ src, float* sink) {
    const size_t base = static_cast<size_t>(blockIdx.x) * U * kThreads + threadIdx.x;
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[base + static_cast<size_t>(u) * kThreads];
    f32x4 acc = v[0];
#pragma unroll
    for (int u = 1; u < U; ++u) acc += v[u];
    if (acc.x == -1.2345e30f) sink[blockIdx.x] = acc.y + acc.z + acc.w;   // never true for the data read
}

template <bool NT, int U>
__global__ __launch_bounds__(kThreads) void write_blocked(f32x4* __restrict__ dst) {
    const size_t base = static_cast<size_t>(blockIdx.x) * U * kThreads + threadIdx.x;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (NT) __builtin_nontemporal_store(z, dst + base + static_cast<size_t>(u) * kThreads);
        else dst[base + static_cast<size_t>(u) * kThreads] = z;
    }
}

template <bool NT, int U>
__global__ __launch_bounds__(kThreads) void copy_blocked(const f32x4* __restrict__ src, f32x4* __restrict__ dst) {
    const size_t base = static_cast<size_t>(blockIdx.x) * U * kThreads + threadIdx.x;
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[base + static_cast<size_t>(u) * kThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (NT) __builtin_nontemporal_store(v[u], dst + base + static_cast<size_t>(u) * kThreads);
        else dst[base + static_cast<size_t>(u) * kThreads] = v[u];
    }
}

// One MFMA shape in a loop of 8 independent accumulator chains per wave: DT 0 fp16
// 16x16x32, 1 bf16 16x16x32, 2 fp16 32x32x16, 3 bf16 32x32x16. The library is built
// with the VGPR form of the MFMA instructions: with AGPR accumulators the 16x16x32
// chains were moved between registers every iteration, which halved the rate.
template <typename AB, typename ACC, ACC (*MF)(AB, AB, ACC)>
__device__ __forceinline__ float mfma_loop(AB a, AB b, int iters) {
    ACC c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = MF(a, b, c0); c1 = MF(a, b, c1); c2 = MF(a, b, c2); c3 = MF(a, b, c3);
        c4 = MF(a, b, c4); c5 = MF(a, b, c5); c6 = MF(a, b, c6); c7 = MF(a, b, c7);
    }
    const ACC t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < static_cast<int>(sizeof(ACC) / sizeof(float)); ++e) s += t[e];
    return s;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ f32x4 mf0(f16x8 a, f16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ f32x4 mf1(bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
__device__ f32x16 mf2(f16x8 a, f16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
__device__ f32x16 mf3(bf16x8 a, bf16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

template <int DT>
__global__ __launch_bounds__(kThreads) void mfma_kernel(float* sink, int iters) {
    const int lane = threadIdx.x & 63;
    float s;
    if constexpr (DT == 0 || DT == 2) {
        f16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = static_cast<_Float16>((lane + e) * 0.001f);
            b[e] = static_cast<_Float16>((lane - e) * 0.001f);
        }
        if constexpr (DT == 0) s = mfma_loop<f16x8, f32x4, mf0>(a, b, iters);
        else s = mfma_loop<f16x8, f32x16, mf2>(a, b, iters);
    } else {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = static_cast<__bf16>((lane + e) * 0.001f);
            b[e] = static_cast<__bf16>((lane - e) * 0.001f);
        }
        if constexpr (DT == 1) s = mfma_loop<bf16x8, f32x4, mf1>(a, b, iters);
        else s = mfma_loop<bf16x8, f32x16, mf3>(a, b, iters);
    }
    if (s == -1.2345e30f) sink[blockIdx.x] = s;   // never true for these operands
}

bool grid_ok(int grid) { return grid >= 1 && grid <= (1 << 20); }
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
int launched() { return hipGetLastError() == hipSuccess ? 0 : 2; }

}  // namespace

extern "C" {

int gdn_ceiling_read(const void* src, size_t bytes, float* sink, int grid, void* stream) {
    if (!src || !sink || !grid_ok(grid) || bytes == 0 || bytes % 64 != 0 || !al16(src)) return 1;
    read_kernel<<<grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const f32x4*>(src), bytes / 16, sink);
    return launched();
}

int gdn_ceiling_write(void* dst, size_t bytes, int nontemporal, int grid, void* stream) {
    if (!dst || !grid_ok(grid) || bytes == 0 || bytes % 64 != 0 || !al16(dst)) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (nontemporal) write_kernel<true><<<grid, kThreads, 0, s>>>(static_cast<f32x4*>(dst), bytes / 16);
    else write_kernel<false><<<grid, kThreads, 0, s>>>(static_cast<f32x4*>(dst), bytes / 16);
    return launched();
}

int gdn_ceiling_copy(const void* src, void* dst, size_t bytes, int nontemporal, int grid, void* stream) {
    if (!src || !dst || !grid_ok(grid) || bytes == 0 || bytes % 64 != 0 || !al16(src) || !al16(dst)) return 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const f32x4* sp = static_cast<const f32x4*>(src);
    f32x4* dp = static_cast<f32x4*>(dst);
    if (nontemporal) copy_kernel<true><<<grid, kThreads, 0, s>>>(sp, dp, bytes / 16);
    else copy_kernel<false><<<grid, kThreads, 0, s>>>(sp, dp, bytes / 16);
    return launched();
}

// blocked forms: per_thread 4, 8 or 16 granules; bytes a multiple of one block
static bool blocked_ok(size_t bytes, int per_thread) {
    if (per_thread != 4 && per_thread != 8 && per_thread != 16) return false;
    const size_t block = static_cast<size_t>(per_thread) * kThreads * 16;
    return bytes > 0 && bytes % block == 0 && bytes / block <= (static_cast<size_t>(1) << 20);
}

int gdn_ceiling_read_blocked(const void* src, size_t bytes, float* sink, int per_thread, void* stream) {
    if (!src || !sink || !blocked_ok(bytes, per_thread) || !al16(src)) return 1;
    const unsigned grid = static_cast<unsigned>(bytes / (static_cast<size_t>(per_thread) * kThreads * 16));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const f32x4* sp = static_cast<const f32x4*>(src);
    if (per_thread == 4) read_blocked<4><<<grid, kThreads, 0, s>>>(sp, sink);
    else if (per_thread == 8) read_blocked<8><<<grid, kThreads, 0, s>>>(sp, sink);
    else read_blocked<16><<<grid, kThreads, 0, s>>>(sp, sink);
    return launched();
}

int gdn_ceiling_write_blocked(void* dst, size_t bytes, int nontemporal, int per_thread, void* stream) {
    if (!dst || !blocked_ok(bytes, per_thread) || !al16(dst)) return 1;
    const unsigned grid = static_cast<unsigned>(bytes / (static_cast<size_t>(per_thread) * kThreads * 16));
    hipStream_t s = static_cast<hipStream_t>(stream);
    f32x4* dp = static_cast<f32x4*>(dst);
    if (nontemporal) {
        if (per_thread == 4) write_blocked<true, 4><<<grid, kThreads, 0, s>>>(dp);
        else if (per_thread == 8) write_blocked<true, 8><<<grid, kThreads, 0, s>>>(dp);
        else write_blocked<true, 16><<<grid, kThreads, 0, s>>>(dp);
    } else {
        if (per_thread == 4) write_blocked<false, 4><<<grid, kThreads, 0, s>>>(dp);
        else if (per_thread == 8) write_blocked<false, 8><<<grid, kThreads, 0, s>>>(dp);
        else write_blocked<false, 16><<<grid, kThreads, 0, s>>>(dp);
    }
    return launched();
}

int gdn_ceiling_copy_blocked(const void* src, void* dst, size_t bytes, int nontemporal, int per_thread, void* stream) {
    if (!src || !dst || !blocked_ok(bytes, per_thread) || !al16(src) || !al16(dst)) return 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return 1;
    const unsigned grid = static_cast<unsigned>(bytes / (static_cast<size_t>(per_thread) * kThreads * 16));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const f32x4* sp = static_cast<const f32x4*>(src);
    f32x4* dp = static_cast<f32x4*>(dst);
    if (nontemporal) {
        if (per_thread == 4) copy_blocked<true, 4><<<grid, kThreads, 0, s>>>(sp, dp);
        else if (per_thread == 8) copy_blocked<true, 8><<<grid, kThreads, 0, s>>>(sp, dp);
        else copy_blocked<true, 16><<<grid, kThreads, 0, s>>>(sp, dp);
    } else {
        if (per_thread == 4) copy_blocked<false, 4><<<grid, kThreads, 0, s>>>(sp, dp);
        else if (per_thread == 8) copy_blocked<false, 8><<<grid, kThreads, 0, s>>>(sp, dp);
        else copy_blocked<false, 16><<<grid, kThreads, 0, s>>>(sp, dp);
    }
    return launched();
}

int gdn_ceiling_mfma(float* sink, int grid, int iters, int dtype, void* stream) {
    if (!sink || !grid_ok(grid) || iters < 1 || dtype < 0 || dtype > 3) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == 0) mfma_kernel<0><<<grid, kThreads, 0, s>>>(sink, iters);
    else if (dtype == 1) mfma_kernel<1><<<grid, kThreads, 0, s>>>(sink, iters);
    else if (dtype == 2) mfma_kernel<2><<<grid, kThreads, 0, s>>>(sink, iters);
    else mfma_kernel<3><<<grid, kThreads, 0, s>>>(sink, iters);
    return launched();
}

int gdn_ceiling_device_info(int device, int* cus, int* clock_khz, int* mem_clock_khz, int* mem_bus_bits) {
    if (!cus || !clock_khz || !mem_clock_khz || !mem_bus_bits) return 1;
    if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 2;
    if (hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, device) != hipSuccess) return 2;
    if (hipDeviceGetAttribute(mem_clock_khz, hipDeviceAttributeMemoryClockRate, device) != hipSuccess) return 2;
    if (hipDeviceGetAttribute(mem_bus_bits, hipDeviceAttributeMemoryBusWidth, device) != hipSuccess) return 2;
    return 0;
}

}  // extern "C"
