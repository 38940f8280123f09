// Chunk slots of packed prompts (cu_seqlens). The chunks of every sequence take
// consecutive slots, sequence after sequence, so sequence n's first slot is the number
// of chunks of the sequences before it. One workgroup of each call writes that
// exclusive prefix sum once (cbase[0..N], cbase[N] = every chunk of the call); the
// kernels after it find a slot's sequence by binary search and a sequence's first slot
// by one load, where summing the chunk counts of the sequences before it in every
// workgroup would cost O(N) per workgroup and O(N^2) per call.
#pragma once
#include "gdn_common.hpp"

namespace gdn {

// cbase[n] = min(chunks of sequences 0 .. n-1, nc_max) for n = 0 .. N, the chunk counts
// taken from the clamped cu_seqlens entries (segment_of). Summed in 64 bits and clamped
// to the slot count, so the table is nondecreasing and no entry overflows even for
// overlapping entries; a sequence whose first slot is below nc_max has its exact base.
// Called by every thread of one workgroup of 256 threads (four waves).
__device__ inline void write_chunk_bases(int N, int L, const int32_t* cu, int C, int nc_max, int* cbase) {
    __shared__ long long s_wave[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    long long run = 0;                                   // chunks of the earlier rounds
    for (int n0 = 0; n0 < N; n0 += 256) {
        const int n = n0 + tid;
        long long nc = 0;
        if (n < N) nc = (segment_of(n, L, cu).len + C - 1) / C;
        long long x = nc;                                // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const long long y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) s_wave[wave] = x;
        __syncthreads();
        long long before = run;
        for (int w = 0; w < wave; ++w) before += s_wave[w];
        if (n < N) cbase[n] = static_cast<int>(min(before + x - nc, static_cast<long long>(nc_max)));
        run += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
        __syncthreads();                                 // s_wave is read before the next round
    }
    if (tid == 0) cbase[N] = static_cast<int>(min(run, static_cast<long long>(nc_max)));
}

// Sequence n of chunk slot id (0 <= id < nc_max) and the chunk's index c inside it;
// false for a slot no sequence fills.
__device__ __forceinline__ bool chunk_slot(int id, int N, const int* cbase, int* n_out, int* c_out) {
    int lo = 0, hi = N - 1, n = -1;
    while (lo <= hi) {                                   // last n whose first slot is <= id
        const int mid = (lo + hi) >> 1;
        if (cbase[mid] <= id) { n = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    if (n < 0 || id >= cbase[n + 1]) return false;
    *n_out = n;
    *c_out = id - cbase[n];
    return true;
}

}  // namespace gdn
