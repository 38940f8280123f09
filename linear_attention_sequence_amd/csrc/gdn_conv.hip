// Step 1 of "MNN Model Support: Qwen3.5" §1.2 on its own: the depthwise causal
// Conv1D + SiLU over qkv [B, D, L], and the conv-state update of §1.4.
//
// conv1d_silu_kernel: one thread per (row, channel, token). Threads of a
// workgroup take consecutive tokens of one channel, so the reads of the
// channel-major input and the writes of y are coalesced; the K-1 overlapping
// reads of neighbouring tokens hit L1/L2. Tokens whose window reaches before the
// start of their sequence read the sequence's conv_state_in instead.
//
// conv_state_kernel: one thread per (sequence, channel) writes the K-1 most
// recent raw inputs of concat(conv_state_in[n], x[sequence n]).
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kConvTile = 256;

// Sequence that owns token p of row 0 under cu_seqlens (clamped entries), or -1.
__device__ __forceinline__ int sequence_of_token(int p, int L, int N, const int32_t* cu, Seg* seg) {
    int lo = 0, hi = N - 1, found = -1;
    while (lo <= hi) {  // last n whose clamped start is <= p
        const int mid = (lo + hi) >> 1;
        int st = cu[mid];
        st = st < 0 ? 0 : (st > L ? L : st);
        if (st <= p) { found = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    if (found < 0) return -1;
    *seg = segment_of(found, L, cu);
    if (p >= seg->start + seg->len) return -1;
    return found;
}

template <typename Tin>
__global__ __launch_bounds__(kConvTile) void conv1d_silu_kernel(ConvArgs a) {
    const int tiles = (a.L + kConvTile - 1) / kConvTile;
    const long long blk = blockIdx.x;
    const int tile = static_cast<int>(blk % tiles);
    const long long rc = blk / tiles;
    const int ch = static_cast<int>(rc % a.D);
    const int row = static_cast<int>(rc / a.D);
    const int p = tile * kConvTile + threadIdx.x;
    if (p >= a.L) return;
    Seg seg;
    int n;
    if (a.cu == nullptr) {
        n = row; seg.row = row; seg.start = 0; seg.len = a.L;
    } else {
        n = sequence_of_token(p, a.L, a.N, a.cu, &seg);
        if (n < 0) return;
    }
    const Tin* x = static_cast<const Tin*>(a.qkv) + (static_cast<size_t>(row) * a.D + ch) * a.L;
    const Tin* st = static_cast<const Tin*>(a.conv_in) + (static_cast<size_t>(n) * a.D + ch) * (kConvK - 1);
    const Tin* w = static_cast<const Tin*>(a.w) + static_cast<size_t>(ch) * kConvK;
    float wv[kConvK], win[kConvK];
    const int u = p - seg.start;  // token index inside its sequence
#pragma unroll
    for (int j = 0; j < kConvK; ++j) {
        wv[j] = to_f32(w[j]);
        const int m = u + j;      // position in concat(state, x[seq])
        win[j] = (m < kConvK - 1) ? to_f32(st[m]) : to_f32(x[seg.start + m - (kConvK - 1)]);
    }
    a.y[(static_cast<size_t>(row) * a.D + ch) * a.L + p] = conv_silu(wv, win);
}

template <typename Tin>
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a) {
    const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<long long>(a.N) * a.D) return;
    const int n = static_cast<int>(idx / a.D);
    const int ch = static_cast<int>(idx - static_cast<long long>(n) * a.D);
    const Seg seg = segment_of(n, a.L, a.cu);
    const Tin* x = static_cast<const Tin*>(a.qkv) + (static_cast<size_t>(seg.row) * a.D + ch) * a.L;
    const Tin* st = static_cast<const Tin*>(a.conv_in) + (static_cast<size_t>(n) * a.D + ch) * (kConvK - 1);
    Tin* co = static_cast<Tin*>(a.conv_out) + (static_cast<size_t>(n) * a.D + ch) * (kConvK - 1);
#pragma unroll
    for (int j = 0; j < kConvK - 1; ++j) {
        const int m = seg.len + j;
        co[j] = (m < kConvK - 1) ? st[m] : x[seg.start + m - (kConvK - 1)];
    }
}

template <typename Tin>
static hipError_t launch_conv_t(const ConvArgs& a, hipStream_t stream) {
    const long long tiles = (a.L + kConvTile - 1) / kConvTile;
    const long long blocks = tiles * a.D * a.B;
    void* args[] = {const_cast<ConvArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_silu_kernel<Tin>),
                           dim3(static_cast<unsigned>(blocks)), dim3(kConvTile), args, 0, stream);
}

hipError_t launch_conv1d_silu(const ConvArgs& a, int in_dtype, hipStream_t stream) {
    return in_dtype == 1 ? launch_conv_t<bf16_t>(a, stream) : launch_conv_t<float>(a, stream);
}

template <typename Tin>
static hipError_t launch_state_t(const ConvArgs& a, hipStream_t stream) {
    const long long blocks = (static_cast<long long>(a.N) * a.D + 255) / 256;
    void* args[] = {const_cast<ConvArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&conv_state_kernel<Tin>),
                           dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0, stream);
}

hipError_t launch_conv_state(const ConvArgs& a, int in_dtype, hipStream_t stream) {
    return in_dtype == 1 ? launch_state_t<bf16_t>(a, stream) : launch_state_t<float>(a, stream);
}

}  // namespace gdn
