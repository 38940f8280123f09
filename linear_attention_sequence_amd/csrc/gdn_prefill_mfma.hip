// Chunked prefill of the Gated DeltaNet layer on MFMA, d_k = d_v = 128
// ("MNN Model Support: Qwen3.5", §1.2 steps 1-5 over whole prompts, §1.3
// reverse GQA, §1.4 carried states).
//
// The chunk algebra is the one stated in gdn_prefill.hip (an exact rewrite of
// step 5 over chunks of C = 64 tokens). Here the dense products run on
// v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation); the state S,
// the triangular solve and every accumulation stay fp32. Operands whose scale
// is set by the data (the state S, the values v, U and the deltas) are brought
// into fp16's range with a power-of-two scale (exact to apply and to undo):
// chosen per chunk for v and U, and for S and the deltas per wave, kept from
// chunk to chunk while their maxima stay inside a window of fp16's range; q and
// k are unit-norm and P, W are bounded by them.
//
//   front_kernel   steps 1-4 for the q and k channels on a (32-token,
//                  128-channel) tile: coalesced channel-major loads, conv + SiLU,
//                  transpose through LDS, per-token L2 norms and the q scale;
//                  fp16 token-major q and k.
//   chunk_kernel   per (chunk, V head), all chunks in parallel: the head's values
//                  (conv + SiLU of its raw channel-major input; v is never stored),
//                  Gam (cumulative log-decay), the Gram matrices K K^T and Q K^T on MFMA,
//                  A and P, T = (I + A)^-1 by a blocked fp32 inverse (16 x 16
//                  diagonal blocks by substitution, off-diagonal blocks by
//                  block products), then W = T diag(beta exp(Gam)) K and
//                  U = T diag(beta) V on MFMA. Writes W, U, P, Gam and a
//                  transposed copy of the chunk's keys.
//   carry_kernel   per (sequence, V head): the state lives in registers in MFMA
//                  accumulator layout (each wave owns 16 of the 128 columns; a
//                  head takes one workgroup of 8 waves or two of 4; the columns
//                  of S evolve independently); chunk by
//                  chunk it forms Delta = U - W S, O = diag(exp(Gam)) Q S +
//                  P Delta and S = exp(Gam_last) S + K^T diag(exp(Gam_last -
//                  Gam)) Delta. The next chunk's operands stream into the other
//                  half of a double-buffered LDS stage with global_load_lds
//                  while the current chunk computes. Accumulator tiles are fed
//                  back as B operands without data movement by pairing the k
//                  slots of the MFMA with the accumulator rows they hold. A lone
//                  prompt with few heads runs in segments: a first pass (segment
//                  0, and each middle segment's state map and zero-entry state)
//                  and a second pass over segments 1 .. nseg - 1, whose workgroups
//                  first form their entry states from those maps.
#include <algorithm>

#include "gdn_common.hpp"
#include "gdn_launch.hpp"
#include "gdn_mfma.hpp"
#include "gdn_packed.hpp"
#include "gdn_prefill_plan.hpp"

namespace gdn {
namespace pf2 {

using plan::C;
using plan::COEF;
using plan::D;
using plan::kidx;
using plan::kMaxSeg;
using plan::kpos;
using plan::seg_begin;
using plan::Stage;
// 16- and 8-byte vectors that need only 4-byte alignment (global loads of several
// dwords need dword alignment only)
typedef unsigned u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef unsigned u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));   // a packed pair, operand of v_dot2_f32_bf16

constexpr int TT = 32;     // front-end tile (tokens): 19 KB of LDS, eight workgroups per CU
constexpr int RAW = TT + 5;  // raw tile row stride (floats): TT + 3 used, odd stride against bank conflicts

// Device view of the workspace (regions and sizes from plan::layout).
struct Ws {
    _Float16* qh;   // [Ttot, Hk, D] q_hat (normalised, scaled), features in k order
    _Float16* kh;   // [Ttot, Hk, D] k_hat, features in k order
    _Float16* W;    // [NC, Hv, C, D] features in k order
    _Float16* U;    // [NC, Hv, D, C] transposed, scaled by 2^-uexp
    _Float16* P;    // [NC, Hv, C, C] keys in k order
    _Float16* KT;   // [NC, Hk, D, C] keys of the chunk, transposed, tokens in k order
    float* coef;    // [NC, Hv, COEF]: exp(Gam_t), exp(Gam_last - Gam_t), exp(Gam_last), 2^uexp
    int* cbase;     // [N + 1] packed prompts: first chunk slot of each sequence (write_chunk_bases)
    // segmented carry (see carry_kernel): the chunks of a sequence split into nseg segments
    float* Sent;    // [N, Hv, D, D] entry state of segment 1
    _Float16* Mhl;  // [nseg - 2, N, Hv, 2, D, D] state maps of segments 1 .. nseg - 2 (S_end = M S_entry + R):
                    // M = hi + lo, fp16 planes, columns in k order, column tile t scaled by 2^-Mexp[t]
    int* Mexp;      // [nseg - 2, N, Hv, D / 16] (kZeroTile: the tile is exactly zero)
    float* Rseg;    // [nseg - 2, N, Hv, D, D] their end states from a zero entry state
    int nc_max;
    int nseg;       // segments per sequence (1: one chain per sequence)
    int pass;       // segmented carry: which of its two carry passes a launch runs
    size_t bytes;
};

static Ws layout(void* base, int B, int L, int N, int Hk, int Hv, bool ragged, bool whole) {
    const plan::Layout l = plan::layout(B, L, N, Hk, Hv, ragged, whole);
    char* b = static_cast<char*>(base);
    auto at = [&](size_t off, size_t n) -> void* { return (b != nullptr && n > 0) ? b + off : nullptr; };
    Ws w;
    w.qh = static_cast<_Float16*>(at(l.qh, l.n_qh));
    w.kh = static_cast<_Float16*>(at(l.kh, l.n_kh));
    w.W = static_cast<_Float16*>(at(l.W, l.n_W));
    w.U = static_cast<_Float16*>(at(l.U, l.n_U));
    w.P = static_cast<_Float16*>(at(l.P, l.n_P));
    w.KT = static_cast<_Float16*>(at(l.KT, l.n_KT));
    w.coef = static_cast<float*>(at(l.coef, l.n_coef));
    w.cbase = static_cast<int*>(at(l.cbase, l.n_cbase));
    w.Sent = static_cast<float*>(at(l.Sent, l.n_Sent));
    w.Mhl = static_cast<_Float16*>(at(l.Mhl, l.n_Mhl));
    w.Mexp = static_cast<int*>(at(l.Mexp, l.n_Mexp));
    w.Rseg = static_cast<float*>(at(l.Rseg, l.n_Rseg));
    w.nc_max = l.nc_max;
    w.nseg = l.nseg;
    w.pass = 0;
    w.bytes = l.bytes;
    return w;
}

__device__ __forceinline__ int chunks_of(const Seg& s) { return (s.len + C - 1) / C; }

// Sequence n of chunk slot id and the chunk's index c inside it: rows of equal length
// unpacked, the table of first slots (write_chunk_bases) packed.
__device__ __forceinline__ bool find_chunk(int id, const PrefillArgs& a, const Ws& ws, int* n_out, int* c_out,
                                           Seg* seg) {
    if (a.cu == nullptr) {
        const int per = plan::chunks_of_len(a.L);
        if (per == 0 || id >= a.N * per) return false;
        *n_out = id / per;
        *c_out = id - *n_out * per;
    } else if (!chunk_slot(id, a.N, ws.cbase, n_out, c_out)) {
        return false;
    }
    *seg = segment_of(*n_out, a.L, a.cu);
    return *c_out >= 0 && *c_out < chunks_of(*seg);   // (always, from the table the front kernel wrote)
}

// Sequence owning token p of a row (clamped cu_seqlens), or -1.
__device__ __forceinline__ int owner_of(int p, int row, const PrefillArgs& a, int* start) {
    if (a.cu == nullptr) { *start = 0; return row; }
    int lo = 0, hi = a.N - 1, n = -1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        int st = a.cu[mid];
        st = st < 0 ? 0 : (st > a.L ? a.L : st);
        if (st <= p) { n = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    if (n < 0) return -1;
    const Seg sg = segment_of(n, a.L, a.cu);
    if (p >= sg.start + sg.len) return -1;
    *start = sg.start;
    return n;
}

// An input value back in its storage type, from fp32 holding a value that was
// widened from that type (so the bf16 case, dropping the low 16 zero bits, is exact).
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return bf16_t{static_cast<uint16_t>(__float_as_uint(x) >> 16)};
}

// SiLU with the hardware exp2 and reciprocal (about 1e-6 relative): the result is
// rounded to fp16 (2^-11) right after, so the accurate library forms would buy nothing.
__device__ __forceinline__ float fast_silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));   // v_exp_f32, v_rcp_f32
}

// Sum over each row of 16 lanes; every lane of the row receives the same total
// (pairs within quads, then the quads of each half row, then the two half rows:
// every step adds two equal partial sums in either order, which gives the same bits).
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
    return x;
}

// ---- steps 1-4 ------------------------------------------------------------------
template <typename Tin>
__global__ __launch_bounds__(256) void front_kernel(PrefillArgs a, Ws ws) {
    __shared__ float buf[D * RAW];           // raw[c][m] (window of TT + 3 tokens), then ys[t][c] (stride 129)
    __shared__ int s_n[TT], s_start[TT];
    __shared__ unsigned s_endmask;           // bit t: token t is the last of its sequence
    static_assert(TT * (D + 1) <= D * RAW, "the transposed outputs reuse the raw tile");
    const int units = 2 * a.Hk;              // q and k heads (v is formed by the chunk kernel)
    const int tiles = (a.L + TT - 1) / TT;
    long long blk = blockIdx.x;
    const int u = static_cast<int>(blk % units); blk /= units;
    const int tile = static_cast<int>(blk % tiles);
    const int row = static_cast<int>(blk / tiles);
    const int p0 = tile * TT;
    const int ch0 = u * D;   // [Q | K] blocks of D channels
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Tin* x = static_cast<const Tin*>(a.qkv) + (static_cast<size_t>(row) * a.D + ch0) * a.L;
    const bool is_q = u < a.Hk;
    // packed prompts: the first workgroup writes the chunk slot table of the chunk and
    // carry kernels
    if (a.cu != nullptr && blockIdx.x == 0) write_chunk_bases(a.N, a.L, a.cu, C, ws.nc_max, ws.cbase);

    // Tiles after the first of unpacked bf16 rows whose length is a multiple of 8 (so that
    // every 8-token group is 16-byte aligned): each lane loads 8 tokens of a channel and the
    // 4 tokens before them in two vector loads and runs the conv in registers. Every window
    // lies inside the row, so there is no masking; in the row's last tile (whose 32 tokens
    // end the sequence) the lanes of the last 8 tokens also write the conv state, those
    // tokens' last K - 1 raw inputs.
    const bool vec = sizeof(Tin) == 2 && a.cu == nullptr && a.L % 8 == 0 && p0 > 0 && p0 + TT <= a.L &&
                     (reinterpret_cast<uintptr_t>(a.qkv) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.w) & 7) == 0;
    if (vec) {
        static_assert(TT == 32 && D == 128, "4 lanes of 8 tokens per channel, 16 channels per instruction");
        const int lq = lane >> 2, g = lane & 3;
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
        const uint16_t* wb = reinterpret_cast<const uint16_t*>(a.w);
        uint4 xr[2];
        uint2 hr[2], wr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int cc = (wave * 2 + i) * 16 + lq;
            const uint16_t* xp = xb + static_cast<size_t>(cc) * a.L + p0 + 8 * g;
            xr[i] = *reinterpret_cast<const uint4*>(xp);
            hr[i] = *reinterpret_cast<const uint2*>(xp - 4);
            wr[i] = *reinterpret_cast<const uint2*>(wb + static_cast<size_t>(ch0 + cc) * kConvK);
        }
        static_assert(kConvK == 4, "the conv state is tokens 5, 6 and 7 of the last 8-token group");
        if (p0 + TT == a.L && g == 3) {   // sequence `row` ends at the tile's last token
            uint16_t* co = static_cast<uint16_t*>(a.conv_out);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const size_t cb = (static_cast<size_t>(row) * a.D + ch0 + (wave * 2 + i) * 16 + lq) * (kConvK - 1);
                co[cb + 0] = static_cast<uint16_t>(xr[i].z >> 16);
                co[cb + 1] = static_cast<uint16_t>(xr[i].w & 0xffffu);
                co[cb + 2] = static_cast<uint16_t>(xr[i].w >> 16);
            }
        }
        const auto lo = [](unsigned v) { return __uint_as_float(v << 16); };
        const auto hi = [](unsigned v) { return __uint_as_float(v & 0xffff0000u); };
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int cc = (wave * 2 + i) * 16 + lq;
            const float xv[11] = {hi(hr[i].x), lo(hr[i].y), hi(hr[i].y),
                                  lo(xr[i].x), hi(xr[i].x), lo(xr[i].y), hi(xr[i].y),
                                  lo(xr[i].z), hi(xr[i].z), lo(xr[i].w), hi(xr[i].w)};
            const float w0 = lo(wr[i].x), w1 = hi(wr[i].x), w2 = lo(wr[i].y), w3 = hi(wr[i].y);
            const int cpos = kpos(cc);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float acc = w0 * xv[j];
                acc = __fmaf_rn(w1, xv[j + 1], acc);
                acc = __fmaf_rn(w2, xv[j + 2], acc);
                acc = __fmaf_rn(w3, xv[j + 3], acc);
                buf[(8 * g + j) * (D + 1) + cpos] = fast_silu(acc);
            }
        }
    } else {

    // a wave loads TT consecutive tokens of 64 / TT channels per instruction
    // (coalesced); the 3 tokens before the tile (3 x 128 values) come from two
    // loads per thread. Every load is unconditional, from a clamped position, and
    // masked afterwards, so that all of them are in flight at once (a load under a
    // branch is waited for inside the branch).
    constexpr int CPI = kWave / TT;                  // channels per load instruction
    constexpr int ROWS = D / 4 / CPI;                // instructions per wave
    const int lt = lane % TT, lc = lane / TT;
    float v[ROWS], hv[2];
    {
        const int p = p0 + lt;
        const bool pv = p < a.L;
        const int pc = pv ? p : a.L - 1;
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            const float lv = to_f32(x[static_cast<size_t>((wave * ROWS + i) * CPI + lc) * a.L + pc]);
            v[i] = pv ? lv : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = tid + 256 * k;                 // < 3 * D for k == 0 and tid < 128 when k == 1
            const int hc = item < 3 * D ? item / 3 : 0, hj = item % 3;
            const int ph = p0 - 3 + hj;                     // < L since p0 < L
            const float lh = to_f32(x[static_cast<size_t>(hc) * a.L + (ph >= 0 ? ph : 0)]);
            hv[k] = ph >= 0 ? lh : 0.f;
        }
    }
    // sequence of every token of the tile; with cu_seqlens the (clamped) table is
    // searched in LDS when it fits in the tile buffer, which is free until the
    // loads above are written into it
    const bool cu_lds = a.cu != nullptr && a.N + 1 <= D * RAW;
    if (cu_lds) {
        int* scu = reinterpret_cast<int*>(buf);
        for (int i = tid; i <= a.N; i += 256) {
            const int v0 = a.cu[i];
            scu[i] = v0 < 0 ? 0 : (v0 > a.L ? a.L : v0);
        }
        __syncthreads();
    }
    if (tid < TT) {
        const int p = p0 + tid;
        int start = 0, end = 0, n = -1;
        if (p < a.L) {
            if (cu_lds) {
                const int* scu = reinterpret_cast<const int*>(buf);
                int lo = 0, hi = a.N - 1;
                while (lo <= hi) {                          // last n whose start is <= p
                    const int mid = (lo + hi) >> 1;
                    if (scu[mid] <= p) { n = mid; lo = mid + 1; } else { hi = mid - 1; }
                }
                if (n >= 0) {
                    start = scu[n];
                    end = scu[n + 1];
                    if (p >= end) n = -1;                   // past the end (or an empty pair)
                }
            } else {
                n = owner_of(p, row, a, &start);
                if (n >= 0) {
                    const Seg sg = segment_of(n, a.L, a.cu);
                    end = sg.start + sg.len;
                }
            }
        }
        s_n[tid] = n;
        s_start[tid] = start;
        static_assert(TT <= 32 && TT <= kWave, "the end mask is one wave's ballot");
        const unsigned long long m = __ballot(n >= 0 && p + 1 == end);
        if (tid == 0) s_endmask = static_cast<unsigned>(m);
    }
    if (cu_lds) __syncthreads();                            // the table is read before buf is reused
#pragma unroll
    for (int i = 0; i < ROWS; ++i) buf[((wave * ROWS + i) * CPI + lc) * RAW + 3 + lt] = v[i];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int item = tid + 256 * k;
        if (item < 3 * D) buf[(item / 3) * RAW + item % 3] = hv[k];
    }
    __syncthreads();
    const int c = tid & (D - 1), th = tid >> 7;   // channel, token half
    const Tin* w = static_cast<const Tin*>(a.w) + static_cast<size_t>(ch0 + c) * kConvK;
    float wv[kConvK];
#pragma unroll
    for (int j = 0; j < kConvK; ++j) wv[j] = to_f32(w[j]);
    const Tin* cin = static_cast<const Tin*>(a.conv_in);
    float y[TT / 2];
    const int t0 = th * (TT / 2);
    // fast path: all 32 tokens of this half belong to one sequence whose start is at
    // least K-1 tokens before the first of them, so every window lies in the tile
    const bool clean = s_n[t0] >= 0 && s_n[t0] == s_n[t0 + TT / 2 - 1] && p0 + t0 - s_start[t0] >= kConvK - 1;
    if (clean) {
        float x0 = buf[c * RAW + t0], x1 = buf[c * RAW + t0 + 1], x2 = buf[c * RAW + t0 + 2];
#pragma unroll
        for (int j = 0; j < TT / 2; ++j) {
            const float x3 = buf[c * RAW + t0 + j + 3];
            float acc = wv[0] * x0;
            acc = __fmaf_rn(wv[1], x1, acc);
            acc = __fmaf_rn(wv[2], x2, acc);
            acc = __fmaf_rn(wv[3], x3, acc);
            y[j] = fast_silu(acc);
            x0 = x1; x1 = x2; x2 = x3;
        }
    } else {
#pragma unroll
        for (int j = 0; j < TT / 2; ++j) {
            const int t = t0 + j;
            const int n = s_n[t];
            float win[kConvK];
            if (n < 0) { y[j] = 0.f; continue; }
            const int uu = p0 + t - s_start[t];  // index inside the sequence
#pragma unroll
            for (int q = 0; q < kConvK; ++q) {
                const int m = uu + q;            // position in concat(state, x[seq])
                win[q] = (m < kConvK - 1) ? to_f32(cin[(static_cast<size_t>(n) * a.D + ch0 + c) * (kConvK - 1) + m])
                                          : buf[c * RAW + t + q];
            }
            float acc = wv[0] * win[0];
            acc = __fmaf_rn(wv[1], win[1], acc);
            acc = __fmaf_rn(wv[2], win[2], acc);
            acc = __fmaf_rn(wv[3], win[3], acc);
            y[j] = fast_silu(acc);
        }
    }
    // step 2's conv-state update: for every sequence whose last token lies in this
    // half of the tile, its K-1 most recent raw inputs (in the tile or its 3-token
    // halo, exact in fp32), or the incoming state for a sequence shorter than K-1
    {
        Tin* co = static_cast<Tin*>(a.conv_out);
        for (unsigned em = (s_endmask >> t0) & ((1u << (TT / 2)) - 1); em != 0; em &= em - 1) {   // usually none
            const int t = t0 + __builtin_ctz(em);
            const int n = s_n[t];
            const int len = p0 + t + 1 - s_start[t];
            const size_t base = (static_cast<size_t>(n) * a.D + ch0 + c) * (kConvK - 1);
#pragma unroll
            for (int j = 0; j < kConvK - 1; ++j) {
                const int m = len + j;                         // position in concat(state, x[seq])
                co[base + j] = m < kConvK - 1 ? cin[base + m] : from_f32<Tin>(buf[c * RAW + t + 1 + j]);
            }
        }
        if (a.cu != nullptr && tile == 0 && row == 0) {        // empty sequences keep their state
            for (int n0 = 0; n0 < a.N; n0 += 64) {             // 64 sequences a round, one per lane
                const int nl = n0 + lane;
                const bool empty = nl < a.N && segment_of(nl, a.L, a.cu).len == 0;
                for (unsigned long long em = __ballot(empty); em != 0; em &= em - 1) {
                    const size_t base = (static_cast<size_t>(n0 + __builtin_ctzll(em)) * a.D + ch0 + c) * (kConvK - 1);
                    if (th == 0) {
#pragma unroll
                        for (int j = 0; j < kConvK - 1; ++j) co[base + j] = cin[base + j];
                    }
                }
            }
        }
    }
    __syncthreads();
    // q and k channels are placed in k order here (the norms below do not depend on the order)
    const int cpos = kpos(c);
#pragma unroll
    for (int j = 0; j < TT / 2; ++j) buf[(th * (TT / 2) + j) * (D + 1) + cpos] = y[j];
    }
    __syncthreads();
    // 16 lanes per token, 8 channels (16 bytes) per lane: a wave stores 4 tokens
    // per instruction, 16 tokens in all. A token's sum of squares is formed from its
    // 16 lanes' partials by a DPP tree that leaves the same total in every lane.
    {
        const int tq = lane >> 4, j = lane & 15;
        _Float16* base = is_q ? ws.qh + u * D : ws.kh + (u - a.Hk) * D;
        const int hs = a.Hk;                         // heads per token in the destination
#pragma unroll
        for (int i = 0; i < TT / 16; ++i) {
            const int t = wave * (TT / 4) + 4 * i + tq;
            float x[8];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = buf[t * (D + 1) + 8 * j + e];
                ss = __fmaf_rn(x[e], x[e], ss);
            }
            ss = row16_sum(ss);
            float r = 1.f;
            if (a.use_l2) r = 1.0f / sqrtf(ss + a.eps);
            if (is_q) r *= 1.0f / sqrtf(static_cast<float>(D));
            f16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = static_cast<_Float16>(x[e] * r);
            const size_t tok = static_cast<size_t>(row) * a.L + p0 + t;
            if (vec || s_n[t] >= 0) *reinterpret_cast<f16x8*>(base + tok * hs * D + 8 * j) = v;
        }
    }
}

// ---- chunk phase --------------------------------------------------------------------
constexpr int KS = D + 8;    // row stride (halfs) of the chunk's keys in LDS
constexpr int TS = C + 8;    // row stride (halfs) of the transposed operands (16-byte aligned rows)
constexpr int AS = C + 1;    // row stride (floats) of A and T

// acc += X Y for 16 x 16 fp32 blocks in LDS (row strides AS) on v_mfma_f32_16x16x4_f32
// (A: lane l holds A[l % 16][l / 16]; B: B[l / 16][l % 16]; D: rows 4 (l / 16) + e,
// column l % 16); step q contracts k = 4q .. 4q + 3.
__device__ __forceinline__ f32x4v mma16_f32_lds(const float* X, const float* Y, int lane, f32x4v acc) {
    const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r16 * AS + 4 * q + g], Y[(4 * q + g) * AS + r16], acc, 0, 0, 0);
    return acc;
}

// acc += X M with X a 16 x 16 fp32 block in LDS and M in accumulator layout in
// registers: step q pairs k slot l / 16 with row 4 (l / 16) + q, the row this lane
// holds as element q, so M feeds the B operand without moving.
__device__ __forceinline__ f32x4v mma16_f32_reg(const float* X, const f32x4v& m, int lane, f32x4v acc) {
    const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r16 * AS + 4 * g + q], m[q], acc, 0, 0, 0);
    return acc;
}


// Every exponent in this kernel is a difference of the chunk's cumulative log-decay
// (non-increasing), so it is <= 0: the hardware exp (about 1e-6 relative) cannot
// overflow, and its error sits far below the fp16 rounding of the results.
template <typename Tin>
__global__ __launch_bounds__(256, 4) void chunk_kernel(PrefillArgs a, Ws ws) {
    // region: {Kc [C][KS] halfs, Am [C][AS] floats} during the Gram phase,
    //         {Tm [C][AS] floats over Kc, Am} during the solve,
    //         {KbT [D][TS], VbT [D][TS] halfs} during the W/U phase.
    // 37.4 KB of LDS in all (and 114 registers): four workgroups per CU.
    constexpr int REGION = 2 * D * TS * 2;  // 36864 B >= 64*136*2 + 64*65*4 = 34048 B
    static_assert(C * AS * 4 <= C * KS * 2, "T must fit where the keys were");
    __shared__ __align__(16) unsigned char region[REGION];
    __shared__ __align__(16) float s_b[C], s_gam[C], s_red[4];
    _Float16* Kc = reinterpret_cast<_Float16*>(region);
    float* Am = reinterpret_cast<float*>(region + C * KS * 2);
    float* Tm = reinterpret_cast<float*>(region);   // written only after the Gram phase's last read of Kc
    _Float16* KbT = reinterpret_cast<_Float16*>(region);
    _Float16* VbT = reinterpret_cast<_Float16*>(region + D * TS * 2);

    // blockIdx -> (chunk, V head), the GQA pair of V heads on one XCD (plan::chunk_unit)
    const int f = a.Hv / a.Hk;
    const plan::ChunkUnit cu = plan::chunk_unit(blockIdx.x, ws.nc_max, a.Hk, a.Hv);
    const int hk = cu.hk, id = cu.id, h = cu.h;
    int n, c;
    Seg seg;
    if (id == 0 && a.cu != nullptr && threadIdx.x < D) {   // empty sequences keep the value channels' conv state
        const int ch = 2 * a.Hk * D + h * D + threadIdx.x;
        for (int m0 = 0; m0 < a.N; m0 += 64) {             // 64 sequences a round, one per lane
            const int ml = m0 + (threadIdx.x & 63);
            const bool empty = ml < a.N && segment_of(ml, a.L, a.cu).len == 0;
            for (unsigned long long em = __ballot(empty); em != 0; em &= em - 1) {
                const size_t cb = (static_cast<size_t>(m0 + __builtin_ctzll(em)) * a.D + ch) * (kConvK - 1);
#pragma unroll
                for (int j = 0; j < kConvK - 1; ++j)
                    static_cast<Tin*>(a.conv_out)[cb + j] = static_cast<const Tin*>(a.conv_in)[cb + j];
            }
        }
    }
    if (id >= ws.nc_max || !find_chunk(id, a, ws, &n, &c, &seg)) return;
    const int nt = min(C, seg.len - c * C);
    const size_t tok0 = static_cast<size_t>(seg.row) * a.L + seg.start + static_cast<size_t>(c) * C;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const Tin* gate = static_cast<const Tin*>(a.gate);
    const Tin* beta = static_cast<const Tin*>(a.beta);

    // 1. keys of the chunk (zero rows past the end), gate, beta. Lane = token, granules
    //    wave + 4 q: the registers also serve step 4 (the keys are not read twice)
    f16x8 kreg[4];
    {
        const int r = lane, rc = r < nt ? r : nt - 1;   // clamped row, masked below
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f16x8 v = *reinterpret_cast<const f16x8*>(ws.kh + ((tok0 + rc) * a.Hk + hk) * D + 8 * (wave + 4 * q));
            kreg[q] = r < nt ? v : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<f16x8*>(Kc + r * KS + 8 * (wave + 4 * q)) = kreg[q];
    }
    // gate and beta of token `lane` (wave 0; zero past the end)
    static_assert(C == kWave, "one wave holds the chunk's gates");
    float gv = 0.f, bv = 0.f;
    if (wave == 0 && tid < nt) gate_beta_at<Tin>(gate, beta, a.fu.A_log, a.fu.dt_bias, (tok0 + tid) * a.Hv + h, h, &gv, &bv);
    // q rows of this wave's 16-token tile, straight into registers (A operands)
    f16x8 aq[4];
    {
        const int t = 16 * wave + r16;
        const int tc = t < nt ? t : nt - 1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f16x8 v = *reinterpret_cast<const f16x8*>(ws.qh + ((tok0 + tc) * a.Hk + hk) * D + 32 * ks + 8 * g);
            aq[ks] = t < nt ? v : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    if (wave == 0) {   // Gam = inclusive cumulative sum of g (wave scan, from the registers)
        float v = gv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(v, off, 64);
            if (lane >= off) v += o;
        }
        s_gam[lane] = v;
        s_b[lane] = bv;
    }
    __syncthreads();

    // 2. Gram matrices on MFMA, transposed (key rows as the A operand): wave w owns token
    //    rows t = 16w..16w+15 (lane column r16); element e of tile n = 2 b5 + hh is key
    //    s = 32 b5 + 16 hh + 4 g + e, so the lane's eight keys of block b5 are positions
    //    32 b5 + 8 g .. + 7 of P's row in k order: one 16-byte store
    {
        f32x4v kk[4], qk[4];
#pragma unroll
        for (int ntile = 0; ntile < 4; ++ntile) { kk[ntile] = f32x4v{0, 0, 0, 0}; qk[ntile] = kk[ntile]; }
        const int prow = 16 * wave + r16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f16x8 ak = *reinterpret_cast<const f16x8*>(Kc + prow * KS + 32 * ks + 8 * g);
#pragma unroll
            for (int ntile = 0; ntile < 4; ++ntile) {
                const f16x8 bk = *reinterpret_cast<const f16x8*>(Kc + (16 * ntile + r16) * KS + 32 * ks + 8 * g);
                kk[ntile] = mfma16x16x32(bk, ak, kk[ntile]);
                qk[ntile] = mfma16x16x32(bk, aq[ks], qk[ntile]);
            }
        }
        _Float16* P = ws.P + (static_cast<size_t>(id) * a.Hv + h) * C * C;
        const int t = 16 * wave + r16;
        const float gt = s_gam[t], bt = s_b[t];
#pragma unroll
        for (int b5 = 0; b5 < 2; ++b5) {
            f16x8 pv;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 32 * b5 + 16 * hh + 4 * g + e;
                    const float dec = (s <= t && t < nt) ? __expf(gt - s_gam[s]) : 0.f;
                    Am[t * AS + s] = (s < t) ? bt * dec * kk[2 * b5 + hh][e] : 0.f;
                    pv[4 * hh + e] = static_cast<_Float16>(dec * qk[2 * b5 + hh][e]);
                }
            }
            *reinterpret_cast<f16x8*>(P + t * C + 32 * b5 + 8 * g) = pv;
        }
    }
    // keys of the chunk (still in LDS until T overwrites them) transposed for the carry
    if ((h % f) == 0) {   // KT[i][s], tokens in k order
        // thread: features 4 fa .. 4 fa + 3 (4 consecutive halfs of a key row, at
        // kpos(4 fa)) of the 8 tokens at positions 8 sg .. 8 sg + 7
        const int fa = tid >> 3, sg = tid & 7;
        _Float16* kt = ws.KT + (static_cast<size_t>(id) * a.Hk + hk) * D * C;
        f16x4 r[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) r[q] = *reinterpret_cast<const f16x4*>(Kc + kidx(8 * sg + q) * KS + kpos(4 * fa));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f16x8 v = {r[0][e], r[1][e], r[2][e], r[3][e], r[4][e], r[5][e], r[6][e], r[7][e]};
            *reinterpret_cast<f16x8*>(kt + (4 * fa + e) * C + 8 * sg) = v;
        }
    }
    __syncthreads();

    // Steps 1-2 for this V head's value channels (v needs no norm), formed here from the
    // raw channel-major input: item i of a thread is channel f0 + 32 i of the head and
    // tokens 8 g8 .. 8 g8 + 7 of the chunk, whose conv windows span the raw positions
    // p - 3 .. p + 7 (p = the item's first token). Chunks after a sequence's first whose
    // loads stay inside the row fetch the 12 positions [p - 4, p + 8) or [p - 3, p + 9),
    // whichever starts on a 4-byte boundary, in two vector loads issued now, so that the
    // solve hides their latency; the other chunks gather theirs in step 4 (a first
    // chunk's windows start in the incoming conv state).
    static_assert(sizeof(Tin) == 2, "the raw value loads assume bf16 inputs");
    const int g8 = tid & 7, f0 = tid >> 3;
    const int cv0 = 2 * a.Hk * D + h * D;                 // first channel of this V head
    const int pc = seg.start + c * C;                      // row position of the chunk's first token
    const uint16_t* xr = reinterpret_cast<const uint16_t*>(a.qkv) + static_cast<size_t>(seg.row) * a.D * a.L;
    const bool vfast = plan::value_fast(c, nt, pc, a.L) && (reinterpret_cast<uintptr_t>(a.qkv) & 3) == 0;
    u32x4a4 vlo[4];
    u32x2a4 vhi[4];
    uint2 wraw[4];                                         // conv taps of the item's channel
    {
        const uint16_t* wb = reinterpret_cast<const uint16_t*>(a.w);
        const bool wal = (reinterpret_cast<uintptr_t>(a.w) & 7) == 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t ch = static_cast<size_t>(cv0 + f0 + 32 * i);
            if (vfast) {
                const size_t e = ch * a.L + pc + 8 * g8 - 4;   // position p - 4
                const size_t q0 = e + (e & 1);
                vlo[i] = *reinterpret_cast<const u32x4a4*>(xr + q0);
                vhi[i] = *reinterpret_cast<const u32x2a4*>(xr + q0 + 8);
            }
            const uint16_t* wp = wb + ch * kConvK;
            wraw[i] = wal ? *reinterpret_cast<const uint2*>(wp)
                          : make_uint2(wp[0] | static_cast<unsigned>(wp[1]) << 16, wp[2] | static_cast<unsigned>(wp[3]) << 16);
        }
    }

    // 3. T = (I + A)^-1, fp32. Diagonal 16x16 blocks by forward substitution
    //    (lane = (block, column)); off-diagonal blocks by merging inverses of
    //    lower-triangular halves, [[P, 0], [Q, R]]^-1 = [[P^-1, 0], [-R^-1 Q P^-1, R^-1]]:
    //    first the two 32 x 32 diagonal halves, then the 32 x 32 lower-left quarter,
    //    every 16 x 16 block product on fp32 MFMA.
    if (wave == 0) {
        const int blk = lane >> 4, j = lane & 15;
        float xcol[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = (t == j) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < t; ++s) acc = __fmaf_rn(-Am[(16 * blk + t) * AS + 16 * blk + s], xcol[s], acc);
            xcol[t] = acc;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) Tm[(16 * blk + t) * AS + 16 * blk + j] = xcol[t];
    } else {
        for (int e = tid - 64; e < C * C; e += 192) {
            const int t = e >> 6, s = e & 63;
            if ((s >> 4) > (t >> 4)) Tm[t * AS + s] = 0.f;
        }
    }
    __syncthreads();
    {
        auto blk = [&](int i, int j) { return 16 * i * AS + 16 * j; };   // offset of block (i, j)
        // merge 16 -> 32: T_{2w+1, 2w} = -T_{2w+1,2w+1} A_{2w+1,2w} T_{2w,2w}, w = 0, 1
        if (wave < 2) {
            const int i = 2 * wave + 1, j = 2 * wave;
            f32x4v m = f32x4v{0, 0, 0, 0};
            m = mma16_f32_lds(Am + blk(i, j), Tm + blk(j, j), lane, m);
            f32x4v t = f32x4v{0, 0, 0, 0};
            t = mma16_f32_reg(Tm + blk(i, i), m, lane, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[blk(i, j) + (4 * g + e) * AS + r16] = -t[e];
        }
        __syncthreads();
        // merge 32 -> 64: with N_mj = A_m0 T_0j + A_m1 T_1j (m = 2, 3),
        // T_ij = -(T_i2 N_2j + T_i3 N_3j) for i = 2 + w / 2, j = w % 2 (T_01 = T_23 = 0)
        {
            const int i = 2 + (wave >> 1), j = wave & 1;
            f32x4v n2 = f32x4v{0, 0, 0, 0}, n3 = f32x4v{0, 0, 0, 0};
            n2 = mma16_f32_lds(Am + blk(2, 0), Tm + blk(0, j), lane, n2);
            n2 = mma16_f32_lds(Am + blk(2, 1), Tm + blk(1, j), lane, n2);
            n3 = mma16_f32_lds(Am + blk(3, 0), Tm + blk(0, j), lane, n3);
            n3 = mma16_f32_lds(Am + blk(3, 1), Tm + blk(1, j), lane, n3);
            f32x4v t = f32x4v{0, 0, 0, 0};
            t = mma16_f32_reg(Tm + blk(i, 2), n2, lane, t);
            t = mma16_f32_reg(Tm + blk(i, 3), n3, lane, t);
            // the blocks written here (rows 2-3, columns 0-1) are read by no wave of this step
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[blk(i, j) + (4 * g + e) * AS + r16] = -t[e];
        }
        __syncthreads();
    }

    // T rows of this wave as the A operands of step 5, read before KbT overwrites T
    f16x8 at[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) at[ks][e] = static_cast<_Float16>(Tm[(16 * wave + r16) * AS + 32 * ks + 8 * g + e]);
    __syncthreads();

    // 4. operands of W and U, transposed (k = token): KbT[i][s] = beta_s exp(Gam_s) k_s[i],
    //    VbT[j][s] = beta_s v_s[j] 2^-eV
    // lanes run along tokens, so the transposed LDS writes of a wave hit
    // consecutive halfs (no bank conflicts); item (s, j) = granule j of token s
    {
        const int s = lane;
        const float fk = s_b[s] * __expf(s_gam[s]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = wave + 4 * q;
            const f16x8 kv = kreg[q];   // zero past the end
#pragma unroll
            for (int e = 0; e < 8; ++e)
                KbT[kidx(8 * j + e) * TS + s] = static_cast<_Float16>(fk * static_cast<float>(kv[e]));   // row: feature
        }
    }
    // v = SiLU(conv) of the items (zero past the end). The window's 11 raw values stay
    // packed as bf16 pairs: A[k] = (x_2k, x_2k+1), B[k] = (x_2k+1, x_2k+2) (x_0 = position
    // p - 3), and each token's four taps are two bf16 dot products (exact products, fp32 sums).
    const f32x4v bt0 = *reinterpret_cast<const f32x4v*>(s_b + 8 * g8), bt1 = *reinterpret_cast<const f32x4v*>(s_b + 8 * g8 + 4);
    const float bt[8] = {bt0[0], bt0[1], bt0[2], bt0[3], bt1[0], bt1[1], bt1[2], bt1[3]};
    float vv[4][8];
    float vmax = 0.f;
    {
        const uint16_t* cin = static_cast<const uint16_t*>(a.conv_in);
        const auto pair = [](unsigned v) { return __builtin_bit_cast(bf16x2, v); };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t ch = static_cast<size_t>(cv0 + f0 + 32 * i);
            unsigned A[6];
            if (vfast) {
                const unsigned d[7] = {vlo[i].x, vlo[i].y, vlo[i].z, vlo[i].w, vhi[i].x, vhi[i].y, 0u};
                // the loads start at p - 4 (drop one value: shift by 2 bytes) or at p - 3
                const unsigned sh = ((ch * a.L + pc + 8 * g8 - 4) & 1) == 0 ? 2u : 0u;
#pragma unroll
                for (int k = 0; k < 6; ++k) A[k] = __builtin_amdgcn_alignbyte(d[k + 1], d[k], sh);
            } else {
                unsigned xs[12];
#pragma unroll
                for (int k = 0; k < 12; ++k) {
                    const int u = c * C + 8 * g8 - 3 + k;            // position inside the sequence
                    unsigned x = 0u;                                 // past the end: masked below
                    if (k < 11 && u < 0) x = cin[(static_cast<size_t>(n) * a.D + ch) * (kConvK - 1) + (kConvK - 1) + u];
                    else if (k < 11 && u < seg.len) x = xr[ch * a.L + seg.start + u];
                    xs[k] = x;
                }
#pragma unroll
                for (int k = 0; k < 6; ++k) A[k] = xs[2 * k] | xs[2 * k + 1] << 16;
            }
            unsigned Bp[5];
#pragma unroll
            for (int k = 0; k < 5; ++k) Bp[k] = __builtin_amdgcn_alignbyte(A[k + 1], A[k], 2u);
            const bf16x2 w01 = pair(wraw[i].x), w23 = pair(wraw[i].y);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const unsigned lo2 = (j & 1) ? Bp[j >> 1] : A[j >> 1];           // (x_j, x_j+1)
                const unsigned hi2 = (j & 1) ? Bp[(j >> 1) + 1] : A[(j >> 1) + 1];   // (x_j+2, x_j+3)
                const float acc = __builtin_amdgcn_fdot2_f32_bf16(w23, pair(hi2),
                                                                  __builtin_amdgcn_fdot2_f32_bf16(w01, pair(lo2), 0.f, false), false);
                vv[i][j] = 8 * g8 + j < nt ? fast_silu(acc) : 0.f;
                vmax = fmaxf(vmax, fabsf(bt[j] * vv[i][j]));
            }
        }
    }
    vmax = wave_max(vmax);
    if (lane == 0) s_red[wave] = vmax;
    __syncthreads();
    const int eV = pow2_exponent(fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3])));
    const float sV = ldexpf(1.f, -eV);
    float bs[8];                    // beta_s 2^-eV (exact: a power of two)
#pragma unroll
    for (int j = 0; j < 8; ++j) bs[j] = bt[j] * sV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // row f of VbT, tokens 8 g8 .. + 7: one 16-byte store
        f16x8 hv;
#pragma unroll
        for (int j = 0; j < 8; ++j) hv[j] = static_cast<_Float16>(bs[j] * vv[i][j]);
        *reinterpret_cast<f16x8*>(VbT + (f0 + 32 * i) * TS + 8 * g8) = hv;
    }
    // the value channels' conv state after the sequence: its last K-1 raw inputs (or the
    // incoming state's for a sequence shorter than K-1)
    if (c == chunks_of(seg) - 1 && tid < D) {
        const size_t ch = static_cast<size_t>(cv0 + tid);
        const size_t cb = (static_cast<size_t>(n) * a.D + ch) * (kConvK - 1);
        const Tin* cin = static_cast<const Tin*>(a.conv_in);
        const Tin* xt = static_cast<const Tin*>(a.qkv) + static_cast<size_t>(seg.row) * a.D * a.L + ch * a.L + seg.start;
        Tin* co = static_cast<Tin*>(a.conv_out);
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j) {
            const int m = seg.len + j;                     // position in concat(state, x[seq])
            co[cb + j] = m < kConvK - 1 ? cin[cb + m] : xt[m - (kConvK - 1)];
        }
    }
    __syncthreads();

    // 5. W^T = KbT T^T and U = T VbT^T on MFMA: wave w owns token rows 16w..16w+15.
    //    In W^T element e of tile n = 2 b5 + hh is feature 32 b5 + 16 hh + 4 g + e, so a
    //    lane holds positions 32 b5 + 8 g .. + 7 of its token's row in k order (one
    //    16-byte store); U is stored transposed, 4 tokens of one feature per lane
    const int trow = 16 * wave + r16;
    _Float16* Wout = ws.W + (static_cast<size_t>(id) * a.Hv + h) * C * D;
    f32x4v uacc[8];
#pragma unroll
    for (int b5 = 0; b5 < 4; ++b5) {
        f32x4v wacc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int ntile = 2 * b5 + hh;
            wacc[hh] = f32x4v{0, 0, 0, 0};
            uacc[ntile] = wacc[hh];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f16x8 bk = *reinterpret_cast<const f16x8*>(KbT + (16 * ntile + r16) * TS + 32 * ks + 8 * g);
                const f16x8 bv = *reinterpret_cast<const f16x8*>(VbT + (16 * ntile + r16) * TS + 32 * ks + 8 * g);
                wacc[hh] = mfma16x16x32(bk, at[ks], wacc[hh]);
                uacc[ntile] = mfma16x16x32(at[ks], bv, uacc[ntile]);   // U itself: rows 4 g + e, column r16
            }
        }
        f16x8 wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wv[e] = static_cast<_Float16>(wacc[0][e]);
            wv[4 + e] = static_cast<_Float16>(wacc[1][e]);
        }
        *reinterpret_cast<f16x8*>(Wout + trow * D + 32 * b5 + 8 * g) = wv;
    }
    float umax = 0.f;
#pragma unroll
    for (int ntile = 0; ntile < 8; ++ntile)
#pragma unroll
        for (int e = 0; e < 4; ++e) umax = fmaxf(umax, fabsf(uacc[ntile][e]));
    umax = wave_max(umax);
    __syncthreads();   // every wave has read s_red
    if (lane == 0) s_red[wave] = umax;
    __syncthreads();
    const int eU = pow2_exponent(fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3])));
    const float sU = ldexpf(1.f, -eU);
    // U^T through LDS (the operand region is dead: every wave's MFMAs have consumed
    // their reads before the barriers above), then stored in whole 128-byte rows
    constexpr int UTS = C + 8;   // row stride (halfs) of U^T in LDS
    static_assert(D * UTS * 2 <= REGION, "U^T fits the operand region");
    _Float16* UT = reinterpret_cast<_Float16*>(region);
#pragma unroll
    for (int ntile = 0; ntile < 8; ++ntile) {   // feature 16 ntile + r16, tokens 16 w + 4 g ..
        const f16x4 uv = {static_cast<_Float16>(uacc[ntile][0] * sU), static_cast<_Float16>(uacc[ntile][1] * sU),
                          static_cast<_Float16>(uacc[ntile][2] * sU), static_cast<_Float16>(uacc[ntile][3] * sU)};
        *reinterpret_cast<f16x4*>(UT + (16 * ntile + r16) * UTS + 16 * wave + 4 * g) = uv;
    }
    __syncthreads();
    _Float16* Uout = ws.U + (static_cast<size_t>(id) * a.Hv + h) * C * D;
#pragma unroll
    for (int q = 0; q < D * C / 8 / 256; ++q) {
        const int it = tid + 256 * q, row = it >> 3, j = it & 7;
        *reinterpret_cast<uint4*>(Uout + row * C + 8 * j) = *reinterpret_cast<const uint4*>(UT + row * UTS + 8 * j);
    }
    float* cf = ws.coef + (static_cast<size_t>(id) * a.Hv + h) * COEF;
    if (tid < C) {
        const float glast = s_gam[nt - 1];
        cf[tid] = __expf(s_gam[tid]);
        cf[C + tid] = __expf(glast - s_gam[tid]);   // rows past the end multiply zero deltas
    }
    if (tid == 0) {
        cf[2 * C] = __expf(s_gam[nt - 1]);
        cf[2 * C + 1] = ldexpf(1.f, eV + eU);
    }
}

// ---- state carry ----------------------------------------------------------------------
// A workgroup of NW waves owns CPW = NW * NTW * 16 columns of one head's state:
// wave w owns the 16-column tiles [col0, col0 + 16 * NTW). A head is split over
// 128 / CPW workgroups (more CUs when there are few sequences). The LDS stage of one
// chunk (W, Q, K^T, P, this workgroup's columns of U^T, the coefficients) and the
// row and granule each lane loads into it are plan::Stage, plan::load16, plan::load8.

// Eight halfs of an A operand whose k slots (g, e) hold logical columns
// 32ks + 4g + e (e < 4) and 32ks + 16 + 4g + (e - 4) (e >= 4): with the row stored in
// k order these are granule 4 ks + g, one 16-byte read of a swizzled row.
template <int RG>   // granules per row (16 or 8)
__device__ __forceinline__ f16x8 lds_a(const _Float16* base, int row, int ks, int g) {
    return *reinterpret_cast<const f16x8*>(base + row * RG * 8 + ((4 * ks + g) ^ (row & (RG - 1))) * 8);
}

// U^T in a stage: row = column of the workgroup (64 tokens, 8 granules, swizzled).
// Tokens t .. t + 3 (t a multiple of 4) of one row, and one token.
__device__ __forceinline__ f16x4 lds_u4(const _Float16* Ul, int row, int t) {
    return *reinterpret_cast<const f16x4*>(Ul + row * 64 + (((t >> 3) ^ (row & 7)) << 3) + (t & 4));
}
__device__ __forceinline__ _Float16 lds_u1(const _Float16* Ul, int row, int t) {
    return Ul[row * 64 + (((t >> 3) ^ (row & 7)) << 3) + (t & 7)];
}

extern __shared__ __align__(1024) unsigned char g_stage[];   // two stages

// Issue the wave-wide 1 KB global->LDS loads of the regions of one stage that
// PARTS selects (bits: W, Q, KT, P, U, coefficients). Every region starts on a
// 1 KB boundary; wave w issues the region's instructions w, w + NW, ... as
// straight-line code. With NW a multiple of 4 the swizzle of a lane's granule is
// the same in every instruction of a region, so each load is a lane base plus a
// constant stride. `wave` must be wave-uniform (readfirstlane'd).
constexpr int ST_W = 1, ST_Q = 2, ST_KT = 4, ST_P = 8, ST_U = 16, ST_CF = 32, ST_ALL = 63;
template <int CPW, int NW, int PARTS>
__device__ __forceinline__ void issue_stage(const PrefillArgs& a, const Ws& ws, int id, size_t tok0, int nt,
                                            int h, int hk, int ucol0, int buf, int wave, int lane) {
    using SG = Stage<CPW>;
    static_assert(NW % 4 == 0 && SG::UG % NW == 0, "stage split assumes 4 or 8 waves");
    static_assert(SG::Q % 64 == 0 && SG::KT % 64 == 0 && SG::P % 64 == 0 && SG::U % 64 == 0 && SG::CF % 64 == 0,
                  "regions must start on instruction boundaries");
    const size_t wbase = (static_cast<size_t>(id) * a.Hv + h) * C * D;
    const size_t ktbase = (static_cast<size_t>(id) * a.Hk + hk) * D * C;
    const size_t pbase = (static_cast<size_t>(id) * a.Hv + h) * C * C;
    const size_t cfbase = (static_cast<size_t>(id) * a.Hv + h) * COEF;
    unsigned char* stage = g_stage + buf * SG::BYTES;
    auto ld = [&](const void* src, int slot) { __builtin_amdgcn_global_load_lds(src, stage + slot * 1024, 16, 0, 0); };
    static_assert(NW % 4 == 0, "plan::step16 / step8 keep the granule swizzle for nw a multiple of 4");
    // W and Q: 16 granules per row, a load covers 4 rows (load i = load 0 + 4 NW i rows)
    const plan::LaneLoad w0 = plan::load16(SG::W / 64, wave, lane), q0 = plan::load16(SG::Q / 64, wave, lane);
    if constexpr ((PARTS & ST_W) != 0) {
        const _Float16* src = ws.W + wbase + w0.row * D + 8 * w0.gran;
#pragma unroll
        for (int i = 0; i < 16 / NW; ++i) ld(src + i * 4 * NW * D, plan::step16(w0, NW, i).slot);
    }
#pragma unroll
    for (int i = 0; i < ((PARTS & ST_Q) ? 16 / NW : 0); ++i) {   // rows past the end: a finite row
        const plan::LaneLoad l = plan::step16(q0, NW, i);
        const int rr = l.row < nt ? l.row : nt - 1;
        ld(ws.qh + ((tok0 + rr) * a.Hk + hk) * D + 8 * l.gran, l.slot);
    }
    // KT and P: 8 granules per row, a load covers 8 rows (load i = load 0 + 8 NW i rows)
    if constexpr ((PARTS & ST_KT) != 0) {
        const plan::LaneLoad k0 = plan::load8(SG::KT / 64, wave, lane);
        const _Float16* src = ws.KT + ktbase + k0.row * C + 8 * k0.gran;
#pragma unroll
        for (int i = 0; i < 16 / NW; ++i) ld(src + i * 8 * NW * C, plan::step8(k0, NW, i).slot);
    }
    if constexpr ((PARTS & ST_P) != 0) {
        const plan::LaneLoad p0 = plan::load8(SG::P / 64, wave, lane);
        const _Float16* src = ws.P + pbase + p0.row * C + 8 * p0.gran;
#pragma unroll
        for (int i = 0; i < 8 / NW; ++i) ld(src + i * 8 * NW * C, plan::step8(p0, NW, i).slot);
    }
    // this workgroup's rows of U^T (its columns): 8 granules per row, like KT
    if constexpr ((PARTS & ST_U) != 0) {
        const plan::LaneLoad u0 = plan::load8(SG::U / 64, wave, lane);
        const _Float16* src = ws.U + wbase + static_cast<size_t>(ucol0 + u0.row) * C + 8 * u0.gran;
#pragma unroll
        for (int i = 0; i < CPW / 8 / NW; ++i) ld(src + i * 8 * NW * C, plan::step8(u0, NW, i).slot);
    }
    // coefficients (40 granules; lanes past the end land in padding)
    if constexpr ((PARTS & ST_CF) != 0) {
        if (wave == NW - 1)
            ld(ws.coef + cfbase + 4 * (lane < COEF / 4 ? lane : 0), SG::CF / 64);
    }
}

using plan::kSortMax;
constexpr int kZeroTile = -(1 << 20);   // state-map tile exponent marking a tile that is exactly zero

// Carried power-of-two scales: values held as x 2^-e with max|x 2^-e| kept inside
// [2^kWinLo, 2^15), a window of fp16's range with room to spare at the top (the fp16
// operands formed from them cannot overflow) and far enough above fp16's smallest
// normal at the bottom that the values keep fp16's full relative precision.
constexpr int kWinLo = 6;
// Wave-uniform: some lane's largest magnitude reached 2^15, or no lane's reached 2^kWinLo.
__device__ __forceinline__ bool outside_window(float lane_max) {
    return __builtin_amdgcn_ballot_w64(lane_max >= 0x1p15f) != 0 ||
           __builtin_amdgcn_ballot_w64(lane_max >= static_cast<float>(1 << kWinLo)) == 0;
}
// The exponent that puts the wave's largest magnitude (now at scale 2^-e) into
// [2^14, 2^15), kept >= ref - 100 so that the products that move values between this
// scale and the one of exponent ref stay inside fp32's range.
__device__ __forceinline__ int rescaled_exponent(int e, float lane_max, int ref) {
    return max(e + pow2_exponent(wave_max_nonneg(lane_max)), ref - 100);
}

// Sequence of rank r when the N packed sequences are ordered by decreasing length
// (ties by index). Every thread ranks up to N / blockDim of them against all N.
__device__ int sequence_of_rank(const PrefillArgs& a, int r) {
    __shared__ int s_len[kSortMax];
    __shared__ int s_pick;
    for (int m = threadIdx.x; m < a.N; m += blockDim.x) s_len[m] = segment_of(m, a.L, a.cu).len;
    if (threadIdx.x == 0) s_pick = r;   // a rank with no match (r >= N) keeps r (never happens)
    __syncthreads();
    for (int m = threadIdx.x; m < a.N; m += blockDim.x) {
        const int lm = s_len[m];
        int rank = 0;
        for (int q = 0; q < a.N; ++q) rank += (s_len[q] > lm || (s_len[q] == lm && q < m)) ? 1 : 0;
        if (rank == r) s_pick = m;
    }
    __syncthreads();
    return s_pick;
}

template <int NTW, int NW, bool LW, bool NORM, int NL>
__global__ __launch_bounds__((NW + (LW ? NL : 0)) * 64) void carry_kernel(PrefillArgs a, Ws ws) {
    constexpr int CPW = NW * NTW * 16;
    // NORM: the gated RMSNorm of each token's head row is applied before its store,
    // which needs the whole row (all 128 columns) in this workgroup
    static_assert(!NORM || (NTW == 1 && NW * 16 == D && !LW), "a fused norm needs a whole-head workgroup");
    static_assert(NL == 1 || (LW && NL == 2 && NW % NL == 0), "one or two loader waves");
    // One wave per SIMD (NW <= 4) leaves registers to hold a whole phase's operands:
    // their LDS reads are then issued ahead of the phase's MFMAs under one wait (a
    // scheduling barrier keeps them there). With two waves per SIMD the waves hide
    // each other's latency and the loops are left to the compiler, which would
    // otherwise spill.
    constexpr bool BATCH = NW <= 4;
    using SG = Stage<CPW>;
    constexpr int NS = 128 / CPW;                        // workgroups per head

    const int tid = threadIdx.x, lane = tid & 63;
    // Segmented mode (ws.nseg > 1): the chunks of each sequence split into nseg
    // segments and the carry runs in two passes. A chunk step is affine in the state
    // (S' = A_c S + B_c, each column on its own), so over a segment j the end state is
    // M_j S_entry + R_j. Pass 1 runs at once: FIRST, segment 0 from the entry state
    // with its outputs, ending in the entry state of segment 1; and for each middle
    // segment, LOCAL (from a zero state: R_j) and XMAP (the identity carried with
    // U = 0: M_j), neither forming outputs. Pass 2 carries segments 1 .. nseg - 1 with
    // outputs, each from its entry state S_j = M_{j-1} S_{j-1} + R_{j-1}, which its
    // workgroups form first on their own columns; the last one ends in the final state.
    const int NK = plan::carry_kinds(ws.nseg, ws.pass);   // kinds per head
    const plan::CarryUnit un = plan::carry_unit(blockIdx.x, NK * NS, a.N, a.Hk, a.Hv);
    const int slice = un.slice;
    const int cs = slice % NS;
    const int kind = slice / NS;
    const int h = un.h;
    int n = un.n;
    // Packed prompts: slots go to sequences longest first, so that the in-order
    // dispatch of workgroups to free CUs schedules the longest chains first.
    if (a.cu != nullptr && a.N <= kSortMax) n = sequence_of_rank(a, n);
    const int f = a.Hv / a.Hk, hk = h / f;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // With LW NL extra waves (waves NW ..) issue every stage load and wait for them, so the
    // compute waves never stall on the memory pipeline's queue.
    const bool loader = LW && wave >= NW;
    const int li = loader ? wave - NW : 0;               // loader li issues the compute waves li, li + NL, ...
    const int g = lane >> 4, r16 = lane & 15;
    const int ucol0 = cs * CPW;                          // first column of this workgroup
    const int lcol0 = wave * 16 * NTW;                   // first column of this wave, inside the workgroup
    const int col0 = ucol0 + lcol0;
    const Seg seg = segment_of(n, a.L, a.cu);
    const int base = a.cu != nullptr ? min(max(ws.cbase[n], 0), ws.nc_max)   // first chunk slot
                                     : n * plan::chunks_of_len(a.L);
    int nch = chunks_of(seg);
    if (base + nch > ws.nc_max) nch = ws.nc_max - base;   // only malformed cu_seqlens get here
    if (nch <= 0) return;
    // this workgroup's job (plan::carry_job): segment sj (chunks [cb, ce)), its entry
    // state, whether it forms outputs and loads U, and where its end state goes
    const size_t tile = (static_cast<size_t>(n) * a.Hv + h) * D * D;
    const size_t tiles = static_cast<size_t>(a.N) * a.Hv * D * D;
    const plan::Job job = plan::carry_job(ws.nseg, ws.pass, kind);
    const int sj = job.sj, entry = job.entry;
    const bool outs = job.outs, useU = job.useU;
    const float* Sin = a.S + tile;
    float* Send = a.S + tile;
    size_t mapo = 0;                                     // XMAP: its map's index in Mhl, Mexp (+ 1)
    if (job.from_sent) Sin = ws.Sent + tile;             // pass 2: S_1; later entry states are formed below
    if (job.end == plan::kEndSent) Send = ws.Sent + tile;
    else if (job.end == plan::kEndRseg) Send = ws.Rseg + static_cast<size_t>(sj - 1) * tiles + tile;
    else if (job.end == plan::kEndNone) Send = nullptr;
    if (job.map >= 0) mapo = (static_cast<size_t>(job.map) * tiles + tile) / (D * D) + 1;
    int m0 = 0;                                          // pass 2: maps 1 .. m0 are not needed
    if (job.from_sent) {
        // A segment whose state map is exactly zero (it has decayed below fp32's range)
        // ends in R whatever its entry state: the chain restarts after the latest one,
        // with the same result, bit for bit, as multiplying through it.
        for (int i = sj - 1; i >= 1 && m0 == 0; --i) {
            const int* ek = ws.Mexp + (static_cast<size_t>(i - 1) * a.N * a.Hv + n * a.Hv + h) * (D / 16);
            bool zero = true;
#pragma unroll
            for (int t = 0; t < D / 16; ++t) zero = zero && ek[t] == kZeroTile;
            if (zero) {
                m0 = i;
                Sin = ws.Rseg + static_cast<size_t>(i - 1) * tiles + tile;
            }
        }
    }
    const int cb = ws.nseg > 1 ? seg_begin(nch, ws.nseg, sj) : 0;
    const int ce = ws.nseg > 1 ? seg_begin(nch, ws.nseg, sj + 1) : nch;

    float S[8][NTW][4];
    float smax = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * mt + 4 * g + e, j = col0 + 16 * nt + r16;
                S[mt][nt][e] = entry == plan::kFromState ? Sin[i * D + j] : (entry == plan::kFromIdentity && i == j ? 1.f : 0.f);
                smax = fmaxf(smax, fabsf(S[mt][nt][e]));
            }

    const size_t row_tok = static_cast<size_t>(seg.row) * a.L + seg.start;
    const size_t ts = static_cast<size_t>(a.Hv) * D;     // token stride of o
    if (!useU && !loader) {   // U = 0: the U regions of both stages are zeroed once and never loaded
        for (int i = tid; i < 64 * SG::UG; i += NW * 64) {
            reinterpret_cast<uint4*>(g_stage + SG::U * 16)[i] = make_uint4(0, 0, 0, 0);
            reinterpret_cast<uint4*>(g_stage + SG::BYTES + SG::U * 16)[i] = make_uint4(0, 0, 0, 0);
        }
    }
    // a whole stage: every region this job reads (no Q and P without outputs, no U when it is 0)
    auto issue_all = [&](int id, size_t tok, int nt, int buf, int w) {
        if (outs) {
            if (useU) issue_stage<CPW, NW, ST_ALL>(a, ws, id, tok, nt, h, hk, ucol0, buf, w, lane);
            else issue_stage<CPW, NW, ST_ALL & ~ST_U>(a, ws, id, tok, nt, h, hk, ucol0, buf, w, lane);
        } else {
            if (useU) issue_stage<CPW, NW, ST_W | ST_KT | ST_U | ST_CF>(a, ws, id, tok, nt, h, hk, ucol0, buf, w, lane);
            else issue_stage<CPW, NW, ST_W | ST_KT | ST_CF>(a, ws, id, tok, nt, h, hk, ucol0, buf, w, lane);
        }
    };
    const int np = (ws.nseg > 1 && ws.pass == 2) ? sj - 1 - m0 : 0;   // maps m0 + 1 .. sj - 1 (see below)
    const bool prologue = NTW == 1 && np > 0;
    if ((!LW || loader) && cb < ce && !prologue) {
#pragma unroll
        for (int k = 0; k < (LW ? NW / NL : 1); ++k)   // a loader: compute waves li, li + NL, ...; else its own
            issue_all(base + cb, row_tok + static_cast<size_t>(cb) * C, min(C, seg.len - cb * C), 0, LW ? li + NL * k : wave);
    }
    // Segmented mode, pass 2: segment sj >= 2 enters with S_sj = M_{sj-1} S_{sj-1} + R_{sj-1}
    // from S_{m0+1} (S_1, or R_m0 after a zero map), formed here on this workgroup's columns
    // before its first chunk. The maps
    // (fp16 hi + lo planes, columns in k order, scaled per 16-column tile) stream into the
    // two stage buffers, the next one loading during the current product; the first
    // chunk's stage is issued once they are done with. The products split both operands
    // (hi*hi + hi*lo + lo*hi in fp32, close to an fp32 product), so these entry states
    // are as good as a carried one.
    if constexpr (NTW == 1) {
        if (np > 0) {
            if (LW && loader) {
                for (int i = 0; i < np; ++i) {
                    __syncthreads();                        // map i is in LDS
                    __syncthreads();                        // every compute wave is done with it
                }
                if (cb < ce)
#pragma unroll
                    for (int k = 0; k < NW / NL; ++k)
                        issue_all(base + cb, row_tok + static_cast<size_t>(cb) * C, min(C, seg.len - cb * C), 0, li + NL * k);
            } else {
                __shared__ int s_ek[kMaxSeg - 2][D / 16];
                static_assert(2 * D * D * 2 <= SG::BYTES, "a map fits a stage buffer");
                const size_t nhh = static_cast<size_t>(a.N) * a.Hv, head = static_cast<size_t>(n) * a.Hv + h;
                if (tid < np * (D / 16))
                    s_ek[tid / (D / 16)][tid % (D / 16)] =
                        ws.Mexp[(static_cast<size_t>(m0 + tid / (D / 16)) * nhh + head) * (D / 16) + tid % (D / 16)];
                // map m0 + i -> stage buffer (i - 1) & 1 as [hi rows, lo rows][16 granules], granule j of
                // row r at position j ^ (r % 16): wave-wide 1 KB loads of 4 rows, this wave's
                // instructions wave, wave + NW, ... (16 each)
                constexpr int MI = 2 * D / 4 / NW;   // 16 with 4 compute waves, 8 with 8
                auto issue_map = [&](int i) {
                    const _Float16* src = ws.Mhl + (static_cast<size_t>(m0 + i - 1) * nhh + head) * 2 * D * D;
                    unsigned char* dst = g_stage + ((i - 1) & 1) * SG::BYTES;
                    const plan::LaneLoad l0 = plan::load16(0, wave, lane);
                    const _Float16* s0 = src + l0.row * D + 8 * l0.gran;
#pragma unroll
                    for (int k = 0; k < MI; ++k)
                        __builtin_amdgcn_global_load_lds(s0 + k * 4 * NW * D, dst + plan::step16(l0, NW, k).slot * 1024, 16, 0, 0);
                };
                issue_map(1);
                if (np >= 2) issue_map(2);
                for (int i = 1; i <= np; ++i) {
                    // map i has landed (this wave's part; map i + 1's MI loads may still be in
                    // flight): vmcnt(MI), its bits [3:0] and [15:14], expcnt and lgkmcnt at their maxima
                    static_assert(MI < 64, "vmcnt holds 6 bits");
                    if (i + 1 <= np) __builtin_amdgcn_s_waitcnt((MI >> 4) << 14 | (MI & 15) | 0x7 << 4 | 0xF << 8);
                    else __builtin_amdgcn_s_waitcnt(0x7 << 4 | 0xF << 8);
                    __syncthreads();                        // ... and every wave's
                    const unsigned char* mb = g_stage + ((i - 1) & 1) * SG::BYTES;
                    float R[8][4];                          // R_{m0+i} at this lane's accumulator positions
                    const float* Rg = ws.Rseg + (static_cast<size_t>(m0 + i - 1) * nhh + head) * D * D;
                    int ro = 4 * g * D + col0 + r16;
                    asm volatile("" : "+v"(ro));            // formed here, not kept live from outside the loop
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) R[mt][e] = Rg[ro + (16 * mt + e) * D];
                    // B operands: the state's rows scaled by their map column tile's 2^e, into fp16 range
                    float sm = 0.f;
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt) {
                        const float sk = ldexpf(1.f, s_ek[i - 1][mt]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            S[mt][0][e] *= sk;
                            sm = fmaxf(sm, fabsf(S[mt][0][e]));
                        }
                    }
                    const int eP = pow2_exponent(wave_max_nonneg(sm));
                    const float sP = ldexpf(1.f, -eP), sc = ldexpf(1.f, eP);
                    f16x8 bh[4], bl[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float x = S[2 * ks + (e >> 2)][0][e & 3] * sP;
                            bh[ks][e] = static_cast<_Float16>(x);
                            bl[ks][e] = static_cast<_Float16>(x - static_cast<float>(bh[ks][e]));
                        }
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt) {
                        f32x4v acc = f32x4v{0, 0, 0, 0};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) {
                            const int row = 16 * mt + r16, pos = (4 * ks + g) ^ r16;
                            const f16x8 ah = *reinterpret_cast<const f16x8*>(mb + (row * 16 + pos) * 16);
                            const f16x8 al = *reinterpret_cast<const f16x8*>(mb + ((row + D) * 16 + pos) * 16);
                            acc = mfma16x16x32(ah, bh[ks], acc);
                            acc = mfma16x16x32(ah, bl[ks], acc);
                            acc = mfma16x16x32(al, bh[ks], acc);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) S[mt][0][e] = __fmaf_rn(acc[e], sc, R[mt][e]);
                    }
                    __syncthreads();                        // every wave is done with map i
                    if (i + 2 <= np) issue_map(i + 2);      // into the buffer just freed
                }
                smax = 0.f;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) smax = fmaxf(smax, fabsf(S[mt][0][e]));
                // without a loader wave each wave issues its share of the first chunk's
                // stage itself, into buffer 0, which the last barrier above freed
                if (!LW && cb < ce)
                    issue_all(base + cb, row_tok + static_cast<size_t>(cb) * C, min(C, seg.len - cb * C), 0, wave);
            }
        }
    }
    if (loader) {   // stage c + 1 is issued after the barrier that frees its buffer
        for (int c = cb; c < ce; ++c) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (c + 1 < ce) {
                const size_t tokn = row_tok + static_cast<size_t>(c + 1) * C;
                const int ntn = min(C, seg.len - (c + 1) * C);
                const int sbn = (c - cb + 1) & 1;
#pragma unroll
                for (int k = 0; k < NW / NL; ++k) issue_all(base + c + 1, tokn, ntn, sbn, li + NL * k);
            }
        }
        return;
    }
    // Fused gated RMSNorm (NORM): y = w * o / rms(o) * z * sigmoid(z) over each token's
    // 128 columns. A lane holds 4 columns of 4 tokens of a chunk's output; it keeps
    // them (and their gates, loaded while the chunk computes) until every wave's
    // share of the tokens' sums of squares is in LDS, i.e. past the next chunk's
    // first barrier (or one more barrier after the last chunk), and then stores y.
    __shared__ float s_ss[NORM ? 2 : 1][NORM ? C : 1][NORM ? NW : 1];   // [chunk parity][token][wave]
    f32x4v ov[4], wn{};
    uint2 zr[4];
    float* pob = nullptr;                                // pending chunk's first output row
    int pnt = 0;                                         // ... and its token count
    const bf16_t* zg = static_cast<const bf16_t*>(a.fu.z);
    if constexpr (NORM) {
        const bf16_t* wg = static_cast<const bf16_t*>(a.fu.norm_w) + col0 + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) wn[e] = to_f32(wg[e]);
    }
    auto bf_lo = [](unsigned u) { return __uint_as_float(u << 16); };
    auto bf_hi = [](unsigned u) { return __uint_as_float(u & 0xffff0000u); };
    auto finish = [&](int buf) {   // the pending chunk's y (sums of squares in s_ss[buf])
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int t = 16 * mt + r16;
            const f32x4v p0 = *reinterpret_cast<const f32x4v*>(&s_ss[buf][t][0]);
            const f32x4v p1 = *reinterpret_cast<const f32x4v*>(&s_ss[buf][t][4]);
            const float ss = ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
            const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.fu.norm_eps);
            const float z[4] = {bf_lo(zr[mt].x), bf_hi(zr[mt].x), bf_lo(zr[mt].y), bf_hi(zr[mt].y)};
            f32x4v y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = wn[e] * (ov[mt][e] * inv) * (z[e] * sigmoid_hw(z[e]));
            if (t < pnt) __builtin_nontemporal_store(y, reinterpret_cast<f32x4v*>(pob + t * ts + col0 + 4 * g));
        }
    };
    // The state is carried as S~ = S 2^-eS and each chunk's Delta formed as Delta 2^-eD,
    // with eS and eD kept from chunk to chunk while the largest magnitude stays inside
    // [2^kWinLo, 2^15) (fp16's range with room to spare; a wave vote, no cross-lane
    // maximum) and reset only when it leaves that window. Powers of two scale exactly,
    // so the results are those of scaling every chunk afresh, without its multiply per
    // element and its cross-lane reduction per chunk on the state's path.
    int eS = pow2_exponent(wave_max_nonneg(smax)), eD = 0;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[mt][nt][e] = ldexpf(S[mt][nt][e], -eS);
    smax = ldexpf(smax, -eS);
    // The next chunk's stage is issued in three parts spread over this chunk's
    // phases (each part before the phase that would otherwise wait on the memory
    // pipeline), so that the vector-memory issue queue never backs up the MFMA work.
    for (int c = cb; c < ce; ++c) {
        if constexpr (!LW) __builtin_amdgcn_s_waitcnt(0);   // this wave's share of the stage has landed
        __syncthreads();                 // ... and every wave's; the other stage is free
        const int id = base + c;
        const int ntc = min(C, seg.len - c * C);
        const size_t tok0 = row_tok + static_cast<size_t>(c) * C;
        const bool more = c + 1 < ce;
        const int ntn = min(C, seg.len - (c + 1) * C);
        const int sb_ = (c - cb + 1) & 1;                // stage buffer of the next chunk
        if (!LW && more) {
            if (useU)
                issue_stage<CPW, NW, ST_W | ST_U | ST_CF>(a, ws, id + 1, tok0 + C, ntn, h, hk, ucol0, sb_, wave, lane);
            else
                issue_stage<CPW, NW, ST_W | ST_CF>(a, ws, id + 1, tok0 + C, ntn, h, hk, ucol0, sb_, wave, lane);
        }
        if constexpr (NORM) {
            if (outs && c > cb) finish((c - 1 - cb) & 1);
        }
        const unsigned char* st = g_stage + ((c - cb) & 1) * SG::BYTES;
        const _Float16* Wl = reinterpret_cast<const _Float16*>(st + SG::W * 16);
        const _Float16* Ql = reinterpret_cast<const _Float16*>(st + SG::Q * 16);
        const _Float16* KTl = reinterpret_cast<const _Float16*>(st + SG::KT * 16);
        const _Float16* Pl = reinterpret_cast<const _Float16*>(st + SG::P * 16);
        const _Float16* Ul = reinterpret_cast<const _Float16*>(st + SG::U * 16);
        const float* cf = reinterpret_cast<const float*>(st + SG::CF * 16);   // exp(Gam_t)
        const float* cfr = cf + C;                                            // exp(Gam_last - Gam_t)
        const float egl = cf[2 * C], uscale = cf[2 * C + 1];

        // S~ as B operands (k = rows of S); back into the window first if it left it
        if (outside_window(smax)) {
            const int e2 = rescaled_exponent(eS, smax, eD);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[mt][nt][e] = ldexpf(S[mt][nt][e], eS - e2);
            eS = e2;
        }
        const float iS = ldexpf(1.f, eS);
        f16x8 sb[NTW][4];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sb[nt][ks][e] = static_cast<_Float16>(S[2 * ks][nt][e]);
                    sb[nt][ks][4 + e] = static_cast<_Float16>(S[2 * ks + 1][nt][e]);
                }

        // Delta 2^-eD = U uscale 2^-eD - (W S~) 2^(eS - eD). Rows past the end of the
        // sequence come out zero: W and U are zero there (zero keys, values and beta).
        float dl[4][NTW][4];
        float dmax = 0.f;
        const float uD = ldexpf(uscale, -eD);
        const int dS = eS - eD;
        if constexpr (BATCH) {
            f16x8 aw[4][4];
            _Float16 uh[4][NTW][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) aw[mt][ks] = lds_a<16>(Wl, 16 * mt + r16, ks, g);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const f16x4 u4 = lds_u4(Ul, lcol0 + 16 * nt + r16, 16 * mt + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) uh[mt][nt][e] = u4[e];
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4v acc[NTW];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4v{0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) acc[nt] = mfma16x16x32(aw[mt][ks], sb[nt][ks], acc[nt]);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float u = static_cast<float>(uh[mt][nt][e]);
                        const float d = __fmaf_rn(u, uD, -ldexpf(acc[nt][e], dS));
                        dl[mt][nt][e] = d;
                        dmax = fmaxf(dmax, fabsf(d));
                    }
            }
        } else {
    #pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4v acc[NTW];
    #pragma unroll
                for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4v{0, 0, 0, 0};
    #pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const f16x8 aw = lds_a<16>(Wl, 16 * mt + r16, ks, g);
    #pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) acc[nt] = mfma16x16x32(aw, sb[nt][ks], acc[nt]);
                }
    #pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * mt + 4 * g + e;
                        const float u = static_cast<float>(lds_u1(Ul, lcol0 + 16 * nt + r16, t));
                        const float d = __fmaf_rn(u, uD, -ldexpf(acc[nt][e], dS));
                        dl[mt][nt][e] = d;
                        dmax = fmaxf(dmax, fabsf(d));
                    }
            }
        }
        if (outside_window(dmax)) {   // Delta back into the window
            int eu;
            frexpf(uscale, &eu);
            const int e2 = rescaled_exponent(eD, dmax, max(eS, eu));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dl[mt][nt][e] = ldexpf(dl[mt][nt][e], eD - e2);
            eD = e2;
        }
        const float iD = ldexpf(1.f, eD);
        f16x8 db[NTW][2], dp[NTW][2];   // Delta and diag(exp(Gam_last - Gam)) Delta as B operands (k = token)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int mt = 2 * ks + (e >> 2), ee = e & 3;
                    const int t = 16 * mt + 4 * g + ee;
                    const float v = dl[mt][nt][ee];
                    db[nt][ks][e] = static_cast<_Float16>(v);
                    dp[nt][ks][e] = static_cast<_Float16>(v * cfr[t]);
                }

        if (!LW && more && outs)
            issue_stage<CPW, NW, ST_Q | ST_P>(a, ws, id + 1, tok0 + C, ntn, h, hk, ucol0, sb_, wave, lane);

        // O = diag(exp(Gam)) Q S + P Delta, stored as soon as it is formed. With one
        // tile per wave the products are formed transposed (S and Delta as the A
        // operands, Q and P as the B operands: the same registers), so that a lane
        // holds 4 consecutive columns of one token and stores them in one 16-byte
        // store: 4 store instructions per tile instead of 16 scattered dword stores.
        constexpr bool OT = NTW == 1;
        float* obase = a.o + (tok0 * a.Hv + h) * D;              // this chunk's first output row
        float* ob = obase + col0 + r16 + 4 * g * ts;
        const bool full = ntc == C;                            // uniform: every row stored
        // operands read ahead of the MFMAs when BATCH, OB row tiles at a time (one
        // with a loader wave: 256 registers, and each tile's reads then overlap the
        // previous tile's MFMAs: 237 -> 225 us at L = 4096), else inside the loop
        constexpr int OB = LW ? 1 : 4;
        if constexpr (NORM) {
            if (outs) {   // this chunk's gates (rows past the end: a row inside)
                const bf16_t* zb = zg + (tok0 * a.Hv + h) * D + col0 + 4 * g;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int t = min(16 * mt + r16, ntc - 1);
                    zr[mt] = *reinterpret_cast<const uint2*>(zb + t * ts);
                }
            }
        }
        if (outs) {
#pragma unroll
        for (int m0 = 0; m0 < 4; m0 += OB) {
        f16x8 aq[OB][4], ap[OB][2];
        if constexpr (BATCH) {
#pragma unroll
            for (int mi = 0; mi < OB; ++mi) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) aq[mi][ks] = lds_a<16>(Ql, 16 * (m0 + mi) + r16, ks, g);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ap[mi][ks] = lds_a<8>(Pl, 16 * (m0 + mi) + r16, ks, g);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int mi = 0; mi < OB; ++mi) {
            const int mt = m0 + mi;
            f32x4v a1[NTW], a2[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) { a1[nt] = f32x4v{0, 0, 0, 0}; a2[nt] = a1[nt]; }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if constexpr (!BATCH) aq[mi][ks] = lds_a<16>(Ql, 16 * mt + r16, ks, g);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    a1[nt] = OT ? mfma16x16x32(sb[nt][ks], aq[mi][ks], a1[nt]) : mfma16x16x32(aq[mi][ks], sb[nt][ks], a1[nt]);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if constexpr (!BATCH) ap[mi][ks] = lds_a<8>(Pl, 16 * mt + r16, ks, g);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    a2[nt] = OT ? mfma16x16x32(db[nt][ks], ap[mi][ks], a2[nt]) : mfma16x16x32(ap[mi][ks], db[nt][ks], a2[nt]);
            }
            if constexpr (OT) {   // lane: token 16 mt + r16, columns col0 + 4 g .. + 3
                const int t = 16 * mt + r16;
                const float eg = cf[t] * iS;
                const float4 v = make_float4(__fmaf_rn(eg, a1[0][0], iD * a2[0][0]), __fmaf_rn(eg, a1[0][1], iD * a2[0][1]),
                                             __fmaf_rn(eg, a1[0][2], iD * a2[0][2]), __fmaf_rn(eg, a1[0][3], iD * a2[0][3]));
                if constexpr (NORM) {   // held for the norm; this wave's 16 columns of the token's sum of squares
                    ov[mt] = f32x4v{v.x, v.y, v.z, v.w};
                    float ss = __fmaf_rn(v.w, v.w, __fmaf_rn(v.z, v.z, __fmaf_rn(v.y, v.y, v.x * v.x)));
                    ss += __shfl_xor(ss, 16);
                    ss += __shfl_xor(ss, 32);
                    if (g == 0) s_ss[(c - cb) & 1][t][wave] = ss;
                } else if (full || t < ntc) {
                    __builtin_nontemporal_store(f32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4v*>(obase + t * ts + col0 + 4 * g));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float eg = cf[16 * mt + 4 * g + e] * iS;
                    if (full || 16 * mt + 4 * g + e < ntc) {
                        float* orow = ob + (16 * mt + e) * ts;
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt)
                            __builtin_nontemporal_store(__fmaf_rn(eg, a1[nt][e], iD * a2[nt][e]), orow + 16 * nt);
                    }
                }
            }
        }
        }
        }
        if constexpr (NORM) {
            pob = obase;
            pnt = ntc;
        }
        if (!LW && more)
            issue_stage<CPW, NW, ST_KT>(a, ws, id + 1, tok0 + C, ntn, h, hk, ucol0, sb_, wave, lane);

        // S~ = exp(Gam_last) S~ + 2^(eD - eS) K^T diag(exp(Gam_last - Gam)) Delta 2^-eD;
        // max|S~| of this lane for the next chunk's window check
        smax = 0.f;
        f16x8 ak[8][2];
        if constexpr (BATCH) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ak[mt][ks] = lds_a<8>(KTl, 16 * mt + r16, ks, g);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            f32x4v acc[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4v{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if constexpr (!BATCH) ak[mt][ks] = lds_a<8>(KTl, 16 * mt + r16, ks, g);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) acc[nt] = mfma16x16x32(ak[mt][ks], dp[nt][ks], acc[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    S[mt][nt][e] = __fmaf_rn(egl, S[mt][nt][e], ldexpf(acc[nt][e], eD - eS));
                    smax = fmaxf(smax, fabsf(S[mt][nt][e]));
                }
        }
    }
    // back to S itself
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[mt][nt][e] = ldexpf(S[mt][nt][e], eS);
    smax = ldexpf(smax, eS);
    if constexpr (NORM) {
        if (outs && ce > cb) {
            __syncthreads();                                 // every wave's sums of the last chunk
            finish((ce - 1 - cb) & 1);
        }
    }
    // end state: S, or in segmented mode an entry state, R_j or M_j (or nothing). M_j
    // goes out split into fp16 high and low parts scaled per 16-column tile (a wave's
    // columns), staged through LDS into row-major planes with the columns in k order
    // (the order in which a state's accumulator tiles act as B operands).
    if constexpr (!LW && NTW == 1) {
        if (mapo != 0) {
            const size_t m = mapo - 1;                   // (segment, sequence, head) of the map
            // the tile's largest magnitude over the whole wave (smax is per lane: a lane
            // holds 32 of the tile's 2048 entries, which can all be zero in a nonzero tile)
            const float tmax = wave_max_nonneg(smax);
            const int eC = pow2_exponent(tmax);
            const float sC = ldexpf(1.f, -eC);
            constexpr int MS = D + 8;                    // LDS row stride (halfs)
            _Float16* lh = reinterpret_cast<_Float16*>(g_stage);
            _Float16* ll = lh + D * MS;
            __syncthreads();                             // every wave is done with the stages
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = S[mt][0][e] * sC;
                    const _Float16 hi = static_cast<_Float16>(x);
                    lh[(16 * mt + 4 * g + e) * MS + kpos(col0 + r16)] = hi;
                    ll[(16 * mt + 4 * g + e) * MS + kpos(col0 + r16)] = static_cast<_Float16>(x - static_cast<float>(hi));
                }
            if (lane == 0) ws.Mexp[m * (D / 16) + col0 / 16] = tmax > 0.f ? eC : kZeroTile;
            __syncthreads();
            _Float16* dst = ws.Mhl + m * 2 * D * D;
            for (int q = tid; q < 2 * D * (D / 8); q += NW * 64) {   // 16-byte granules of both planes
                const int pl = q / (D * D / 8), row = (q / (D / 8)) % D, j8 = q % (D / 8);
                const uint4 v = *reinterpret_cast<const uint4*>(lh + pl * D * MS + row * MS + 8 * j8);
                *reinterpret_cast<uint4*>(dst + static_cast<size_t>(pl) * D * D + row * D + 8 * j8) = v;
            }
        }
    }
    if (Send != nullptr) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_nontemporal_store(S[mt][nt][e], Send + (16 * mt + 4 * g + e) * D + col0 + 16 * nt + r16);
    }
}

}  // namespace pf2

size_t prefill_mfma_workspace_bytes(int B, int L, int N, int Hk, int Hv, bool ragged, bool norm) {
    return pf2::layout(nullptr, B, L, N, Hk, Hv, ragged, norm).bytes;
}

// Whole-head carry workgroups: 8 waves of one 16-column tile each (two waves per
// SIMD hide each other's LDS and MFMA latencies; on the 8-sequence ragged prefill
// this beat 4 waves of two tiles by 10%).
constexpr int kWholeNTW = 1, kWholeNW = 8;

// Compute units of the current device (queried once per device).
static int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// The carry configurations: (tiles per wave, waves per workgroup, loader waves, fused
// norm, number of loader waves).
template <int NTW, int NW, bool LW = false, bool NORM = false, int NL = 1>
static hipError_t launch_carry(void** args, long long heads, hipStream_t stream) {
    constexpr int CPW = NW * NTW * 16;
    constexpr size_t lds = 2 * pf2::Stage<CPW>::BYTES;
    static_assert(lds + 8 * 1024 <= 160 * 1024, "LDS of one CU (the stages and the kernel's static arrays)");
    const void* k = reinterpret_cast<const void*>(&pf2::carry_kernel<NTW, NW, LW, NORM, NL>);
    // dynamic LDS above 64 KB must be allowed per kernel before its first launch
    static const hipError_t allowed = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (allowed != hipSuccess) return allowed;
    return hipLaunchKernel(k, dim3(static_cast<unsigned>(heads * (128 / CPW))), dim3((NW + (LW ? NL : 0)) * 64), args, lds,
                           stream);
}

template <typename Tin>
static hipError_t launch_mfma_t(const PrefillArgs& a, int in_dtype, hipStream_t stream) {
    const bool ragged = a.cu != nullptr;
    const bool norm = a.fu.z != nullptr;   // the gated RMSNorm fused into the carry's output store
    pf2::Ws ws = pf2::layout(a.ws, a.B, a.L, a.N, a.Hk, a.Hv, ragged, norm);
    const int cus = device_cu_count();
    ws.nseg = plan::carry_plan(a.B, a.L, a.N, a.Hv, ragged, cus, norm).nseg;   // within the workspace's
    void* args[] = {const_cast<PrefillArgs*>(&a), &ws};
    hipError_t e;
    const long long fblocks = static_cast<long long>(a.B) * ((a.L + pf2::TT - 1) / pf2::TT) * (2 * a.Hk);
    if (fblocks > 0) {
        e = hipLaunchKernel(reinterpret_cast<const void*>(&pf2::front_kernel<Tin>), dim3(static_cast<unsigned>(fblocks)),
                            dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    if (fblocks == 0) {   // no tokens: every state stays as it is, and the conv windows are copied
        ConvArgs ca{a.B, a.L, a.D, a.N, a.qkv, a.w, a.conv_in, a.conv_out, nullptr, a.cu};
        return launch_conv_state(ca, in_dtype, stream);
    }
    // (the front kernel wrote the chunk slot table of packed prompts that the next kernels read)
    const long long cblocks = static_cast<long long>(ws.nc_max) * a.Hv;
    if (cblocks > 0) {
        e = hipLaunchKernel(reinterpret_cast<const void*>(&pf2::chunk_kernel<Tin>), dim3(static_cast<unsigned>(cblocks)),
                            dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    // carry launches (plan::carry_plan: whole-head or half-head workgroups, one pass or
    // the two of the segmented carry); with the gated RMSNorm fused into the output
    // store, whole-head workgroups only
    const plan::CarryPlan cp = plan::carry_plan(a.B, a.L, a.N, a.Hv, ragged, cus, norm);
    for (int i = 0; i < cp.count; ++i) {
        pf2::Ws wp = ws;
        wp.pass = cp.l[i].pass;
        void* argp[] = {const_cast<PrefillArgs*>(&a), &wp};
        static_assert(kWholeNTW == 1, "the first pass writes the state maps from one column tile per wave");
        if (norm) e = launch_carry<kWholeNTW, kWholeNW, false, true>(argp, cp.l[i].units, stream);
        // the second pass (entry states from the maps first) with two loader waves: the
        // first chunk's stage goes out sooner after the prologue (L=4096 1-3 us faster);
        // one loader for the unsegmented carry, where two measured no gain
        else if (cp.l[i].half && cp.l[i].pass == 2) e = launch_carry<1, 4, true, false, 2>(argp, cp.l[i].units, stream);
        else if (cp.l[i].half) e = launch_carry<1, 4, true>(argp, cp.l[i].units, stream);
        else e = launch_carry<kWholeNTW, kWholeNW>(argp, cp.l[i].units, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;   // the front and chunk kernels wrote the conv state
}

// Runs the gated RMSNorm of gdn_prefill_ex too when a.fu.z is set (fused into the carry).
hipError_t launch_prefill_mfma(const PrefillArgs& a, int in_dtype, hipStream_t stream) {
    // bf16 inputs only: fp32 inputs take the fp32 path, whose tolerance the fp16 operands would not meet
    return in_dtype == 1 ? launch_mfma_t<bf16_t>(a, in_dtype, stream) : hipErrorInvalidValue;
}

}  // namespace gdn
