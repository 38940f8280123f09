// Chunked prefill of the Gated DeltaNet layer ("MNN Model Support: Qwen3.5",
// §1.2 steps 1-5 over a whole prompt, §1.3 reverse GQA, §1.4 carried states).
// This file holds the fp32 vector-ALU version, used for fp32 inputs and for
// head dim 16; bf16 inputs at head dim 128 run on MFMA (gdn_prefill_mfma.hip)
// with the same chunk algebra.
//
// Step 5 is evaluated chunk by chunk (chunk length C). Inside a chunk, with
// Gam_t the inclusive cumulative sum of the log-decays g and S0 the state on
// entry, unrolling the recurrence gives exactly
//   A_ts  = beta_t exp(Gam_t - Gam_s) (k_t . k_s)         (s < t, else 0)
//   T     = (I + A)^-1                                      (unit lower triangular)
//   W     = T diag(beta exp(Gam)) K,   U = T diag(beta) V
//   Delta = U - W S0                     (row t = the delta of token t)
//   O     = diag(exp(Gam)) Q S0 + P Delta,  P_ts = exp(Gam_t - Gam_s) (q_t . k_s), s <= t
//   S_C   = exp(Gam_last) S0 + K^T diag(exp(Gam_last - Gam)) Delta
// Every exponent is Gam_t - Gam_s with s <= t or Gam itself, all <= 0, so no
// exp() can overflow however strong the decay.
//
// Three kernels:
//   prefill_front_kernel  steps 1-4: conv + SiLU of a (head, 32-token) tile,
//                         transposed through LDS from channel-major input to
//                         token-major head vectors, L2 norms and q scale.
//   prefill_chunk_kernel  per (chunk, V head): Gam, A, T, W, U and P; parallel
//                         over every chunk of every sequence.
//   prefill_carry_kernel  per (sequence, V head, 16-column slice of S): the
//                         state carried from chunk to chunk and the outputs.
//                         The columns of S evolve independently (each needs
//                         only k, q, g, beta and its own v column), which is
//                         what lets the sequential part split over slices.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"
#include "gdn_packed.hpp"

namespace gdn {

constexpr int kFrontTile = 32;   // tokens per front-end workgroup
constexpr int kSlice = 16;       // columns of S per carry workgroup

// ---- workspace layout --------------------------------------------------------
struct PrefillWs {
    float* qh;    // [Ttot, Hk, d]   q_hat (normalised, scaled)
    float* kh;    // [Ttot, Hk, d]   k_hat
    float* vv;    // [Ttot, Hv, d]   v
    float* W;     // [Ttot, Hv, d]
    float* U;     // [Ttot, Hv, d]
    float* gam;   // [Ttot, Hv]      cumulative log-decay inside the chunk
    float* P;     // [NCmax, Hv, C, C]
    int* cbase;   // [N + 1] packed prompts: first chunk slot of each sequence (write_chunk_bases)
    int nc_max;   // chunk slots of P
    size_t bytes;
};

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static int max_chunks(int B, int L, int N, int C, bool ragged) {
    const int per = (L + C - 1) / C;
    return ragged ? per + N : B * per;
}

static PrefillWs ws_layout(void* base, int B, int L, int N, int Hk, int Hv, int d, int C, bool ragged) {
    PrefillWs w;
    const size_t Ttot = static_cast<size_t>(B) * L;
    const size_t nc = static_cast<size_t>(max_chunks(B, L, N, C, ragged));
    size_t off = 0;
    auto take = [&](size_t n) {
        float* r = base ? reinterpret_cast<float*>(static_cast<char*>(base) + off) : nullptr;
        off = align256(off + n * sizeof(float));
        return r;
    };
    w.qh = take(Ttot * Hk * d);
    w.kh = take(Ttot * Hk * d);
    w.vv = take(Ttot * Hv * d);
    w.W = take(Ttot * Hv * d);
    w.U = take(Ttot * Hv * d);
    w.gam = take(Ttot * Hv);
    w.P = take(nc * Hv * C * C);
    w.cbase = ragged ? reinterpret_cast<int*>(take(static_cast<size_t>(N) + 1)) : nullptr;
    w.nc_max = static_cast<int>(nc);
    w.bytes = off;
    return w;
}

size_t prefill_workspace_bytes(int B, int L, int N, int Hk, int Hv, int d, int chunk, int in_dtype, bool ragged,
                               bool norm) {
    // the layout of the path the call takes: MFMA for bf16 inputs at d = 128, else the
    // fp32 path (whose gated RMSNorm is a pass over o that needs no workspace)
    if (d == 128 && in_dtype == 1) return prefill_mfma_workspace_bytes(B, L, N, Hk, Hv, ragged, norm);
    return ws_layout(nullptr, B, L, N, Hk, Hv, d, chunk, ragged).bytes;
}

// Number of chunks of sequence n.
__device__ __forceinline__ int chunks_of(const Seg& s, int C) { return (s.len + C - 1) / C; }

// ---- steps 1-4 -----------------------------------------------------------------
template <typename Tin, int DH>
__global__ __launch_bounds__(256) void prefill_front_kernel(PrefillArgs a, PrefillWs ws) {
    constexpr int TT = kFrontTile;
    constexpr int HALO = kConvK - 1;
    __shared__ float raw[DH][TT + HALO];
    __shared__ float ys[TT][DH + 1];
    __shared__ int s_n[TT], s_start[TT];

    const int units = 2 * a.Hk + a.Hv;
    const int tiles = (a.L + TT - 1) / TT;
    long long blk = blockIdx.x;
    const int u = static_cast<int>(blk % units); blk /= units;
    const int tile = static_cast<int>(blk % tiles);
    const int row = static_cast<int>(blk / tiles);
    const int p0 = tile * TT;
    const int ch0 = u * DH;  // [Q | K | V] blocks of DH channels (dk == dv)
    const Tin* x = static_cast<const Tin*>(a.qkv) + (static_cast<size_t>(row) * a.D + ch0) * a.L;
    const Tin* w = static_cast<const Tin*>(a.w);
    const Tin* cin = static_cast<const Tin*>(a.conv_in);
    // packed prompts: the first workgroup writes the chunk slot table of the chunk and
    // carry kernels
    if (a.cu != nullptr && blockIdx.x == 0) write_chunk_bases(a.N, a.L, a.cu, a.chunk, ws.nc_max, ws.cbase);

    if (threadIdx.x < TT) {
        const int p = p0 + threadIdx.x;
        int n = -1, start = 0;
        if (p < a.L) {
            if (a.cu == nullptr) { n = row; start = 0; }
            else {
                int lo = 0, hi = a.N - 1;
                while (lo <= hi) {
                    const int mid = (lo + hi) >> 1;
                    int st = a.cu[mid];
                    st = st < 0 ? 0 : (st > a.L ? a.L : st);
                    if (st <= p) { n = mid; lo = mid + 1; } else { hi = mid - 1; }
                }
                if (n >= 0) {
                    const Seg sg = segment_of(n, a.L, a.cu);
                    if (p >= sg.start + sg.len) n = -1; else start = sg.start;
                }
            }
        }
        s_n[threadIdx.x] = n;
        s_start[threadIdx.x] = start;
    }
    for (int e = threadIdx.x; e < DH * (TT + HALO); e += 256) {
        const int c = e / (TT + HALO), m = e - c * (TT + HALO);
        const int pos = p0 - HALO + m;
        raw[c][m] = (pos >= 0 && pos < a.L) ? to_f32(x[static_cast<size_t>(c) * a.L + pos]) : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < DH * TT; e += 256) {
        const int c = e / TT, t = e - c * TT;
        const int n = s_n[t];
        if (n < 0) { ys[t][c] = 0.f; continue; }
        const int ch = ch0 + c;
        const int uu = p0 + t - s_start[t];  // index inside the sequence
        float wv[kConvK], win[kConvK];
#pragma unroll
        for (int j = 0; j < kConvK; ++j) {
            wv[j] = to_f32(w[static_cast<size_t>(ch) * kConvK + j]);
            const int m = uu + j;  // position in concat(state, x[seq])
            win[j] = (m < HALO) ? to_f32(cin[(static_cast<size_t>(n) * a.D + ch) * HALO + m]) : raw[c][t + j];
        }
        ys[t][c] = conv_silu(wv, win);
    }
    __syncthreads();
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const bool is_q = u < a.Hk, is_k = !is_q && u < 2 * a.Hk;
    const float qscale = 1.0f / sqrtf(static_cast<float>(DH));
    for (int t = wave; t < TT; t += 256 / kWave) {
        if (s_n[t] < 0) continue;
        float r = 1.0f;
        if (is_q || is_k) {
            float ss = 0.f;
            for (int c = lane; c < DH; c += kWave) ss = __fmaf_rn(ys[t][c], ys[t][c], ss);
            ss = wave_sum(ss);
            if (a.use_l2) r = 1.0f / sqrtf(ss + a.eps);
            if (is_q) r *= qscale;
        }
        const size_t tok = static_cast<size_t>(row) * a.L + p0 + t;
        float* dst;
        if (is_q) dst = ws.qh + (tok * a.Hk + u) * DH;
        else if (is_k) dst = ws.kh + (tok * a.Hk + (u - a.Hk)) * DH;
        else dst = ws.vv + (tok * a.Hv + (u - 2 * a.Hk)) * DH;
        for (int c = lane; c < DH; c += kWave) dst[c] = ys[t][c] * r;
    }
}

// Locate chunk slot `id` of the launch: sequence n and chunk index inside it (rows of
// equal length unpacked, the table of first slots packed).
__device__ __forceinline__ bool find_chunk(int id, const PrefillArgs& a, const PrefillWs& ws, int* n_out,
                                           int* c_out, Seg* seg) {
    if (a.cu == nullptr) {
        const int per = (a.L + a.chunk - 1) / a.chunk;
        if (per == 0 || id >= a.N * per) return false;
        *n_out = id / per;
        *c_out = id - *n_out * per;
    } else if (!chunk_slot(id, a.N, ws.cbase, n_out, c_out)) {
        return false;
    }
    *seg = segment_of(*n_out, a.L, a.cu);
    return *c_out >= 0 && *c_out < chunks_of(*seg, a.chunk);   // (always, from the table the front kernel wrote)
}

// ---- chunk phase: Gam, A, T, W, U, P ---------------------------------------------
template <typename Tin, int DK, int DV, int C>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(PrefillArgs a, PrefillWs ws) {
    __shared__ float sA[C][C + 1];
    __shared__ float sT[C][C + 1];
    __shared__ float s_g[C], s_b[C], s_gam[C];
    const int h = blockIdx.x % a.Hv;
    const int id = blockIdx.x / a.Hv;
    int n, c;
    Seg seg;
    if (id >= ws.nc_max || !find_chunk(id, a, ws, &n, &c, &seg)) return;
    const int f = a.Hv / a.Hk, hk = h / f;
    const int nt = min(C, seg.len - c * C);
    const size_t tok0 = static_cast<size_t>(seg.row) * a.L + seg.start + static_cast<size_t>(c) * C;
    const Tin* gate = static_cast<const Tin*>(a.gate);
    const Tin* beta = static_cast<const Tin*>(a.beta);
    const int tid = threadIdx.x;
    if (tid < C) {
        float gv = 0.f, bv = 0.f;
        if (tid < nt) gate_beta_at<Tin>(gate, beta, a.fu.A_log, a.fu.dt_bias, (tok0 + tid) * a.Hv + h, h, &gv, &bv);
        s_g[tid] = gv;
        s_b[tid] = bv;
    }
    __syncthreads();
    if (tid == 0) {
        float acc = 0.f;
        for (int t = 0; t < C; ++t) { acc += s_g[t]; s_gam[t] = acc; }
    }
    __syncthreads();
    const float* kh = ws.kh + hk * DK;  // row t at kh + tok * Hk * DK
    const float* qh = ws.qh + hk * DK;
    const size_t kstride = static_cast<size_t>(a.Hk) * DK;
    float* P = ws.P + (static_cast<size_t>(id) * a.Hv + h) * C * C;
    for (int e = tid; e < C * C; e += 256) {
        const int t = e / C, s = e - t * C;
        float kk = 0.f, qk = 0.f;
        if (t < nt && s < nt && s <= t) {
            const float* kt = kh + (tok0 + t) * kstride;
            const float* ks = kh + (tok0 + s) * kstride;
            const float* qt = qh + (tok0 + t) * kstride;
            for (int i = 0; i < DK; ++i) {
                kk = __fmaf_rn(kt[i], ks[i], kk);
                qk = __fmaf_rn(qt[i], ks[i], qk);
            }
        }
        const float dec = (s <= t) ? expf(s_gam[t] - s_gam[s]) : 0.f;
        sA[t][s] = (s < t) ? s_b[t] * dec * kk : 0.f;
        P[e] = dec * qk;
    }
    __syncthreads();
    // T = (I + A)^-1 by forward substitution, one row at a time
    for (int t = 0; t < C; ++t) {
        if (tid < C) {
            const int j = tid;
            float v = (j == t) ? 1.f : 0.f;
            if (j < t) {
                for (int s = j; s < t; ++s) v = __fmaf_rn(-sA[t][s], sT[s][j], v);
            }
            sT[t][j] = v;
        }
        __syncthreads();
    }
    // W = T diag(beta exp(Gam)) K,  U = T diag(beta) V
    const float* vv = ws.vv + static_cast<size_t>(h) * DV;
    const size_t vstride = static_cast<size_t>(a.Hv) * DV;
    for (int e = tid; e < nt * DK; e += 256) {
        const int t = e / DK, i = e - t * DK;
        float acc = 0.f;
        for (int s = 0; s <= t; ++s)
            acc = __fmaf_rn(sT[t][s] * (s_b[s] * expf(s_gam[s])), kh[(tok0 + s) * kstride + i], acc);
        ws.W[((tok0 + t) * a.Hv + h) * DK + i] = acc;
    }
    for (int e = tid; e < nt * DV; e += 256) {
        const int t = e / DV, j = e - t * DV;
        float acc = 0.f;
        for (int s = 0; s <= t; ++s)
            acc = __fmaf_rn(sT[t][s] * s_b[s], vv[(tok0 + s) * vstride + j], acc);
        ws.U[((tok0 + t) * a.Hv + h) * DV + j] = acc;
    }
    if (tid < nt) ws.gam[(tok0 + tid) * a.Hv + h] = s_gam[tid];
}

// ---- state carry + outputs -----------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(256) void prefill_carry_kernel(PrefillArgs a, PrefillWs ws) {
    constexpr int NS = DV / kSlice;
    __shared__ float Ss[DK][kSlice];
    __shared__ float Dl[C][kSlice];
    __shared__ float s_gam[C];
    const int sl = blockIdx.x % NS;
    const int h = (blockIdx.x / NS) % a.Hv;
    const int n = blockIdx.x / (NS * a.Hv);
    const int j0 = sl * kSlice;
    const int f = a.Hv / a.Hk, hk = h / f;
    const int tid = threadIdx.x;
    const Seg seg = segment_of(n, a.L, a.cu);
    // chunk slot of this sequence's first chunk
    const int base = a.cu != nullptr ? min(max(ws.cbase[n], 0), ws.nc_max) : n * ((a.L + C - 1) / C);
    const int nchunks = chunks_of(seg, C);

    float* Sg = a.S + (static_cast<size_t>(n) * a.Hv + h) * DK * DV + j0;
    for (int e = tid; e < DK * kSlice; e += 256) Ss[e / kSlice][e % kSlice] = Sg[static_cast<size_t>(e / kSlice) * DV + e % kSlice];
    __syncthreads();

    const size_t kstride = static_cast<size_t>(a.Hk) * DK;
    for (int c = 0; c < nchunks; ++c) {
        // only malformed cu_seqlens (overlapping sequences) can run past the chunk slots
        if (base + c >= ws.nc_max) break;
        const int nt = min(C, seg.len - c * C);
        const size_t tok0 = static_cast<size_t>(seg.row) * a.L + seg.start + static_cast<size_t>(c) * C;
        if (tid < C) s_gam[tid] = tid < nt ? ws.gam[(tok0 + tid) * a.Hv + h] : 0.f;
        // Delta = U - W S
        {
            const int t = tid / 4, jq = (tid % 4) * 4;
            float d[4] = {0.f, 0.f, 0.f, 0.f};
            if (t < nt) {
                const float* Wt = ws.W + ((tok0 + t) * a.Hv + h) * DK;
                const float* Ut = ws.U + ((tok0 + t) * a.Hv + h) * DV + j0 + jq;
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
                for (int i = 0; i < DK; ++i) {
                    const float wv = Wt[i];
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q] = __fmaf_rn(wv, Ss[i][jq + q], acc[q]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) d[q] = Ut[q] - acc[q];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) Dl[t][jq + q] = d[q];
        }
        __syncthreads();
        const float gl = s_gam[nt - 1 < 0 ? 0 : nt - 1];
        // O = diag(exp(Gam)) Q S + P Delta
        {
            const int t = tid / 4, jq = (tid % 4) * 4;
            if (t < nt) {
                const float* Qt = ws.qh + (tok0 + t) * kstride + hk * DK;
                float qs[4] = {0.f, 0.f, 0.f, 0.f};
                for (int i = 0; i < DK; ++i) {
                    const float qv = Qt[i];
#pragma unroll
                    for (int q = 0; q < 4; ++q) qs[q] = __fmaf_rn(qv, Ss[i][jq + q], qs[q]);
                }
                const float* Pt = ws.P + ((static_cast<size_t>(base + c) * a.Hv + h) * C + t) * C;
                float pd[4] = {0.f, 0.f, 0.f, 0.f};
                for (int s = 0; s <= t; ++s) {
                    const float pv = Pt[s];
#pragma unroll
                    for (int q = 0; q < 4; ++q) pd[q] = __fmaf_rn(pv, Dl[s][jq + q], pd[q]);
                }
                const float eg = expf(s_gam[t]);
                float* ot = a.o + ((tok0 + t) * a.Hv + h) * DV + j0 + jq;
#pragma unroll
                for (int q = 0; q < 4; ++q) ot[q] = __fmaf_rn(eg, qs[q], pd[q]);
            }
        }
        __syncthreads();
        // S = exp(Gam_last) S + K^T diag(exp(Gam_last - Gam)) Delta
        {
            constexpr int ITEMS = DK * (kSlice / 8);
            const int i = tid / 2, jq = (tid % 2) * 8;
            float nv[8];
            if (tid < ITEMS) {
                float acc[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = 0.f;
                for (int s = 0; s < nt; ++s) {
                    const float kv = ws.kh[(tok0 + s) * kstride + hk * DK + i] * expf(gl - s_gam[s]);
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc[q] = __fmaf_rn(kv, Dl[s][jq + q], acc[q]);
                }
                const float eg = expf(gl);
#pragma unroll
                for (int q = 0; q < 8; ++q) nv[q] = __fmaf_rn(eg, Ss[i][jq + q], acc[q]);
            }
            __syncthreads();
            if (tid < ITEMS) {
#pragma unroll
                for (int q = 0; q < 8; ++q) Ss[i][jq + q] = nv[q];
            }
        }
        __syncthreads();
    }
    for (int e = tid; e < DK * kSlice; e += 256) Sg[static_cast<size_t>(e / kSlice) * DV + e % kSlice] = Ss[e / kSlice][e % kSlice];
}

template <typename Tin, int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, int in_dtype, hipStream_t stream) {
    constexpr int C = 64;
    const bool ragged = a.cu != nullptr;
    PrefillWs ws = ws_layout(a.ws, a.B, a.L, a.N, a.Hk, a.Hv, D, C, ragged);
    const int nc = max_chunks(a.B, a.L, a.N, C, ragged);
    hipError_t e;
    {
        const long long blocks = static_cast<long long>(a.B) * ((a.L + kFrontTile - 1) / kFrontTile) * (2 * a.Hk + a.Hv);
        void* args[] = {const_cast<PrefillArgs*>(&a), &ws};
        if (blocks == 0) {   // no tokens: every state stays as it is, and the conv windows are copied
            ConvArgs ca{a.B, a.L, a.D, a.N, a.qkv, a.w, a.conv_in, a.conv_out, nullptr, a.cu};
            return launch_conv_state(ca, in_dtype, stream);
        }
        e = hipLaunchKernel(reinterpret_cast<const void*>(&prefill_front_kernel<Tin, D>),
                            dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    // (the front kernel wrote the chunk slot table of packed prompts that the next kernels read)
    {
        const long long blocks = static_cast<long long>(nc) * a.Hv;
        void* args[] = {const_cast<PrefillArgs*>(&a), &ws};
        if (blocks > 0) {
            e = hipLaunchKernel(reinterpret_cast<const void*>(&prefill_chunk_kernel<Tin, D, D, C>),
                                dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0, stream);
            if (e != hipSuccess) return e;
        }
    }
    {
        const long long blocks = static_cast<long long>(a.N) * a.Hv * (D / kSlice);
        void* args[] = {const_cast<PrefillArgs*>(&a), &ws};
        if (blocks > 0) {
            e = hipLaunchKernel(reinterpret_cast<const void*>(&prefill_carry_kernel<D, D, C>),
                                dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0, stream);
            if (e != hipSuccess) return e;
        }
    }
    ConvArgs ca{a.B, a.L, a.D, a.N, a.qkv, a.w, a.conv_in, a.conv_out, nullptr, a.cu};
    return launch_conv_state(ca, in_dtype, stream);
}

// Gated RMSNorm of the prefill output in place (the epilogue of gdn_fusion).
// One workgroup per token (all Hv rows of it; tokens outside every sequence are
// left untouched, decided once per workgroup); a row of DV channels is reduced
// by a group of G = min(DV, 64) lanes, and a wave's rows are loaded before any
// is reduced so that their loads are in flight together.
template <typename Tin, int DV>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(PrefillArgs a) {
    constexpr int G = DV < kWave ? DV : kWave;          // lanes per row
    constexpr int RPW = kWave / G;                      // rows per wave pass
    constexpr int PER = DV / G;                         // channels per lane
    constexpr int UNR = 4;                              // passes in flight
    const long long tok = blockIdx.x;                   // row * L + position
    if (a.cu != nullptr && token_owner(static_cast<int>(tok % a.L), a.L, a.N, a.cu) < 0) return;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int sub = lane / G, gl = lane % G;
    float* o = a.o + tok * a.Hv * DV;
    const Tin* z = static_cast<const Tin*>(a.fu.z) + tok * a.Hv * DV;
    const Tin* w = static_cast<const Tin*>(a.fu.norm_w);
    float wn[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) wn[q] = to_f32(w[gl + q * G]);
    // pass k of this wave covers heads (k * 4 + wave) * RPW + sub
    for (int k0 = 0; (k0 * 4 + wave) * RPW < a.Hv; k0 += UNR) {
        float v[UNR][PER], zv[UNR][PER];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int h = ((k0 + u) * 4 + wave) * RPW + sub;
            const int hc = h < a.Hv ? h : a.Hv - 1;     // clamped: loads stay unconditional
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                v[u][q] = o[static_cast<size_t>(hc) * DV + gl + q * G];
                zv[u][q] = to_f32(z[static_cast<size_t>(hc) * DV + gl + q * G]);
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int h = ((k0 + u) * 4 + wave) * RPW + sub;
            float ss = 0.f;
#pragma unroll
            for (int q = 0; q < PER; ++q) ss = __fmaf_rn(v[u][q], v[u][q], ss);
#pragma unroll
            for (int m = G / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);
            const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + a.fu.norm_eps);
            if (h < a.Hv) {
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    o[static_cast<size_t>(h) * DV + gl + q * G] = wn[q] * (v[u][q] * inv) * (zv[u][q] * sigmoid_hw(zv[u][q]));
            }
        }
    }
}

template <typename Tin, int DV>
static hipError_t launch_epi_t(const PrefillArgs& a, hipStream_t stream) {
    const long long toks = static_cast<long long>(a.B) * a.L;
    if (toks == 0) return hipSuccess;
    if (toks > 0x7fffffffLL) return hipErrorInvalidValue;
    void* args[] = {const_cast<PrefillArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gated_rmsnorm_kernel<Tin, DV>),
                           dim3(static_cast<unsigned>(toks)), dim3(256), args, 0, stream);
}

hipError_t launch_prefill_epilogue(const PrefillArgs& a, int in_dtype, int d, hipStream_t stream) {
    if (d == 128) return in_dtype == 1 ? launch_epi_t<bf16_t, 128>(a, stream) : launch_epi_t<float, 128>(a, stream);
    if (d == 64) return in_dtype == 1 ? launch_epi_t<bf16_t, 64>(a, stream) : launch_epi_t<float, 64>(a, stream);
    return in_dtype == 1 ? launch_epi_t<bf16_t, 16>(a, stream) : launch_epi_t<float, 16>(a, stream);
}

static hipError_t launch_prefill_core(const PrefillArgs& a, int in_dtype, int d, hipStream_t stream) {
    // bf16 inputs run the dense products on fp16 MFMA (within the bf16 error
    // budget); fp32 inputs keep every operation in fp32 on the vector ALUs.
    if (d == 128) {
        return in_dtype == 1 ? launch_prefill_mfma(a, in_dtype, stream)
                             : launch_prefill_t<float, 128>(a, in_dtype, stream);
    }
    if (d == 64) {   // the dense products stay on the vector ALUs at this head size
        return in_dtype == 1 ? launch_prefill_t<bf16_t, 64>(a, in_dtype, stream)
                             : launch_prefill_t<float, 64>(a, in_dtype, stream);
    }
    return in_dtype == 1 ? launch_prefill_t<bf16_t, 16>(a, in_dtype, stream)
                         : launch_prefill_t<float, 16>(a, in_dtype, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, int in_dtype, int d, hipStream_t stream) {
    if (a.chunk != 64) return hipErrorInvalidValue;
    hipError_t e = launch_prefill_core(a, in_dtype, d, stream);
    // the MFMA path (bf16, d = 128) applies the gated RMSNorm in its carry's output store
    const bool norm_fused = d == 128 && in_dtype == 1;
    if (e == hipSuccess && a.fu.z != nullptr && !norm_fused) e = launch_prefill_epilogue(a, in_dtype, d, stream);
    return e;
}

}  // namespace gdn
