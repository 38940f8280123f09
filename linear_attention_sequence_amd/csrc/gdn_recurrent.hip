// Decode step, speculative verify block and commit for the Gated DeltaNet layer
// ("MNN Model Support: Qwen3.5", §1.2 steps 1-5, §1.3 reverse GQA, §1.4 states).
//
// One workgroup owns one (sequence b, V head h) pair for the whole call. It
//   1. issues the loads of its fp32 state tile S[b,h] (dk x dv) into registers
//      first, so the HBM stream starts before anything else;
//   2. computes, for every token of the block, the conv+SiLU of the 2*dk + dv
//      channels it needs (the q and k channels of K head h/(Hv/Hk), the v
//      channels of V head h) from the conv window, the per-head L2 norms, the
//      1/sqrt(dk) scale and k.q, all into LDS;
//   3. runs the recurrence token by token on the register-resident tile with a
//      single pass per token: both dot products S^T k and S^T q come from the
//      same registers, then
//         p = a * S^T k,  delta = beta (v - p),  o = a * S^T q + delta (k.q),
//         S' = a S + k delta^T,
//      which is S' = exp(g) S + k delta^T followed by o = S'^T q, rearranged so
//      that each element of S is read once and written once per token;
//   4. writes the state after every token (verify: snapshots; decode: in place).
// Decode is the same kernel with T = 1, so a verify snapshot equals the state
// after the same number of decode steps bit for bit.
//
// Thread layout for a dk x dv tile with NT threads: thread (rg, cg) holds the
// 4 consecutive columns 4*cg..4*cg+3 of rows rg, rg + RG, rg + 2*RG, ... as
// float4 registers (CG = dv/4 column groups, RG = NT/CG row groups), so each
// row is read by CG consecutive lanes with 16-byte loads (fully coalesced).
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <typename Tin, int DK, int DV, int NT, int CW, bool NT_STORE, bool NT_LOAD>
__global__ __launch_bounds__(NT) void recurrent_kernel(RecArgs a) {
    static_assert(CW % 4 == 0 && DV % CW == 0, "column split must divide dv");
    constexpr int NSPLIT = DV / CW;
    constexpr int CG = CW / 4;
    constexpr int RG = NT / CG;
    constexpr int RPT = DK / RG;
    constexpr int NW = NT / kWave;
    static_assert(NT % CG == 0 && DK % RG == 0, "tile does not divide the workgroup");
    static_assert(kWave % CG == 0, "a column group set must fit in one wave");
    constexpr int NCH = 2 * DK + CW;

    extern __shared__ float lds[];
    const int T = a.T;
    float* sq = lds;                       // [T][DK] q_hat
    float* sk = sq + T * DK;               // [T][DK] k_hat
    float* sv = sk + T * DK;               // [T][CW] v (this workgroup's columns)
    float* s_alpha = sv + T * CW;          // [T] exp(gate)
    float* s_beta = s_alpha + T;           // [T]
    float* s_kq = s_beta + T;              // [T] k_hat . q_hat
    float* red = s_kq + T;                 // [NW][CG][8] partial dot products
    float* s_delta = red + NW * CG * 8;    // [CW]

    const int bh = blockIdx.x / NSPLIT;
    const int split = blockIdx.x - bh * NSPLIT;
    const int j0 = split * CW;
    const int b = bh / a.Hv;
    const int h = bh - b * a.Hv;
    const int f = a.Hv / a.Hk;
    const int hk = h / f;                  // reverse GQA: repeat_interleave
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int lane = tid % kWave;
    const int wave = tid / kWave;

    // 1. state tile -> registers
    const float* Sin = a.S_in + static_cast<size_t>(bh) * DK * DV + j0;
    float4 s[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float* src = Sin + static_cast<size_t>(rg + r * RG) * DV + 4 * cg;
        if constexpr (NT_LOAD) {
            const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
            s[r] = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            s[r] = *reinterpret_cast<const float4*>(src);
        }
    }

    // 2. conv + SiLU of this unit's channels for every token of the block
    const Tin* x = static_cast<const Tin*>(a.qkv);
    const Tin* w = static_cast<const Tin*>(a.w);
    const Tin* cin = static_cast<const Tin*>(a.conv_in);
    Tin* cout = static_cast<Tin*>(a.conv_out);
    const bool qk_owner = (h % f) == 0 && split == 0;
    for (int c = tid; c < NCH; c += NT) {
        int ch, stride;
        float* dst;
        bool owner;
        if (c < DK) {                       // q channels of K head hk
            ch = hk * DK + c; dst = sq + c; owner = qk_owner; stride = DK;
        } else if (c < 2 * DK) {            // k channels of K head hk
            ch = a.Hk * DK + hk * DK + (c - DK); dst = sk + (c - DK); owner = qk_owner; stride = DK;
        } else {                            // v channels j0.. of V head h
            ch = 2 * a.Hk * DK + h * DV + j0 + (c - 2 * DK); dst = sv + (c - 2 * DK); owner = true; stride = CW;
        }
        float wv[kConvK];
#pragma unroll
        for (int j = 0; j < kConvK; ++j) wv[j] = to_f32(w[static_cast<size_t>(ch) * kConvK + j]);
        const Tin* st = cin + (static_cast<size_t>(b) * a.D + ch) * (kConvK - 1);
        const Tin* xc = x + (static_cast<size_t>(b) * a.D + ch) * T;
        float win[kConvK];
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j) win[j] = to_f32(st[j]);
        for (int t = 0; t < T; ++t) {
            win[kConvK - 1] = to_f32(xc[t]);
            dst[t * stride] = conv_silu(wv, win);
#pragma unroll
            for (int j = 0; j < kConvK - 1; ++j) win[j] = win[j + 1];
        }
        if (cout != nullptr && owner) {
            // new window: the K-1 most recent raw inputs of concat(state, x[0..T-1])
            Tin* co = cout + (static_cast<size_t>(b) * a.D + ch) * (kConvK - 1);
#pragma unroll
            for (int j = 0; j < kConvK - 1; ++j) {
                const int pos = T + j;  // position in the concatenated window
                co[j] = (pos < kConvK - 1) ? st[pos] : xc[pos - (kConvK - 1)];
            }
        }
    }
    __syncthreads();

    // 3. L2 norms, q scale and k.q, one wave per token
    const Tin* gate = static_cast<const Tin*>(a.gate);
    const Tin* beta = static_cast<const Tin*>(a.beta);
    const float qscale = 1.0f / sqrtf(static_cast<float>(DK));
    for (int t = wave; t < T; t += NW) {
        float qq = 0.f, kk = 0.f, kq = 0.f;
        for (int i = lane; i < DK; i += kWave) {
            const float qv = sq[t * DK + i], kv = sk[t * DK + i];
            qq = __fmaf_rn(qv, qv, qq);
            kk = __fmaf_rn(kv, kv, kk);
            kq = __fmaf_rn(kv, qv, kq);
        }
        qq = wave_sum(qq);
        kk = wave_sum(kk);
        kq = wave_sum(kq);
        const float rq = a.use_l2 ? 1.0f / sqrtf(qq + a.eps) : 1.0f;
        const float rk = a.use_l2 ? 1.0f / sqrtf(kk + a.eps) : 1.0f;
        const float qs = rq * qscale;
        for (int i = lane; i < DK; i += kWave) {
            sq[t * DK + i] *= qs;
            sk[t * DK + i] *= rk;
        }
        if (lane == 0) {
            const size_t gi = (static_cast<size_t>(b) * T + t) * a.Hv + h;
            s_alpha[t] = expf(to_f32(gate[gi]));
            s_beta[t] = to_f32(beta[gi]);
            s_kq[t] = kq * rk * qs;
        }
    }
    __syncthreads();

    // 4. the recurrence, token by token
    for (int t = 0; t < T; ++t) {
        float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + r * RG;
            const float kv = sk[t * DK + i], qv = sq[t * DK + i];
            pk[0] = __fmaf_rn(s[r].x, kv, pk[0]); pq[0] = __fmaf_rn(s[r].x, qv, pq[0]);
            pk[1] = __fmaf_rn(s[r].y, kv, pk[1]); pq[1] = __fmaf_rn(s[r].y, qv, pq[1]);
            pk[2] = __fmaf_rn(s[r].z, kv, pk[2]); pq[2] = __fmaf_rn(s[r].z, qv, pq[2]);
            pk[3] = __fmaf_rn(s[r].w, kv, pk[3]); pq[3] = __fmaf_rn(s[r].w, qv, pq[3]);
        }
        // sum over the row groups held by this wave (lanes that share cg)
#pragma unroll
        for (int m = CG; m < kWave; m <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pk[c] += __shfl_xor(pk[c], m, kWave);
                pq[c] += __shfl_xor(pq[c], m, kWave);
            }
        }
        if (lane < CG) {
            float* rp = red + (wave * CG + lane) * 8;
#pragma unroll
            for (int c = 0; c < 4; ++c) { rp[c] = pk[c]; rp[4 + c] = pq[c]; }
        }
        __syncthreads();
        const float al = s_alpha[t], be = s_beta[t];
        if (tid < CW) {
            const int j = tid, jg = j / 4, jc = j % 4;
            float PK = 0.f, PQ = 0.f;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                PK += red[(wv * CG + jg) * 8 + jc];
                PQ += red[(wv * CG + jg) * 8 + 4 + jc];
            }
            const float p = al * PK;
            const float d = be * (sv[t * CW + j] - p);
            s_delta[j] = d;
            a.o[((static_cast<size_t>(b) * T + t) * a.Hv + h) * DV + j0 + j] = __fmaf_rn(d, s_kq[t], al * PQ);
        }
        __syncthreads();
        const float4 dl = *reinterpret_cast<const float4*>(s_delta + 4 * cg);
        float* Sout = a.S_out + ((static_cast<size_t>(b) * T + t) * a.Hv + h) * DK * DV + j0;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float kv = sk[t * DK + rg + r * RG];
            s[r].x = __fmaf_rn(kv, dl.x, al * s[r].x);
            s[r].y = __fmaf_rn(kv, dl.y, al * s[r].y);
            s[r].z = __fmaf_rn(kv, dl.z, al * s[r].z);
            s[r].w = __fmaf_rn(kv, dl.w, al * s[r].w);
            float* dst = Sout + static_cast<size_t>(rg + r * RG) * DV + 4 * cg;
            if constexpr (NT_STORE) {
                const f32x4 v = {s[r].x, s[r].y, s[r].z, s[r].w};
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
            } else {
                *reinterpret_cast<float4*>(dst) = s[r];
            }
        }
    }
}

template <int DK, int CW, int NT>
size_t recurrent_lds_bytes(int T) {
    constexpr int CG = CW / 4;
    constexpr int NW = NT / kWave;
    return sizeof(float) * (static_cast<size_t>(T) * (2 * DK + CW) + 3 * T + NW * CG * 8 + CW);
}

// Commit: S_out[b,h] = S_snap[b, a_b, h]; the conv window after token a_b.
// One workgroup per (b, h); the conv channels are split evenly over the Hv
// workgroups of a row.
template <typename Tin, int DK, int DV>
__global__ __launch_bounds__(256) void commit_kernel(CommitArgs a) {
    const int bh = blockIdx.x;
    const int b = bh / a.Hv;
    const int h = bh - b * a.Hv;
    int acc = a.accept[b];
    acc = acc < 0 ? 0 : (acc > a.T - 1 ? a.T - 1 : acc);
    const float4* src = reinterpret_cast<const float4*>(
        a.S_snap + ((static_cast<size_t>(b) * a.T + acc) * a.Hv + h) * DK * DV);
    float4* dst = reinterpret_cast<float4*>(a.S_out + static_cast<size_t>(bh) * DK * DV);
    for (int e = threadIdx.x; e < DK * DV / 4; e += 256) dst[e] = src[e];

    const Tin* x = static_cast<const Tin*>(a.qkv);
    const Tin* cin = static_cast<const Tin*>(a.conv_in);
    Tin* cout = static_cast<Tin*>(a.conv_out);
    const int per = (a.D + a.Hv - 1) / a.Hv;
    const int c0 = h * per;
    const int c1 = min(a.D, c0 + per);
    for (int ch = c0 + threadIdx.x; ch < c1; ch += 256) {
        const Tin* st = cin + (static_cast<size_t>(b) * a.D + ch) * (kConvK - 1);
        const Tin* xc = x + (static_cast<size_t>(b) * a.D + ch) * a.T;
        Tin* co = cout + (static_cast<size_t>(b) * a.D + ch) * (kConvK - 1);
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j) {
            const int pos = acc + 1 + j;
            co[j] = (pos < kConvK - 1) ? st[pos] : xc[pos - (kConvK - 1)];
        }
    }
}

template <typename Tin, int DK, int DV, int NT, int CW, bool NT_STORE, bool NT_LOAD>
hipError_t launch_rec(const RecArgs& a, hipStream_t stream) {
    const size_t lds = recurrent_lds_bytes<DK, CW, NT>(a.T);
    void* args[] = {const_cast<RecArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&recurrent_kernel<Tin, DK, DV, NT, CW, NT_STORE, NT_LOAD>),
                           dim3(a.B * a.Hv * (DV / CW)), dim3(NT), args, lds, stream);
}

// d = 128: 512 threads (8 waves) hold the 128 x 128 tile as 8 float4 per thread,
// so 4 workgroups fit a CU and the 2048 workgroups of a B = 64, Hv = 32 decode
// run in two full rounds. The state is streamed: it is written with
// non-temporal stores (each tile is read once and written once per call, so
// caching the writes only evicts useful lines); in a cold-cache sweep this
// took the decode step from 67.7 us to 50.8 us.
hipError_t launch_recurrent(const RecArgs& a, int in_dtype, int d, hipStream_t stream) {
    if (d == 128) {
        return in_dtype == 1 ? launch_rec<bf16_t, 128, 128, 512, 128, true, false>(a, stream)
                             : launch_rec<float, 128, 128, 512, 128, true, false>(a, stream);
    }
    return in_dtype == 1 ? launch_rec<bf16_t, 16, 16, 64, 16, true, false>(a, stream)
                         : launch_rec<float, 16, 16, 64, 16, true, false>(a, stream);
}

template <typename Tin, int DK, int DV>
static hipError_t launch_com(const CommitArgs& a, hipStream_t stream) {
    void* args[] = {const_cast<CommitArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&commit_kernel<Tin, DK, DV>),
                           dim3(a.B * a.Hv), dim3(256), args, 0, stream);
}

hipError_t launch_commit(const CommitArgs& a, int in_dtype, int d, hipStream_t stream) {
    if (d == 128) {
        return in_dtype == 1 ? launch_com<bf16_t, 128, 128>(a, stream)
                             : launch_com<float, 128, 128>(a, stream);
    }
    return in_dtype == 1 ? launch_com<bf16_t, 16, 16>(a, stream)
                         : launch_com<float, 16, 16>(a, stream);
}

}  // namespace gdn
