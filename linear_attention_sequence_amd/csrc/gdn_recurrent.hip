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
//
// Verify blocks at dk = dv = 128 (without the RMSNorm epilogue) run a narrow layout
// on 1024 threads: thread (rg, cg) = (wave, lane) holds 2 columns of the same rows
// rg + 16 r (r < 8), so each column's partial sums are the same FMA chains as in the
// 512-thread layout, and the row groups 2w and 2w + 1 (one wave each here, two halves
// of one wave there) are added before the waves' sums, in the same order: a verify
// block still equals its decode steps bit for bit.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

#include <type_traits>

namespace gdn {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Tile geometry: NT threads own a DK x CW slice (columns j0..j0+CW) of one
// (sequence, V head) state tile.
template <int DK, int DV, int NT, int CW>
struct RecGeom {
    static_assert(CW % 4 == 0 && DV % CW == 0, "column split must divide dv");
    static constexpr int NSPLIT = DV / CW;
    static constexpr int CG = CW / 4;
    static constexpr int RG = NT / CG;
    static constexpr int RPT = DK / RG;
    static constexpr int NW = NT / kWave;
    static constexpr int NCH = 2 * DK + CW;
    static_assert(NT % CG == 0 && DK % RG == 0, "tile does not divide the workgroup");
    static_assert(kWave % CG == 0, "a column group set must fit in one wave");
};

struct RecLds {
    float *sq, *sk, *sv, *s_alpha, *s_beta, *s_kq, *red, *s_gz;
};

template <int DK, int CW, int NW>
__device__ __forceinline__ RecLds rec_lds(float* lds, int T) {
    RecLds L;
    L.sq = lds;                          // [T][DK] q (raw: the norms scale the reduced products)
    L.sk = L.sq + T * DK;                // [T][DK] k (raw)
    L.sv = L.sk + T * DK;                // [T][CW] v (this workgroup's columns)
    L.s_alpha = L.sv + T * CW;           // [T] exp(gate)
    L.s_beta = L.s_alpha + T;            // [T]
    L.s_kq = L.s_beta + T;               // [T][3] per token: 1/|k|, the q scale, k_hat . q_hat
    // the partial sums and the gated RMSNorm factors are read as float4: 16-byte boundaries
    L.red = lds + ((static_cast<int>(L.s_kq - lds) + 3 * T + 3) & ~3);   // [2][NW][CG][8] partial S^T k, S^T q
    L.s_gz = L.red + 2 * NW * (CW / 4) * 8;                              // [T][CW] norm_weight * silu(z)
    return L;
}

template <int DK, int CW, int NT, bool EPI>
size_t recurrent_lds_bytes(int T) {
    constexpr int CG = CW / 4;
    constexpr int NW = NT / kWave;
    return sizeof(float) * (static_cast<size_t>(T) * (2 * DK + CW) + 5 * T + 3 + 2 * NW * CG * 8 +
                            (EPI ? static_cast<size_t>(T) * CW : 0));
}

// Which (sequence, V head, column slice) a unit index names.
struct Unit {
    int bh, b, h, hk, j0;
    bool qk_owner;   // writes the q/k conv-state channels (one of the GQA group, slice 0)
};

template <int NSPLIT, int CW>
__device__ __forceinline__ Unit unit_of(const RecArgs& a, int unit) {
    Unit u;
    u.bh = unit / NSPLIT;
    const int split = unit - u.bh * NSPLIT;
    u.j0 = split * CW;
    u.b = u.bh / a.Hv;
    u.h = u.bh - u.b * a.Hv;
    const int f = a.Hv / a.Hk;
    u.hk = u.h / f;                      // reverse GQA: repeat_interleave
    u.qk_owner = (u.h % f) == 0 && split == 0;
    return u;
}

// Conv channel c (0 <= c < 2*DK + CW) of a unit: global channel, LDS row and
// stride, and whether this unit writes its conv-state window.
template <int DK, int DV, int CW>
__device__ __forceinline__ void fe_channel(const RecArgs& a, const Unit& u, const RecLds& L, int c, int* ch,
                                           float** dst, int* stride, bool* owner) {
    if (c < DK) {                        // q channels of K head hk
        *ch = u.hk * DK + c; *dst = L.sq + c; *owner = u.qk_owner; *stride = DK;
    } else if (c < 2 * DK) {             // k channels of K head hk
        *ch = a.Hk * DK + u.hk * DK + (c - DK); *dst = L.sk + (c - DK); *owner = u.qk_owner; *stride = DK;
    } else {                             // v channels j0.. of V head h
        *ch = 2 * a.Hk * DK + u.h * DV + u.j0 + (c - 2 * DK); *dst = L.sv + (c - 2 * DK); *owner = true; *stride = CW;
    }
}

template <int DK, int DV, int NT, int CW, bool NT_LOAD>
__device__ __forceinline__ void load_tile(const RecArgs& a, const Unit& u, float4 (&s)[RecGeom<DK, DV, NT, CW>::RPT]) {
    using G = RecGeom<DK, DV, NT, CW>;
    const int cg = threadIdx.x % G::CG, rg = threadIdx.x / G::CG;
    size_t src = u.bh;                   // (sequence, head) tile of S_in
    if (a.slot != nullptr) {             // snapshot slot[b] of a previous verify block
        int k = a.slot[u.b];
        k = k < 0 ? 0 : (k > a.slot_T - 1 ? a.slot_T - 1 : k);
        src = (static_cast<size_t>(u.b) * a.slot_T + k) * a.Hv + u.h;
    }
    const float* Sin = a.S_in + src * DK * DV + u.j0;
#pragma unroll
    for (int r = 0; r < G::RPT; ++r) {
        const float* src = Sin + static_cast<size_t>(rg + r * G::RG) * DV + 4 * cg;
        if constexpr (NT_LOAD) {
            const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
            s[r] = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            s[r] = *reinterpret_cast<const float4*>(src);
        }
    }
}

// Steps 3-5 once the conv outputs of every token sit in LDS: L2 norms, the q
// scale and k.q (one wave per token), then the recurrence token by token on the
// register tile, writing the state after each token and the outputs.
template <typename Tin, int DK, int DV, int NT, int CW, bool NT_STORE, bool PRO, bool EPI>
__device__ __forceinline__ void recur_tail(const RecArgs& a, const Unit& u, const RecLds& L, int T,
                                           float4 (&s)[RecGeom<DK, DV, NT, CW>::RPT]) {
    using G = RecGeom<DK, DV, NT, CW>;
    constexpr int CG = G::CG, RG = G::RG, RPT = G::RPT, NW = G::NW;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const float qscale = 1.0f / sqrtf(static_cast<float>(DK));
    // Norms of every token (wave t % NW takes token t). q and k stay raw in LDS: the scales
    // are applied to the reduced dot products (S^T k_hat = rk S^T k, S^T q_hat = qs S^T q)
    // and to delta (k_hat delta^T = k (rk delta)^T), so this pass needs no barrier of its
    // own and overlaps the other waves' dot products; its results are read after the first
    // token's reduction barrier.
    for (int t = wave; t < T; t += NW) {
        float qq = 0.f, kk = 0.f, kq = 0.f;
        for (int i = lane; i < DK; i += kWave) {
            const float qv = L.sq[t * DK + i], kv = L.sk[t * DK + i];
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
        if (lane == 0) {
            L.s_kq[3 * t] = rk;
            L.s_kq[3 * t + 1] = qs;
            L.s_kq[3 * t + 2] = kq * rk * qs;
        }
    }

    for (int t = 0; t < T; ++t) {
        float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + r * RG;
            const float kv = L.sk[t * DK + i], qv = L.sq[t * DK + i];
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
        // One barrier per token: after it every thread forms delta for its own four columns
        // from the reduced partials. A wave may then write token t + 1's partials while others
        // still read token t's, hence two buffers (token t + 2 reuses the first only after
        // token t + 1's barrier).
        float* red = L.red + (t & 1) * (NW * CG * 8);
        if (lane < CG) {
            float* rp = red + (wave * CG + lane) * 8;
#pragma unroll
            for (int c = 0; c < 4; ++c) { rp[c] = pk[c]; rp[4 + c] = pq[c]; }
        }
        __syncthreads();
        const float al = L.s_alpha[t], be = L.s_beta[t];
        const float rk = L.s_kq[3 * t], qs = L.s_kq[3 * t + 1], kqh = L.s_kq[3 * t + 2];
        float4 PK = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            const float4 v = *reinterpret_cast<const float4*>(red + (wv * CG + cg) * 8);
            PK.x += v.x; PK.y += v.y; PK.z += v.z; PK.w += v.w;
        }
        const float4 vv = *reinterpret_cast<const float4*>(L.sv + t * CW + 4 * cg);
        const float4 d = make_float4(be * (vv.x - al * (PK.x * rk)), be * (vv.y - al * (PK.y * rk)),
                                     be * (vv.z - al * (PK.z * rk)), be * (vv.w - al * (PK.w * rk)));
        const float4 dl = make_float4(d.x * rk, d.y * rk, d.z * rk, d.w * rk);
        float* Sout = a.S_out + ((static_cast<size_t>(u.b) * T + t) * a.Hv + u.h) * DK * DV + u.j0;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float kv = L.sk[t * DK + rg + r * RG];
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
        // The output row, after the state tile's stores are issued (this order measured
        // 1 us faster per decode step): row group 0, CG lanes of wave 0 with four columns
        // each, so the gated RMSNorm reduces its row within the wave.
        if (wave == 0) {
            float4 ov = make_float4(0.f, 0.f, 0.f, 0.f);
            if (rg == 0) {
                float4 PQ = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int wv = 0; wv < NW; ++wv) {
                    const float4 v = *reinterpret_cast<const float4*>(red + (wv * CG + cg) * 8 + 4);
                    PQ.x += v.x; PQ.y += v.y; PQ.z += v.z; PQ.w += v.w;
                }
                ov = make_float4(__fmaf_rn(d.x, kqh, al * (PQ.x * qs)), __fmaf_rn(d.y, kqh, al * (PQ.y * qs)),
                                 __fmaf_rn(d.z, kqh, al * (PQ.z * qs)), __fmaf_rn(d.w, kqh, al * (PQ.w * qs)));
            }
            if constexpr (EPI) {   // the other lanes of the wave add zeros
                const float ss = wave_sum_uniform(ov.x * ov.x + ov.y * ov.y + ov.z * ov.z + ov.w * ov.w);
                const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + a.fu.norm_eps);
                if (rg == 0) {
                    const float4 gz = *reinterpret_cast<const float4*>(L.s_gz + t * CW + 4 * cg);
                    ov = make_float4((ov.x * inv) * gz.x, (ov.y * inv) * gz.y, (ov.z * inv) * gz.z, (ov.w * inv) * gz.w);
                }
            }
            const size_t orow = ((static_cast<size_t>(u.b) * T + t) * a.Hv + u.h) * DV + u.j0;
            if (rg == 0) *reinterpret_cast<float4*>(a.o + orow + 4 * cg) = ov;
        }
    }
}

// The narrow layout (see the top of the file): DK x CW tile on NT threads of 2 columns.
template <int DK, int CW, int NT>
struct NarrowGeom {
    static constexpr int CG = CW / 2;         // column pairs: one wave's lanes
    static constexpr int RG = NT / CG;        // row groups: one per wave
    static constexpr int RPT = DK / RG;
    static constexpr int NW = NT / kWave;
    static_assert(CG == kWave && RG == NW && RG % 2 == 0, "one row group per wave, pairs of waves");
};

template <int DK, int DV, int NT, int CW, bool NT_LOAD>
__device__ __forceinline__ void load_tile_narrow(const RecArgs& a, const Unit& u, float2 (&s)[NarrowGeom<DK, CW, NT>::RPT]) {
    using G = NarrowGeom<DK, CW, NT>;
    const int cg = threadIdx.x % G::CG, rg = threadIdx.x / G::CG;
    size_t src = u.bh;
    if (a.slot != nullptr) {
        int k = a.slot[u.b];
        k = k < 0 ? 0 : (k > a.slot_T - 1 ? a.slot_T - 1 : k);
        src = (static_cast<size_t>(u.b) * a.slot_T + k) * a.Hv + u.h;
    }
    const float* Sin = a.S_in + src * DK * DV + u.j0;
#pragma unroll
    for (int r = 0; r < G::RPT; ++r) {
        const float* p = Sin + static_cast<size_t>(rg + r * G::RG) * DV + 2 * cg;
        if constexpr (NT_LOAD) {
            const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
            s[r] = make_float2(v[0], v[1]);
        } else {
            s[r] = *reinterpret_cast<const float2*>(p);
        }
    }
}

// recur_tail on the narrow layout. With the epilogue, each row's sum of squares is
// formed in the 512-thread layout's pattern (lane j < 32 holds columns 4j .. 4j + 3 as
// ((x^2 + y^2) + z^2) + w^2, the other lanes zero) before the same wave sum.
template <typename Tin, int DK, int DV, int NT, int CW, bool NT_STORE, bool EPI>
__device__ __forceinline__ void recur_tail_narrow(const RecArgs& a, const Unit& u, const RecLds& L, int T,
                                                  float2 (&s)[NarrowGeom<DK, CW, NT>::RPT]) {
    using G = NarrowGeom<DK, CW, NT>;
    constexpr int CG = G::CG, RG = G::RG, RPT = G::RPT, NW = G::NW;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const float qscale = 1.0f / sqrtf(static_cast<float>(DK));
    for (int t = wave; t < T; t += NW) {   // norms, as in recur_tail
        float qq = 0.f, kk = 0.f, kq = 0.f;
        for (int i = lane; i < DK; i += kWave) {
            const float qv = L.sq[t * DK + i], kv = L.sk[t * DK + i];
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
        if (lane == 0) {
            L.s_kq[3 * t] = rk;
            L.s_kq[3 * t + 1] = qs;
            L.s_kq[3 * t + 2] = kq * rk * qs;
        }
    }
    for (int t = 0; t < T; ++t) {
        float pk[2] = {0.f, 0.f}, pq[2] = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + r * RG;
            const float kv = L.sk[t * DK + i], qv = L.sq[t * DK + i];
            pk[0] = __fmaf_rn(s[r].x, kv, pk[0]); pq[0] = __fmaf_rn(s[r].x, qv, pq[0]);
            pk[1] = __fmaf_rn(s[r].y, kv, pk[1]); pq[1] = __fmaf_rn(s[r].y, qv, pq[1]);
        }
        // one row group per wave: its partials go to LDS as they are, S^T k and S^T q in
        // separate planes (double-buffered by token)
        float* redk = L.red + (t & 1) * (NW * CG * 4);
        float* redq = redk + NW * CG * 2;
        *reinterpret_cast<float2*>(redk + (wave * CG + cg) * 2) = make_float2(pk[0], pk[1]);
        *reinterpret_cast<float2*>(redq + (wave * CG + cg) * 2) = make_float2(pq[0], pq[1]);
        __syncthreads();
        const float al = L.s_alpha[t], be = L.s_beta[t];
        const float rk = L.s_kq[3 * t], qs = L.s_kq[3 * t + 1], kqh = L.s_kq[3 * t + 2];
        // row groups 2w and 2w + 1 added first, then those sums in order of w
        auto total = [&](const float* plane) {
            float2 v = make_float2(0.f, 0.f);
#pragma unroll
            for (int w = 0; w < NW; w += 2) {
                const float2 v0 = *reinterpret_cast<const float2*>(plane + (w * CG + cg) * 2);
                const float2 v1 = *reinterpret_cast<const float2*>(plane + ((w + 1) * CG + cg) * 2);
                v.x += v0.x + v1.x;
                v.y += v0.y + v1.y;
            }
            return v;
        };
        const float2 PK = total(redk);   // S^T k of this lane's two columns
        const float2 vv = *reinterpret_cast<const float2*>(L.sv + t * CW + 2 * cg);
        const float2 d = make_float2(be * (vv.x - al * (PK.x * rk)), be * (vv.y - al * (PK.y * rk)));
        const float2 dl = make_float2(d.x * rk, d.y * rk);
        float* Sout = a.S_out + ((static_cast<size_t>(u.b) * T + t) * a.Hv + u.h) * DK * DV + u.j0;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float kv = L.sk[t * DK + rg + r * RG];
            s[r].x = __fmaf_rn(kv, dl.x, al * s[r].x);
            s[r].y = __fmaf_rn(kv, dl.y, al * s[r].y);
            float* dst = Sout + static_cast<size_t>(rg + r * RG) * DV + 2 * cg;
            if constexpr (NT_STORE) {
                const f32x2 v = {s[r].x, s[r].y};
                __builtin_nontemporal_store(v, reinterpret_cast<f32x2*>(dst));
            } else {
                *reinterpret_cast<float2*>(dst) = s[r];
            }
        }
        if (wave == 0) {   // the output row: row group 0 is wave 0, two columns per lane
            const float2 PQ = total(redq);
            float2 ov = make_float2(__fmaf_rn(d.x, kqh, al * (PQ.x * qs)), __fmaf_rn(d.y, kqh, al * (PQ.y * qs)));
            if constexpr (EPI) {
                const float z0 = __shfl_down(ov.x, 1, kWave), z1 = __shfl_down(ov.y, 1, kWave);   // the odd lane's columns
                const float sq = ((ov.x * ov.x + ov.y * ov.y) + z0 * z0) + z1 * z1;                 // valid in even lanes
                const float sj = __shfl(sq, 2 * (lane & 31), kWave);
                const float ss = wave_sum_uniform(lane < 32 ? sj : 0.f);
                const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + a.fu.norm_eps);
                const float2 gz = *reinterpret_cast<const float2*>(L.s_gz + t * CW + 2 * cg);
                ov = make_float2((ov.x * inv) * gz.x, (ov.y * inv) * gz.y);
            }
            const size_t orow = ((static_cast<size_t>(u.b) * T + t) * a.Hv + u.h) * DV + u.j0;
            *reinterpret_cast<float2*>(a.o + orow + 2 * cg) = ov;
        }
    }
}

struct NoGeom { static constexpr int RPT = 1; };

// Any T (verify blocks, and decode at head dim 16): one unit per workgroup. NARROW: the
// narrow layout (verify blocks at dk = dv = 128, no epilogue).
template <typename Tin, int DK, int DV, int NT, int CW, bool NT_STORE, bool NT_LOAD, bool PRO, bool EPI,
          bool NARROW = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NARROW ? 8 : 1)))
void recurrent_kernel(RecArgs a) {   // narrow: 64 registers, two workgroups per CU
    using G = RecGeom<DK, DV, NT, CW>;
    using NG = std::conditional_t<NARROW, NarrowGeom<DK, CW, NT>, NoGeom>;
    static_assert(!NARROW || (DK == 128 && CW == DV), "the narrow layout: dk = dv = 128");
    extern __shared__ float lds[];
    const int T = a.T;
    const RecLds L = rec_lds<DK, CW, G::NW>(lds, T);
    const Unit u = unit_of<G::NSPLIT, CW>(a, blockIdx.x);

    // 1. state tile -> registers, issued first
    float4 s[NARROW ? 1 : G::RPT];
    float2 s2[NG::RPT];
    if constexpr (NARROW) load_tile_narrow<DK, DV, NT, CW, NT_LOAD>(a, u, s2);
    else load_tile<DK, DV, NT, CW, NT_LOAD>(a, u, s);

    // gate and beta of token t = threadIdx.x, issued right behind the tile: their round trip
    // then overlaps the tile's instead of following the conv barrier, where it held up the
    // whole workgroup (the prologue's per-head A_log and dt_bias likewise)
    const int tg = threadIdx.x;
    float g_in = 0.f, b_in = 0.f, alog_in = 0.f, dtb_in = 0.f;
    if (tg < T) {
        const size_t gi = (static_cast<size_t>(u.b) * T + tg) * a.Hv + u.h;
        g_in = to_f32(static_cast<const Tin*>(a.gate)[gi]);
        b_in = to_f32(static_cast<const Tin*>(a.beta)[gi]);
        if constexpr (PRO) {
            alog_in = to_f32(static_cast<const Tin*>(a.fu.A_log)[u.h]);
            dtb_in = to_f32(static_cast<const Tin*>(a.fu.dt_bias)[u.h]);
        }
    }

    // 2. conv + SiLU of this unit's channels for every token of the block
    const Tin* x = static_cast<const Tin*>(a.qkv);
    const Tin* w = static_cast<const Tin*>(a.w);
    const Tin* cin = static_cast<const Tin*>(a.conv_in);
    Tin* cout = static_cast<Tin*>(a.conv_out);
    for (int c = threadIdx.x; c < G::NCH; c += NT) {
        int ch, stride;
        float* dst;
        bool owner;
        fe_channel<DK, DV, CW>(a, u, L, c, &ch, &dst, &stride, &owner);
        float wv[kConvK];
#pragma unroll
        for (int j = 0; j < kConvK; ++j) wv[j] = to_f32(w[static_cast<size_t>(ch) * kConvK + j]);
        const Tin* st = cin + (static_cast<size_t>(u.b) * a.D + ch) * (kConvK - 1);
        const Tin* xc = x + (static_cast<size_t>(u.b) * a.D + ch) * T;
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
            Tin* co = cout + (static_cast<size_t>(u.b) * a.D + ch) * (kConvK - 1);
#pragma unroll
            for (int j = 0; j < kConvK - 1; ++j) {
                const int pos = T + j;  // position in the concatenated window
                co[j] = (pos < kConvK - 1) ? st[pos] : xc[pos - (kConvK - 1)];
            }
        }
    }
    if constexpr (EPI) {
        // gated RMSNorm factors of every token: norm_weight[j] * silu(z[j])
        const Tin* z = static_cast<const Tin*>(a.fu.z);
        const Tin* nw = static_cast<const Tin*>(a.fu.norm_w);
        for (int i = threadIdx.x; i < T * CW; i += NT) {
            const int t = i / CW, j = i % CW;
            const float zv = to_f32(z[((static_cast<size_t>(u.b) * T + t) * a.Hv + u.h) * DV + u.j0 + j]);
            L.s_gz[i] = to_f32(nw[u.j0 + j]) * (zv * sigmoid_hw(zv));
        }
    }
    if (tg < T) {
        float gv = g_in, bv = b_in;
        if constexpr (PRO) gate_beta_of(g_in, b_in, alog_in, dtb_in, &gv, &bv);
        L.s_alpha[tg] = expf(gv);
        L.s_beta[tg] = bv;
    }
    __syncthreads();
    if constexpr (NARROW) recur_tail_narrow<Tin, DK, DV, NT, CW, NT_STORE, EPI>(a, u, L, T, s2);
    else recur_tail<Tin, DK, DV, NT, CW, NT_STORE, PRO, EPI>(a, u, L, T, s);
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
    if (a.S_out != nullptr) {   // in passes of four loads, then their four (non-temporal) stores
        const f32x4* src = reinterpret_cast<const f32x4*>(
            a.S_snap + ((static_cast<size_t>(b) * a.T + acc) * a.Hv + h) * DK * DV);
        f32x4* dst = reinterpret_cast<f32x4*>(a.S_out + static_cast<size_t>(bh) * DK * DV);
        constexpr int NV = DK * DV / 4;
        constexpr int PER = NV >= 256 ? NV / 256 : 1;
        static_assert(NV < 256 || NV % 256 == 0, "tile must split evenly over the workgroup");
        // (all 16 loads of a thread before any store: 2% slower on the 128 x 32 tiles of
        // 64 KB, whose copy then holds 64 registers; passes of 2 or 8 lie in between)
        constexpr int Q = PER < 4 ? PER : 4;
#pragma unroll
        for (int i0 = 0; i0 < PER; i0 += Q) {
            f32x4 r[Q];
#pragma unroll
            for (int i = 0; i < Q; ++i) {
                const int e = threadIdx.x + 256 * (i0 + i);
                if (e < NV) r[i] = src[e];
            }
#pragma unroll
            for (int i = 0; i < Q; ++i) {
                const int e = threadIdx.x + 256 * (i0 + i);
                if (e < NV) __builtin_nontemporal_store(r[i], dst + e);
            }
        }
    }

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

template <typename Tin, int DK, int DV, int NT, int CW, bool NT_STORE, bool NT_LOAD, bool PRO, bool EPI,
          bool NARROW = false>
hipError_t launch_rec_t(const RecArgs& a, hipStream_t stream) {
    // the fused gated RMSNorm needs the whole dv row of a head in one workgroup
    static_assert(CW == DV, "column slices would split the RMSNorm row");
    const size_t lds = recurrent_lds_bytes<DK, CW, NT, EPI>(a.T);
    const void* k = reinterpret_cast<const void*>(&recurrent_kernel<Tin, DK, DV, NT, CW, NT_STORE, NT_LOAD, PRO, EPI, NARROW>);
    // dynamic LDS above 64 KB (1024 threads with the epilogue at T = 16: 66 KB) must be
    // allowed per kernel before its first launch; the largest block (T = 16) sets the bound
    constexpr int kMaxBlock = 16;
    static const hipError_t allowed =
        hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(recurrent_lds_bytes<DK, CW, NT, EPI>(kMaxBlock)));
    if (allowed != hipSuccess) return allowed;
    void* args[] = {const_cast<RecArgs*>(&a)};
    return hipLaunchKernel(k, dim3(a.B * a.Hv * (DV / CW)), dim3(NT), args, lds, stream);
}

// Verify blocks at d = 128 on the narrow layout, with or without either fusion.
template <typename Tin>
hipError_t launch_rec_narrow(const RecArgs& a, hipStream_t stream) {
    const bool pro = a.fu.A_log != nullptr, epi = a.fu.z != nullptr;
    if (pro)
        return epi ? launch_rec_t<Tin, 128, 128, 1024, 128, true, false, true, true, true>(a, stream)
                   : launch_rec_t<Tin, 128, 128, 1024, 128, true, false, true, false, true>(a, stream);
    return epi ? launch_rec_t<Tin, 128, 128, 1024, 128, true, false, false, true, true>(a, stream)
               : launch_rec_t<Tin, 128, 128, 1024, 128, true, false, false, false, true>(a, stream);
}

// The fusions are compile-time variants, so the plain kernel carries none of
// their registers (its occupancy decides how many state bytes are in flight).
template <typename Tin, int DK, int DV, int NT, int CW, bool NT_STORE, bool NT_LOAD>
hipError_t launch_rec(const RecArgs& a, hipStream_t stream) {
    const bool pro = a.fu.A_log != nullptr, epi = a.fu.z != nullptr;
    if (pro) {
        return epi ? launch_rec_t<Tin, DK, DV, NT, CW, NT_STORE, NT_LOAD, true, true>(a, stream)
                   : launch_rec_t<Tin, DK, DV, NT, CW, NT_STORE, NT_LOAD, true, false>(a, stream);
    }
    return epi ? launch_rec_t<Tin, DK, DV, NT, CW, NT_STORE, NT_LOAD, false, true>(a, stream)
               : launch_rec_t<Tin, DK, DV, NT, CW, NT_STORE, NT_LOAD, false, false>(a, stream);
}

// d = 128: 512 threads (8 waves) hold the 128 x 128 tile as 8 float4 per thread.
// The state is streamed: it is written with non-temporal stores (each tile is
// read once and written once per call, so caching the writes only evicts useful
// lines); in a cold-cache sweep this took the decode step from 67.7 us to
// 50.8 us. (A persistent variant that prefetched the next tile measured the
// same: reads and writes are both already streaming near the box's mixed
// read/write limit.)
hipError_t launch_recurrent(const RecArgs& a, int in_dtype, int d, hipStream_t stream) {
    if (d == 128) {
        // verify blocks on the narrow 1024-thread layout (the same sums as the 512-thread
        // decode layout, half the columns per thread: B=128, T=4 247 -> 238 us), decode on 512
        // threads (a 1024-thread decode measured 62 us against 48.6)
        if (a.T > 1)
            return in_dtype == 1 ? launch_rec_narrow<bf16_t>(a, stream) : launch_rec_narrow<float>(a, stream);
        return in_dtype == 1 ? launch_rec<bf16_t, 128, 128, 512, 128, true, false>(a, stream)
                             : launch_rec<float, 128, 128, 512, 128, true, false>(a, stream);
    }
    if (d == 64) {   // 256 threads, 4 float4 of the 64 x 64 tile each
        return in_dtype == 1 ? launch_rec<bf16_t, 64, 64, 256, 64, true, false>(a, stream)
                             : launch_rec<float, 64, 64, 256, 64, true, false>(a, stream);
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
    if (d == 64) {
        return in_dtype == 1 ? launch_com<bf16_t, 64, 64>(a, stream)
                             : launch_com<float, 64, 64>(a, stream);
    }
    return in_dtype == 1 ? launch_com<bf16_t, 16, 16>(a, stream)
                         : launch_com<float, 16, 16>(a, stream);
}

}  // namespace gdn
