// C-ABI entry points of libgdn.so: synchronous argument validation, then one or
// more kernel launches on the caller's stream. See include/gdn.h for the
// contract of each call.
#include "gdn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <hip/hip_runtime.h>

#include "gdn_launch.hpp"

namespace {

constexpr int kK = 4;
constexpr int kMaxT = 16;
constexpr long long kMaxGrid = 0x7fffffffLL;

struct Buf {
    const void* p;
    size_t bytes;
    bool out;
};

bool overlaps(const Buf& a, const Buf& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output must be disjoint from every other buffer of the call.
template <size_t N>
gdn_status check_alias(const Buf (&bufs)[N]) {
    for (size_t i = 0; i < N; ++i)
        for (size_t j = i + 1; j < N; ++j)
            if ((bufs[i].out || bufs[j].out) && overlaps(bufs[i], bufs[j])) return GDN_ERR_ALIAS;
    return GDN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gdn_status check_params(const gdn_params* p) {
    if (p == nullptr) return GDN_ERR_NULL;
    if (p->in_dtype != GDN_F32 && p->in_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (p->num_k_heads <= 0 || p->num_v_heads <= 0 || p->head_k_dim <= 0 || p->head_v_dim <= 0 ||
        p->conv_kernel <= 0)
        return GDN_ERR_SHAPE;
    if (p->num_v_heads % p->num_k_heads != 0) return GDN_ERR_SHAPE;
    if (p->use_qk_l2norm != 0 && p->use_qk_l2norm != 1) return GDN_ERR_SHAPE;
    if (!std::isfinite(p->l2norm_eps) || p->l2norm_eps < 0.f) return GDN_ERR_SHAPE;
    if (p->head_k_dim != p->head_v_dim ||
        (p->head_k_dim != 16 && p->head_k_dim != 64 && p->head_k_dim != 128))
        return GDN_ERR_UNSUPPORTED;
    if (p->conv_kernel != kK) return GDN_ERR_UNSUPPORTED;
    const long long D = 2LL * p->num_k_heads * p->head_k_dim + 1LL * p->num_v_heads * p->head_v_dim;
    if (D > 0x7fffffffLL) return GDN_ERR_SHAPE;
    return GDN_OK;
}

long long dimD(const gdn_params* p) {
    return 2LL * p->num_k_heads * p->head_k_dim + 1LL * p->num_v_heads * p->head_v_dim;
}
size_t esize(const gdn_params* p) { return p->in_dtype == GDN_BF16 ? 2 : 4; }
size_t tile_bytes(const gdn_params* p) {
    return static_cast<size_t>(p->head_k_dim) * p->head_v_dim * sizeof(float);
}

gdn_status launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

// gdn_fusion -> kernel view; checks that each enabled fusion has all its arrays.
gdn_status fusion_of(const gdn_fusion* f, gdn::Fusion* out) {
    *out = gdn::Fusion{nullptr, nullptr, nullptr, nullptr, 0.f};
    if (f == nullptr) return GDN_OK;
    if (f->A_log != nullptr && f->dt_bias == nullptr) return GDN_ERR_NULL;
    if (f->z != nullptr) {
        if (f->norm_weight == nullptr) return GDN_ERR_NULL;
        if (!std::isfinite(f->norm_eps) || f->norm_eps < 0.f) return GDN_ERR_SHAPE;
    }
    out->A_log = f->A_log;
    out->dt_bias = f->A_log ? f->dt_bias : nullptr;
    out->z = f->z;
    out->norm_w = f->z ? f->norm_weight : nullptr;
    out->norm_eps = f->z ? f->norm_eps : 0.f;
    return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "invalid or inconsistent sizes";
        case GDN_ERR_DTYPE: return "in_dtype is not GDN_F32 or GDN_BF16";
        case GDN_ERR_UNSUPPORTED: return "configuration outside the supported set";
        case GDN_ERR_ALIAS: return "an output buffer overlaps another buffer";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_LAUNCH: return "kernel launch failed";
        case GDN_ERR_ALIGN: return "tensor pointer misaligned";
        case GDN_ERR_TOO_LARGE: return "the call needs more than the library's static scratch (128 MiB)";
    }
    return "unknown status";
}

int32_t gdn_version(void) { return 1 * 10000 + 0 * 100 + 0; }

gdn_status gdn_conv1d_silu(const gdn_params* p, int32_t B, int32_t L, const void* qkv,
                           const void* conv_weight, const void* conv_state_in,
                           void* conv_state_out, float* y, const int32_t* cu_seqlens,
                           int32_t N, void* stream) {
    gdn_status st = check_params(p);
    if (st != GDN_OK) return st;
    if (B < 0 || L < 0 || N < 0) return GDN_ERR_SHAPE;
    if (cu_seqlens == nullptr ? (N != B) : (B != 1)) return GDN_ERR_SHAPE;
    const long long D = dimD(p);
    if ((static_cast<long long>(L) + 255) / 256 * D * B > kMaxGrid) return GDN_ERR_SHAPE;
    if (static_cast<long long>(N) * D > kMaxGrid * 256) return GDN_ERR_SHAPE;
    const bool has_tokens = static_cast<long long>(B) * L > 0;
    if (N == 0 && !has_tokens) return GDN_OK;
    // with no tokens, qkv and y may be empty (NULL): only the conv window is copied
    if ((has_tokens && (!qkv || !y)) || !conv_weight || !conv_state_in || !conv_state_out)
        return GDN_ERR_NULL;
    const size_t es = esize(p);
    const Buf bufs[] = {
        {qkv, static_cast<size_t>(B) * D * L * es, false},
        {conv_weight, static_cast<size_t>(D) * kK * es, false},
        {conv_state_in, static_cast<size_t>(N) * D * (kK - 1) * es, false},
        {cu_seqlens, cu_seqlens ? static_cast<size_t>(N + 1) * 4 : 0, false},
        {conv_state_out, static_cast<size_t>(N) * D * (kK - 1) * es, true},
        {y, static_cast<size_t>(B) * D * L * 4, true},
    };
    if ((st = check_alias(bufs)) != GDN_OK) return st;
    const gdn::ConvArgs a{B, L, static_cast<int>(D), N, qkv, conv_weight, conv_state_in,
                          conv_state_out, y, cu_seqlens};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (has_tokens) {
        if ((st = launched(gdn::launch_conv1d_silu(a, p->in_dtype, s))) != GDN_OK) return st;
    }
    if (N > 0) return launched(gdn::launch_conv_state(a, p->in_dtype, s));
    return GDN_OK;
}

// decode (in_place: S_out == S_in), verify (S_out = snapshots) and verify from
// the snapshots of a previous block (slot != NULL: S_in is [B, slot_T, Hv, dk, dv]
// and sequence b starts from its snapshot slot[b]; S_in == S_out is allowed when
// slot_T == T, since every (sequence, head) tile is read whole before it is written)
static gdn_status recurrent_common(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                                   int32_t T, const void* qkv, const void* gate, const void* beta,
                                   const void* conv_weight, const void* conv_state_in,
                                   void* conv_state_out, const float* S_in, float* S_out, float* o,
                                   void* stream, bool in_place, bool slots = false,
                                   const int32_t* slot = nullptr, int32_t slot_T = 0) {
    gdn_status st = check_params(p);
    if (st != GDN_OK) return st;
    if (slots && slot_T < 1) return GDN_ERR_SHAPE;
    if (slots && slot_T > kMaxT) return GDN_ERR_UNSUPPORTED;
    gdn::Fusion fu;
    if ((st = fusion_of(fusion, &fu)) != GDN_OK) return st;
    if (B < 0) return GDN_ERR_SHAPE;
    if (T < 1) return GDN_ERR_SHAPE;
    if (T > kMaxT) return GDN_ERR_UNSUPPORTED;
    if (static_cast<long long>(B) * p->num_v_heads > kMaxGrid) return GDN_ERR_SHAPE;
    if (B == 0) return GDN_OK;
    if (!qkv || !gate || !beta || !conv_weight || !conv_state_in || !S_in || !S_out || !o)
        return GDN_ERR_NULL;
    if (slots && slot == nullptr) return GDN_ERR_NULL;
    if (in_place && !conv_state_out) return GDN_ERR_NULL;
    if (!aligned(S_in, 16) || !aligned(S_out, 16) || !aligned(o, 16)) return GDN_ERR_ALIGN;
    const long long D = dimD(p);
    const size_t es = esize(p);
    const size_t Hv = static_cast<size_t>(p->num_v_heads);
    const size_t state = static_cast<size_t>(B) * Hv * tile_bytes(p);
    const bool same = slot != nullptr && S_in == S_out && slot_T == T;   // snapshots updated in place
    const size_t in_bytes = (in_place || same) ? 0 : state * (slot != nullptr ? slot_T : 1);
    const Buf bufs[] = {
        {qkv, static_cast<size_t>(B) * D * T * es, false},
        {gate, static_cast<size_t>(B) * T * Hv * es, false},
        {beta, static_cast<size_t>(B) * T * Hv * es, false},
        {conv_weight, static_cast<size_t>(D) * kK * es, false},
        {conv_state_in, static_cast<size_t>(B) * D * (kK - 1) * es, false},
        {slot, slot != nullptr ? static_cast<size_t>(B) * 4 : 0, false},
        // an input updated in place is listed once, as an output
        {S_in, in_bytes, false},
        {conv_state_out, conv_state_out ? static_cast<size_t>(B) * D * (kK - 1) * es : 0, true},
        {S_out, state * T, true},
        {o, static_cast<size_t>(B) * T * Hv * p->head_v_dim * sizeof(float), true},
        {fu.A_log, fu.A_log ? Hv * es : 0, false},
        {fu.dt_bias, fu.dt_bias ? Hv * es : 0, false},
        {fu.z, fu.z ? static_cast<size_t>(B) * T * Hv * p->head_v_dim * es : 0, false},
        {fu.norm_w, fu.norm_w ? static_cast<size_t>(p->head_v_dim) * es : 0, false},
    };
    if ((st = check_alias(bufs)) != GDN_OK) return st;
    const gdn::RecArgs a{B, T, p->num_k_heads, p->num_v_heads, static_cast<int>(D),
                         p->use_qk_l2norm, p->l2norm_eps, qkv, gate, beta, conv_weight,
                         conv_state_in, conv_state_out, S_in, S_out, o, fu, slot, slot_T};
    return launched(gdn::launch_recurrent(a, p->in_dtype, p->head_k_dim, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_step(const gdn_params* p, int32_t B, const void* qkv, const void* gate,
                           const void* beta, const void* conv_weight, const void* conv_state_in,
                           void* conv_state_out, float* S, float* o, void* stream) {
    return recurrent_common(p, nullptr, B, 1, qkv, gate, beta, conv_weight, conv_state_in,
                            conv_state_out, S, S, o, stream, true);
}

gdn_status gdn_decode_step_ex(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                              const void* qkv, const void* gate, const void* beta,
                              const void* conv_weight, const void* conv_state_in,
                              void* conv_state_out, float* S, float* o, void* stream) {
    return recurrent_common(p, fusion, B, 1, qkv, gate, beta, conv_weight, conv_state_in,
                            conv_state_out, S, S, o, stream, true);
}

gdn_status gdn_verify_block(const gdn_params* p, int32_t B, int32_t T, const void* qkv,
                            const void* gate, const void* beta, const void* conv_weight,
                            const void* conv_state_in, const float* S_in, float* S_snap,
                            float* o, void* stream) {
    return recurrent_common(p, nullptr, B, T, qkv, gate, beta, conv_weight, conv_state_in, nullptr,
                            S_in, S_snap, o, stream, false);
}

gdn_status gdn_verify_block_ex(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                               int32_t T, const void* qkv, const void* gate, const void* beta,
                               const void* conv_weight, const void* conv_state_in,
                               const float* S_in, float* S_snap, float* o, void* stream) {
    return recurrent_common(p, fusion, B, T, qkv, gate, beta, conv_weight, conv_state_in, nullptr,
                            S_in, S_snap, o, stream, false);
}

gdn_status gdn_verify_block_slots(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                                  int32_t T, const void* qkv, const void* gate, const void* beta,
                                  const void* conv_weight, const void* conv_state_in,
                                  const float* S_prev, int32_t T_prev, const int32_t* slot,
                                  float* S_snap, float* o, void* stream) {
    return recurrent_common(p, fusion, B, T, qkv, gate, beta, conv_weight, conv_state_in, nullptr,
                            S_prev, S_snap, o, stream, false, true, slot, T_prev);
}

gdn_status gdn_verify_commit(const gdn_params* p, int32_t B, int32_t T,
                             const int32_t* accept_len, const void* qkv,
                             const void* conv_state_in, const float* S_snap,
                             void* conv_state_out, float* S_out, void* stream) {
    gdn_status st = check_params(p);
    if (st != GDN_OK) return st;
    if (B < 0 || T < 1) return GDN_ERR_SHAPE;
    if (T > kMaxT) return GDN_ERR_UNSUPPORTED;
    if (static_cast<long long>(B) * p->num_v_heads > kMaxGrid) return GDN_ERR_SHAPE;
    if (B == 0) return GDN_OK;
    if (!accept_len || !qkv || !conv_state_in || !conv_state_out) return GDN_ERR_NULL;
    if ((S_snap == nullptr) != (S_out == nullptr)) return GDN_ERR_NULL;   // both NULL: window only
    if (!aligned(S_snap, 16) || !aligned(S_out, 16)) return GDN_ERR_ALIGN;
    const long long D = dimD(p);
    const size_t es = esize(p);
    const size_t state = static_cast<size_t>(B) * p->num_v_heads * tile_bytes(p);
    const Buf bufs[] = {
        {accept_len, static_cast<size_t>(B) * 4, false},
        {qkv, static_cast<size_t>(B) * D * T * es, false},
        {conv_state_in, static_cast<size_t>(B) * D * (kK - 1) * es, false},
        {S_snap, S_snap ? state * T : 0, false},
        {conv_state_out, static_cast<size_t>(B) * D * (kK - 1) * es, true},
        {S_out, S_out ? state : 0, true},
    };
    if ((st = check_alias(bufs)) != GDN_OK) return st;
    const gdn::CommitArgs a{B, T, p->num_v_heads, static_cast<int>(D), accept_len, qkv,
                            conv_state_in, S_snap, conv_state_out, S_out};
    return launched(gdn::launch_commit(a, p->in_dtype, p->head_k_dim, static_cast<hipStream_t>(stream)));
}

static gdn_status prefill_check_sizes(const gdn_params* p, int32_t B, int32_t L, int32_t N,
                                      int32_t chunk, bool ragged) {
    gdn_status st = check_params(p);
    if (st != GDN_OK) return st;
    if (B < 0 || L < 0 || N < 0 || chunk <= 0) return GDN_ERR_SHAPE;
    if (chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (ragged ? (B != 1) : (N != B)) return GDN_ERR_SHAPE;
    const long long D = dimD(p);
    const long long units = 2LL * p->num_k_heads + p->num_v_heads;
    if (static_cast<long long>(B) * ((L + 31) / 32) * units > kMaxGrid) return GDN_ERR_SHAPE;
    if ((static_cast<long long>(B) * ((L + chunk - 1) / chunk) + N) * p->num_v_heads > kMaxGrid)
        return GDN_ERR_SHAPE;
    if (static_cast<long long>(N) * D > kMaxGrid * 256) return GDN_ERR_SHAPE;
    return GDN_OK;
}

size_t gdn_prefill_workspace_size(const gdn_params* p, int32_t B, int32_t L, int32_t N,
                                  int32_t chunk) {
    // valid for either packing, with cu_seqlens (B == 1) or without (N == B), and with or
    // without the gated RMSNorm epilogue: the largest of those layouts
    if (prefill_check_sizes(p, B, L, N, chunk, B == 1) != GDN_OK &&
        prefill_check_sizes(p, B, L, N, chunk, false) != GDN_OK)
        return 0;
    size_t most = 0;
    for (const bool ragged : {false, true})
        for (const bool norm : {false, true})
            most = std::max(most, gdn::prefill_workspace_bytes(B, L, N, p->num_k_heads, p->num_v_heads,
                                                               p->head_k_dim, chunk, p->in_dtype, ragged, norm));
    return most;
}

gdn_status gdn_prefill(const gdn_params* p, int32_t B, int32_t L, const void* qkv,
                       const void* gate, const void* beta, const void* conv_weight,
                       const void* conv_state_in, void* conv_state_out, float* S, float* o,
                       const int32_t* cu_seqlens, int32_t N, int32_t chunk, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return gdn_prefill_ex(p, nullptr, B, L, qkv, gate, beta, conv_weight, conv_state_in,
                          conv_state_out, S, o, cu_seqlens, N, chunk, workspace, workspace_bytes,
                          stream);
}

gdn_status gdn_prefill_ex(const gdn_params* p, const gdn_fusion* fusion, int32_t B, int32_t L,
                          const void* qkv, const void* gate, const void* beta,
                          const void* conv_weight, const void* conv_state_in,
                          void* conv_state_out, float* S, float* o, const int32_t* cu_seqlens,
                          int32_t N, int32_t chunk, void* workspace, size_t workspace_bytes,
                          void* stream) {
    const bool ragged = cu_seqlens != nullptr;
    gdn_status st = prefill_check_sizes(p, B, L, N, chunk, ragged);
    if (st != GDN_OK) return st;
    gdn::Fusion fu;
    if ((st = fusion_of(fusion, &fu)) != GDN_OK) return st;
    if (N == 0) return GDN_OK;
    // with no tokens (B*L == 0) qkv, gate, beta and o may be empty (NULL): S is kept
    // and the conv window copied
    const bool has_tokens = static_cast<long long>(B) * L > 0;
    if ((has_tokens && (!qkv || !gate || !beta || !o)) || !conv_weight || !conv_state_in ||
        !conv_state_out || !S)
        return GDN_ERR_NULL;
    if (!aligned(S, 16) || (o && !aligned(o, 16))) return GDN_ERR_ALIGN;
    const size_t need = gdn::prefill_workspace_bytes(B, L, N, p->num_k_heads, p->num_v_heads, p->head_k_dim,
                                                     chunk, p->in_dtype, ragged, fu.z != nullptr);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 256)) return GDN_ERR_ALIGN;
    const long long D = dimD(p);
    const size_t es = esize(p);
    const size_t Hv = static_cast<size_t>(p->num_v_heads);
    const Buf bufs[] = {
        {qkv, static_cast<size_t>(B) * D * L * es, false},
        {gate, static_cast<size_t>(B) * L * Hv * es, false},
        {beta, static_cast<size_t>(B) * L * Hv * es, false},
        {conv_weight, static_cast<size_t>(D) * kK * es, false},
        {conv_state_in, static_cast<size_t>(N) * D * (kK - 1) * es, false},
        {cu_seqlens, ragged ? static_cast<size_t>(N + 1) * 4 : 0, false},
        {conv_state_out, static_cast<size_t>(N) * D * (kK - 1) * es, true},
        {S, static_cast<size_t>(N) * Hv * tile_bytes(p), true},
        {o, static_cast<size_t>(B) * L * Hv * p->head_v_dim * sizeof(float), true},
        {workspace, need, true},
        {fu.A_log, fu.A_log ? Hv * es : 0, false},
        {fu.dt_bias, fu.dt_bias ? Hv * es : 0, false},
        {fu.z, fu.z ? static_cast<size_t>(B) * L * Hv * p->head_v_dim * es : 0, false},
        {fu.norm_w, fu.norm_w ? static_cast<size_t>(p->head_v_dim) * es : 0, false},
    };
    if ((st = check_alias(bufs)) != GDN_OK) return st;
    const gdn::PrefillArgs a{B, L, N, p->num_k_heads, p->num_v_heads, static_cast<int>(D), chunk,
                             p->use_qk_l2norm, p->l2norm_eps, qkv, gate, beta, conv_weight,
                             conv_state_in, conv_state_out, S, o, cu_seqlens, workspace,
                             workspace_bytes, fu};
    return launched(gdn::launch_prefill(a, p->in_dtype, p->head_k_dim, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace gdn {

// The workspace one prefill call needs, for its own packing and fusion (at most what
// gdn_prefill_workspace_size reports), or 0 for arguments that gdn_prefill_ex rejects
// before it looks at the workspace.
size_t prefill_call_workspace_bytes(const gdn_params* p, const gdn_fusion* fusion, int B, int L, int N, int chunk,
                                    bool ragged) {
    Fusion fu;
    if (prefill_check_sizes(p, B, L, N, chunk, ragged) != GDN_OK || fusion_of(fusion, &fu) != GDN_OK) return 0;
    return prefill_workspace_bytes(B, L, N, p->num_k_heads, p->num_v_heads, p->head_k_dim, chunk, p->in_dtype,
                                   ragged, fu.z != nullptr);
}

}  // namespace gdn
