// Internal launch interface between the C-ABI layer (gdn_api.cpp) and the
// kernel files. Every struct is passed to its kernel by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Optional prologue (A_log != nullptr: gate/beta hold the raw a/b) and epilogue
// (z != nullptr: gated RMSNorm of o). See gdn_fusion in gdn.h.
struct Fusion {
    const void* A_log;      // [Hv]
    const void* dt_bias;    // [Hv]
    const void* z;          // like o
    const void* norm_w;     // [dv]
    float norm_eps;
};

// decode (T = 1, S_out == S_in allowed) and verify (S_out = snapshots)
struct RecArgs {
    int B, T, Hk, Hv, D;
    int use_l2;
    float eps;
    const void* qkv;      // [B, D, T]
    const void* gate;     // [B, T, Hv]
    const void* beta;     // [B, T, Hv]
    const void* w;        // [D, 1, K]
    const void* conv_in;  // [B, D, K-1]
    void* conv_out;       // [B, D, K-1] or nullptr
    const float* S_in;    // [B, Hv, dk, dv], or [B, slot_T, Hv, dk, dv] with slot
    float* S_out;         // [B, T, Hv, dk, dv]
    float* o;             // [B, T, Hv, dv]
    Fusion fu;
    const int32_t* slot;  // [B] snapshot index per sequence (clamped to [0, slot_T)), or nullptr
    int slot_T;           // snapshots per sequence in S_in when slot is set
};

struct CommitArgs {
    int B, T, Hv, D;
    const int32_t* accept;  // [B]
    const void* qkv;        // [B, D, T]
    const void* conv_in;    // [B, D, K-1]
    const float* S_snap;    // [B, T, Hv, dk, dv]
    void* conv_out;         // [B, D, K-1]
    float* S_out;           // [B, Hv, dk, dv], or nullptr (then S_snap is unused: conv window only)
};

struct ConvArgs {
    int B, L, D, N;
    const void* qkv;         // [B, D, L]
    const void* w;           // [D, 1, K]
    const void* conv_in;     // [N, D, K-1]
    void* conv_out;          // [N, D, K-1]
    float* y;                // [B, D, L] or nullptr
    const int32_t* cu;       // [N+1] or nullptr
};

struct PrefillArgs {
    int B, L, N, Hk, Hv, D, chunk;
    int use_l2;
    float eps;
    const void* qkv;         // [B, D, L]
    const void* gate;        // [B, L, Hv]
    const void* beta;        // [B, L, Hv]
    const void* w;           // [D, 1, K]
    const void* conv_in;     // [N, D, K-1]
    void* conv_out;          // [N, D, K-1]
    float* S;                // [N, Hv, dk, dv]
    float* o;                // [B, L, Hv, dv]
    const int32_t* cu;       // [N+1] or nullptr
    void* ws;                // workspace
    size_t ws_bytes;
    Fusion fu;
};

hipError_t launch_recurrent(const RecArgs& a, int in_dtype, int d, hipStream_t stream);
hipError_t launch_commit(const CommitArgs& a, int in_dtype, int d, hipStream_t stream);
hipError_t launch_conv1d_silu(const ConvArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_conv_state(const ConvArgs& a, int in_dtype, hipStream_t stream);
// workspace of a prefill call with (ragged) or without cu_seqlens, with (norm) or without
// the gated RMSNorm epilogue
size_t prefill_workspace_bytes(int B, int L, int N, int Hk, int Hv, int d, int chunk, int in_dtype, bool ragged,
                               bool norm);
hipError_t launch_prefill(const PrefillArgs& a, int in_dtype, int d, hipStream_t stream);
size_t prefill_mfma_workspace_bytes(int B, int L, int N, int Hk, int Hv, bool ragged, bool norm);
hipError_t launch_prefill_mfma(const PrefillArgs& a, int in_dtype, hipStream_t stream);
// gated RMSNorm of o in place over the tokens of every sequence (prefill epilogue)
hipError_t launch_prefill_epilogue(const PrefillArgs& a, int in_dtype, int d, hipStream_t stream);

}  // namespace gdn
