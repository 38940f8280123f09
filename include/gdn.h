/*
 * gdn.h — C ABI of the Gated DeltaNet linear-attention layer on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is the one the page "MNN Model Support: Qwen3.5" (alibaba/MNN
 * discussion 4354) defines in §1.2 "Algorithm Principles":
 *   Step 1  depthwise causal Conv1D over qkv [B, D, L] with conv_weight
 *           [D, 1, K], followed by SiLU;
 *   Step 2  split of the conv output into Q, K, V and the GQA expansion of §1.3
 *           ("Reverse GQA": K and Q heads repeat_interleave'd to the V heads);
 *   Step 3  optional per-head L2 normalisation of Q and K;
 *   Step 4  Q scaled by 1/sqrt(d_k);
 *   Step 5  the gated delta rule, token by token, on a per-V-head state
 *           S in R^{d_k x d_v}:  S *= exp(gate_t); v_pred = S^T k_t;
 *           delta = beta_t (v_t - v_pred); S += k_t delta^T; o_t = S^T q_t.
 * §1.4 gives the parameter table (LinearAttentionParam) and the two persistent
 * states, conv state [B, D, K-1] and recurrent state [B, H, d_k, d_v], that the
 * caller zero-fills before the first call and carries across calls.
 *
 * Readings taken where the page is silent:
 *   - D = 2*Hk*dk + Hv*dv, channels ordered [Q | K | V], each head-major
 *     (channel = head*d + i); V head h reads K/Q head h / (Hv/Hk).
 *   - conv: cross-correlation over concat(conv_state, x) whose last tap
 *     w[c][0][K-1] multiplies the current token, no bias. The conv state holds
 *     the K-1 most recent raw (pre-conv) inputs, oldest first, in the input
 *     dtype, so carrying it is lossless.
 *   - L2 norm: x * (sum x^2 + eps)^(-1/2), per token and head, before the
 *     1/sqrt(dk) scale.
 *   - gate and beta hold one value per V head: [B, L, Hv]. gate is the
 *     log-decay (applied as exp(gate)); it is not clamped.
 *   - the output of a token is read from the state after that token's write.
 *   - outputs o and the state S are fp32; inputs (qkv, gate, beta,
 *     conv_weight, conv states) are bf16 or fp32 as `in_dtype` says.
 *
 * Conventions for every call:
 *   - All tensor pointers are device pointers to caller-owned, contiguous
 *     memory in the layouts stated per call, 16-byte aligned. The library never
 *     allocates; prefill takes a caller-provided workspace.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on it and returns without synchronising.
 *   - Arguments are validated synchronously. On any error the call returns a
 *     non-zero gdn_status and enqueues nothing. A failed launch returns
 *     GDN_ERR_LAUNCH. Faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Index arrays that live on the device (cu_seqlens, accept_len) cannot be
 *     validated on the host; the kernels clamp them (stated per call) so that
 *     no value makes them read or write out of bounds.
 *   - The library is stateless and reentrant. Calls on one stream run in order.
 *   - Supported set: head_k_dim == head_v_dim in {16, 64, 128}; conv_kernel == 4;
 *     Hv % Hk == 0; verify T in [1, 16]; prefill chunk == 64. Anything else
 *     returns GDN_ERR_UNSUPPORTED.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,         /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,        /* a size is negative/zero where it must not be, or sizes disagree */
    GDN_ERR_DTYPE = 3,        /* in_dtype is not a gdn_dtype */
    GDN_ERR_UNSUPPORTED = 4,  /* a valid configuration outside the supported set */
    GDN_ERR_ALIAS = 5,        /* two buffers that must not overlap do */
    GDN_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than the call needs */
    GDN_ERR_LAUNCH = 7,       /* the HIP runtime refused a kernel launch */
    GDN_ERR_ALIGN = 8,        /* a tensor pointer is not 16-byte aligned (workspace: 256) */
    GDN_ERR_TOO_LARGE = 9     /* gdn_prefill_ex_noalloc: the call needs more than its static scratch */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* LinearAttentionParam of §1.4 plus the conv width, the L2-norm epsilon and the
 * input storage type. */
typedef struct {
    int32_t num_k_heads;    /* Hk: K/Q heads                                  */
    int32_t num_v_heads;    /* Hv: V heads (= recurrent states per sequence)  */
    int32_t head_k_dim;     /* dk                                             */
    int32_t head_v_dim;     /* dv                                             */
    int32_t conv_kernel;    /* K (taps of the depthwise conv)                 */
    int32_t use_qk_l2norm;  /* 0 or 1                                         */
    float l2norm_eps;       /* eps of the L2 norm (1e-6 in the tests)         */
    int32_t in_dtype;       /* gdn_dtype of qkv, gate, beta, conv_weight, conv states */
} gdn_params;

/* Optional fusions. A NULL gdn_fusion pointer, or NULL fields, disable them.
 *
 * Prologue ("MNN Model Support: Qwen3.5", §1.2, the gate parameterisation after
 * Step 5): when A_log is non-NULL, the `gate` and `beta` arguments of a call hold
 * the raw projections a and b, and the kernels use, in fp32,
 *     gate = -exp(A_log[h]) * softplus(a + dt_bias[h]),   beta = sigmoid(b).
 *   A_log, dt_bias  [Hv] in_dtype (dt_bias must be non-NULL with A_log)
 *
 * Epilogue (§2 "Gated RMSNorm"): when z is non-NULL, `o` receives, for each
 * (token, V head) over its dv channels,
 *     norm_weight[j] * o[j] * rsqrt(mean_j(o^2) + norm_eps) * silu(z[j])
 * instead of the raw recurrence output.
 *   z            laid out like o ([B, L, Hv, dv]), in_dtype; must not overlap o
 *   norm_weight  [dv] in_dtype (must be non-NULL with z)
 *   norm_eps     >= 0, finite */
typedef struct {
    const void* A_log;
    const void* dt_bias;
    const void* z;
    const void* norm_weight;
    float norm_eps;
} gdn_fusion;

/* Human-readable name of a status code (static storage). */
const char* gdn_status_string(gdn_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t gdn_version(void);

/*
 * gdn_conv1d_silu — Step 1 alone (§1.2 Step 1 and the conv state of §1.4).
 *   qkv            [B, D, L]    in_dtype  input columns
 *   conv_weight    [D, 1, K]    in_dtype
 *   conv_state_in  [N, D, K-1]  in_dtype  window before the first token of each sequence
 *   conv_state_out [N, D, K-1]  in_dtype  window after the last token (must not overlap conv_state_in)
 *   y              [B, D, L]    fp32      silu(conv(x))
 *   cu_seqlens     [N+1] int32 on the device, or NULL. NULL: N == B sequences of
 *                  length L. Otherwise B == 1 and sequence n owns tokens
 *                  [cu[n], cu[n+1]) of row 0; the kernel clamps entries into
 *                  [0, L] and treats a decreasing pair as an empty sequence;
 *                  tokens outside every sequence keep y untouched.
 */
gdn_status gdn_conv1d_silu(const gdn_params* p, int32_t B, int32_t L, const void* qkv,
                           const void* conv_weight, const void* conv_state_in,
                           void* conv_state_out, float* y, const int32_t* cu_seqlens,
                           int32_t N, void* stream);

/*
 * gdn_decode_step — one token per sequence through Steps 1-5 (§1.2), the
 * states carried per §1.4.
 *   qkv            [B, D, 1]          in_dtype
 *   gate, beta     [B, 1, Hv]         in_dtype
 *   conv_weight    [D, 1, K]          in_dtype
 *   conv_state_in  [B, D, K-1]        in_dtype
 *   conv_state_out [B, D, K-1]        in_dtype  (must not overlap conv_state_in: with
 *                                      GQA several workgroups read the same channels)
 *   S              [B, Hv, dk, dv]    fp32, updated in place
 *   o              [B, 1, Hv, dv]     fp32
 */
gdn_status gdn_decode_step(const gdn_params* p, int32_t B, const void* qkv, const void* gate,
                           const void* beta, const void* conv_weight, const void* conv_state_in,
                           void* conv_state_out, float* S, float* o, void* stream);

/*
 * gdn_verify_block — T tokens per sequence (a speculative block: one accepted
 * token followed by T-1 drafted ones) through Steps 1-5, writing the state
 * after every token so that a rejected suffix can be rolled back. The
 * per-token arithmetic is the decode step's, so snapshot t equals the state
 * after t+1 calls of gdn_decode_step bit for bit.
 *   qkv            [B, D, T]          in_dtype
 *   gate, beta     [B, T, Hv]         in_dtype
 *   conv_weight    [D, 1, K]          in_dtype
 *   conv_state_in  [B, D, K-1]        in_dtype  (read only)
 *   S_in           [B, Hv, dk, dv]    fp32      (read only; must not overlap S_snap)
 *   S_snap         [B, T, Hv, dk, dv] fp32      state after each token
 *   o              [B, T, Hv, dv]     fp32
 */
gdn_status gdn_verify_block(const gdn_params* p, int32_t B, int32_t T, const void* qkv,
                            const void* gate, const void* beta, const void* conv_weight,
                            const void* conv_state_in, const float* S_in, float* S_snap,
                            float* o, void* stream);

/*
 * gdn_verify_commit — keep the accepted prefix of a verify block.
 * For row b with a = accept_len[b] (device int32, clamped into [0, T-1]):
 *   S_out[b]          = S_snap[b, a]        (the state after 1 + a tokens)
 *   conv_state_out[b] = the K-1 raw inputs preceding token a+1 in
 *                       concat(conv_state_in[b], qkv[b, :, 0..T-1]), oldest first.
 *   accept_len     [B] int32 (device)
 *   qkv            [B, D, T] in_dtype (the block given to gdn_verify_block)
 *   conv_state_in  [B, D, K-1] in_dtype (the one given to gdn_verify_block)
 *   S_snap         [B, T, Hv, dk, dv] fp32
 *   conv_state_out [B, D, K-1] in_dtype (must not overlap conv_state_in)
 *   S_out          [B, Hv, dk, dv] fp32 (must not overlap S_snap)
 * S_snap and S_out may both be NULL: then only the conv window is rolled (the
 * state stays in the snapshots, for gdn_verify_block_slots).
 */
gdn_status gdn_verify_commit(const gdn_params* p, int32_t B, int32_t T,
                             const int32_t* accept_len, const void* qkv,
                             const void* conv_state_in, const float* S_snap,
                             void* conv_state_out, float* S_out, void* stream);

/*
 * gdn_verify_block_slots — the next verify block started straight from the
 * snapshots of the previous one, so that accepting a prefix copies no state
 * ("mlxcel benchmarks" page, lablup/mlxcel docs/benchmarks.md, the MTP
 * speculative-decoding section: a drafted block is verified in one forward
 * pass and its block width is swept from 2 to 8). Identical to
 * gdn_verify_block_ex, bit for bit, with S_in[b] = S_prev[b, slot[b]].
 *   S_prev         [B, T_prev, Hv, dk, dv] fp32  snapshots of the previous block
 *   T_prev         1..16
 *   slot           [B] int32 (device), clamped into [0, T_prev-1]; for the
 *                  speculative loop it is the accept_len of the previous block
 *   S_snap         [B, T, Hv, dk, dv] fp32; may be S_prev itself when
 *                  T == T_prev (every (sequence, head) tile is read whole by one
 *                  workgroup before that workgroup writes it); any other overlap
 *                  with S_prev is GDN_ERR_ALIAS
 *   conv_state_in  the window after the accepted prefix, e.g. from
 *                  gdn_verify_commit with S_snap = S_out = NULL
 * Other arguments as for gdn_verify_block_ex. slot NULL: GDN_ERR_NULL.
 */
gdn_status gdn_verify_block_slots(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                                  int32_t T, const void* qkv, const void* gate, const void* beta,
                                  const void* conv_weight, const void* conv_state_in,
                                  const float* S_prev, int32_t T_prev, const int32_t* slot,
                                  float* S_snap, float* o, void* stream);

/*
 * gdn_prefill_workspace_size — bytes of device workspace gdn_prefill needs for
 * these sizes and p->in_dtype (bf16 inputs at head dim 128 take the MFMA path,
 * whose workspace is smaller than the fp32 path's); an upper bound that holds
 * whatever cu_seqlens contains, and with or without the fusions of gdn_prefill_ex.
 * Returns 0 when the arguments are invalid or unsupported.
 */
size_t gdn_prefill_workspace_size(const gdn_params* p, int32_t B, int32_t L, int32_t N,
                                  int32_t chunk);

/*
 * gdn_prefill — a whole prompt through Steps 1-5 with the recurrence evaluated
 * in chunks (an exact algebraic rewrite of Step 5: within a chunk the
 * sequential updates are solved at once through a unit-lower-triangular
 * system; the state is carried from chunk to chunk).
 *   qkv            [B, D, L]          in_dtype
 *   gate, beta     [B, L, Hv]         in_dtype
 *   conv_weight    [D, 1, K]          in_dtype
 *   conv_state_in  [N, D, K-1]        in_dtype
 *   conv_state_out [N, D, K-1]        in_dtype (must not overlap conv_state_in)
 *   S              [N, Hv, dk, dv]    fp32, initial state in, final state out (in place)
 *   o              [B, L, Hv, dv]     fp32 (tokens outside every sequence untouched)
 *   cu_seqlens     as for gdn_conv1d_silu (NULL: N == B sequences of length L)
 *   chunk          chunk length (64)
 *   workspace      device memory, 256-byte aligned, of workspace_bytes bytes:
 *                  gdn_prefill_workspace_size() always suffices; a call given fewer
 *                  bytes than its own layout needs (which depends on cu_seqlens and,
 *                  for gdn_prefill_ex, on the fusions) returns GDN_ERR_WORKSPACE. Its
 *                  contents on entry do not matter.
 */
gdn_status gdn_prefill(const gdn_params* p, int32_t B, int32_t L, const void* qkv,
                       const void* gate, const void* beta, const void* conv_weight,
                       const void* conv_state_in, void* conv_state_out, float* S, float* o,
                       const int32_t* cu_seqlens, int32_t N, int32_t chunk, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * The same calls with the optional prologue/epilogue fusions of gdn_fusion
 * (fusion may be NULL: identical to the calls above). Arguments, layouts and
 * errors are as above; with a prologue `gate`/`beta` carry the raw a/b.
 */
gdn_status gdn_decode_step_ex(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                              const void* qkv, const void* gate, const void* beta,
                              const void* conv_weight, const void* conv_state_in,
                              void* conv_state_out, float* S, float* o, void* stream);
gdn_status gdn_verify_block_ex(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                               int32_t T, const void* qkv, const void* gate, const void* beta,
                               const void* conv_weight, const void* conv_state_in,
                               const float* S_in, float* S_snap, float* o, void* stream);
gdn_status gdn_prefill_ex(const gdn_params* p, const gdn_fusion* fusion, int32_t B, int32_t L,
                          const void* qkv, const void* gate, const void* beta,
                          const void* conv_weight, const void* conv_state_in,
                          void* conv_state_out, float* S, float* o, const int32_t* cu_seqlens,
                          int32_t N, int32_t chunk, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * gdn_prefill_ex_noalloc — gdn_prefill_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops that must not call hipMalloc, harnesses
 * that forbid it). Identical to gdn_prefill_ex, bit for bit, except that the workspace is
 * a static array of 128 MiB (134217728 bytes) inside the library instead of a caller
 * buffer; the caller still passes every input and output. The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the array's address is looked
 * up once per device (hipGetSymbolAddress, on the first call made with that device
 * current) and the device holds the array until the process ends.
 *   Limit: a call whose own workspace (for its packing and fusion; at most
 *   gdn_prefill_workspace_size()) exceeds 134217728 bytes returns GDN_ERR_TOO_LARGE and
 *   enqueues nothing: with bf16 inputs at 16 K / 32 V heads of dimension 128, one
 *   prompt of up to 3,584 tokens, or 3,200 with the gated RMSNorm epilogue (whose
 *   carry runs in more segments).
 *   Sharing: every call on one device uses that device's one array. Calls that can run
 *   at the same time on one device (different streams, or different host threads) race
 *   on it and must be serialised by the caller; calls on one stream run in order and
 *   are safe. The array's contents on entry do not matter (nothing in it is read before
 *   the call writes it).
 * Other arguments, layouts and errors as gdn_prefill_ex.
 */
gdn_status gdn_prefill_ex_noalloc(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                                  int32_t L, const void* qkv, const void* gate, const void* beta,
                                  const void* conv_weight, const void* conv_state_in,
                                  void* conv_state_out, float* S, float* o,
                                  const int32_t* cu_seqlens, int32_t N, int32_t chunk,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
