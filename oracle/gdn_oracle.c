/*
 * Gated DeltaNet layer: plain, slow fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library. The product path (the HIP
 * library) never calls it, shares no code with it and is not linked with it.
 *
 * What it computes follows the page "MNN Model Support: Qwen3.5" (alibaba/MNN
 * discussion 4354):
 *   - §1.2 "Algorithm Principles": the operator inputs qkv [B,D,L], gate [B,L,H],
 *     beta [B,L,H], conv_weight [D,1,K] and the five steps (depthwise causal
 *     Conv1D + SiLU; split Q/K/V + GQA expansion; optional per-head L2
 *     normalisation of Q and K; Q scaled by 1/sqrt(d_k); the gated delta rule
 *     recurrence, token by token).
 *   - §1.3 "Reverse GQA": K and Q heads are expanded to the V heads with
 *     repeat_interleave, so V head h reads K/Q head h / (Hv/Hk).
 *   - §1.4 "MNN Implementation": LinearAttentionParam (head counts, head dims,
 *     use_qk_l2norm) and the two persistent states, the conv state [B,D,K-1]
 *     (sliding window history) and the recurrent state [B,H,d_k,d_v], both
 *     carried across calls.
 * Readings taken where the page is silent (each one also listed in the design
 * notes):
 *   - channel order inside D is [Q | K | V], each head-major (head*d + i);
 *   - the conv is a cross-correlation over the window
 *     concat(conv_state, x) whose last tap w[d][K-1] multiplies the current
 *     token, no bias; the conv state holds the K-1 most recent raw inputs,
 *     oldest first;
 *   - L2 norm is x * (sum x^2 + eps)^(-1/2), applied before the 1/sqrt(d_k)
 *     scale (step 3 precedes step 4);
 *   - gate and beta carry one value per V head (one per recurrent state);
 *   - the output of token t is read from the state after token t's write.
 *   - ragged packing: with cu_seqlens, B must be 1 and sequence n owns the
 *     tokens [cu[n], cu[n+1]) of row 0 and its own states [n].
 *   - speculative commit keeps the snapshot after token index a (1 + a tokens)
 *     and the conv window after the same token; a is clamped to [0, T-1].
 *
 * Everything is fp64 with plain loops. Independent (sequence, V head) units run
 * on a small pool of pthreads; the arithmetic inside a unit is in the page's
 * order. A test-only "mutation" switch plants one known mistake at a time so
 * that the tests can show each pin catches it.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_NOMEM (-2)

typedef struct {
    int num_k_heads;   /* Hk */
    int num_v_heads;   /* Hv */
    int head_k_dim;    /* dk */
    int head_v_dim;    /* dv */
    int conv_k;        /* K  */
    int use_qk_l2norm;
    double eps;
} orc_params;

/* ---- test-only mistake planting ---------------------------------------- */
enum {
    MUT_NONE = 0,
    MUT_NO_DECAY_BEFORE_PREDICT = 1, /* predict from the undecayed state */
    MUT_DELTA_SIGN = 2,              /* delta = beta (v_pred - v) */
    MUT_GQA_TILED = 3,               /* V head h reads K head h % Hk */
    MUT_OUT_PRE_WRITE = 4,           /* o read before the outer-product write */
    MUT_SCALE_BEFORE_NORM = 5,       /* 1/sqrt(dk) applied before the L2 norm */
    MUT_CONV_REVERSED = 6,           /* conv taps reversed */
    MUT_K_NOT_NORMED = 7,            /* L2 norm applied to q only */
    MUT_CONV_STATE_SHIFT = 8,        /* conv state window one token early */
    MUT_PREDICT_TRANSPOSED = 9,      /* v_pred = S k instead of S^T k */
    MUT_NO_BETA = 10,                /* delta = v - v_pred */
    MUT_QK_SWAPPED = 11,             /* Q and K channel blocks swapped */
    MUT_NO_SILU = 12,                /* conv output without SiLU */
    MUT_DECAY_AFTER_WRITE = 13,      /* decay applied after the write */
    MUT_GATE_SIGN = 14,              /* gate = +exp(A_log) softplus(..) */
    MUT_RMS_SUM = 15,                /* RMSNorm with the sum of squares, not the mean */
    MUT_RMS_SIGMOID_GATE = 16,       /* output gated by sigmoid(z), not silu(z) */
};
static int g_mutation = 0;
void orc_set_mutation(int m) { g_mutation = m; }
int orc_get_mutation(void) { return g_mutation; }

/* ---- small helpers ------------------------------------------------------ */
static double silu(double x) { return x / (1.0 + exp(-x)); }

static int check_params(const orc_params* p) {
    if (!p) return ORC_ERR_ARG;
    if (p->num_k_heads <= 0 || p->num_v_heads <= 0 || p->head_k_dim <= 0 || p->head_v_dim <= 0)
        return ORC_ERR_ARG;
    if (p->conv_k < 1) return ORC_ERR_ARG;
    if (p->num_v_heads % p->num_k_heads != 0) return ORC_ERR_ARG;
    return ORC_OK;
}

static int64_t dim_D(const orc_params* p) {
    return 2LL * p->num_k_heads * p->head_k_dim + (int64_t)p->num_v_heads * p->head_v_dim;
}

/* Sequence n -> (batch row, first token, length). */
static int segment(int n, int L, const int32_t* cu, int* row, int* start, int* len) {
    if (cu) {
        *row = 0;
        *start = cu[n];
        *len = cu[n + 1] - cu[n];
    } else {
        *row = n;
        *start = 0;
        *len = L;
    }
    return (*len >= 0) ? ORC_OK : ORC_ERR_ARG;
}

static int check_segments(int B, int L, const int32_t* cu, int N) {
    if (B < 0 || L < 0 || N < 0) return ORC_ERR_ARG;
    if (!cu) return (N == B) ? ORC_OK : ORC_ERR_ARG;
    if (B != 1 || cu[0] != 0 || cu[N] != L) return ORC_ERR_ARG;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return ORC_ERR_ARG;
    return ORC_OK;
}

/* ---- Step 1: depthwise causal Conv1D + SiLU of one channel ------------------
 * Window xh = concat(conv_state[c][0..K-2], x[c][start .. start+len-1]).
 * y[t] = silu( sum_j w[c][j] * xh[t + j] ),  t = 0..len-1.
 * The new conv state is the last K-1 entries of xh. */
static void conv_channel(int K, const double* w_c, const double* state_c, const double* x_c,
                         int len, double* y_c, double* state_out_c) {
    for (int t = 0; t < len; ++t) {
        double acc = 0.0;
        for (int j = 0; j < K; ++j) {
            int tap = (g_mutation == MUT_CONV_REVERSED) ? (K - 1 - j) : j;
            int pos = t + j; /* position in xh */
            double xv = (pos < K - 1) ? state_c[pos] : x_c[pos - (K - 1)];
            acc += w_c[tap] * xv;
        }
        y_c[t] = (g_mutation == MUT_NO_SILU) ? acc : silu(acc);
    }
    if (state_out_c) {
        int shift = (g_mutation == MUT_CONV_STATE_SHIFT) ? 1 : 0;
        for (int p = 0; p < K - 1; ++p) {
            int pos = len + p - shift; /* last K-1 of xh: positions len .. len+K-2 */
            if (pos < 0) pos = 0;
            state_out_c[p] = (pos < K - 1) ? state_c[pos] : x_c[pos - (K - 1)];
        }
    }
}

/* ---- Steps 2-4 for one (sequence, V head): gather q, k, v of every token -----
 * y_q, y_k: conv outputs of the dk channels of K head hk, y_v: of V head h;
 * each laid out [channel][t]. Writes token-major q[t][i], k[t][i], v[t][j]. */
static void l2_normalise(double* x, int n, double eps) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; ++i) x[i] *= r;
}

static void qkv_heads(const orc_params* p, int len, const double* y_q, const double* y_k,
                      const double* y_v, double* q, double* k, double* v) {
    const int dk = p->head_k_dim, dv = p->head_v_dim;
    const double scale = 1.0 / sqrt((double)dk);
    for (int t = 0; t < len; ++t) {
        double* qt = q + (size_t)t * dk;
        double* kt = k + (size_t)t * dk;
        double* vt = v + (size_t)t * dv;
        for (int i = 0; i < dk; ++i) {
            qt[i] = y_q[(size_t)i * len + t];
            kt[i] = y_k[(size_t)i * len + t];
        }
        for (int j = 0; j < dv; ++j) vt[j] = y_v[(size_t)j * len + t];
        if (g_mutation == MUT_SCALE_BEFORE_NORM)
            for (int i = 0; i < dk; ++i) qt[i] *= scale;
        if (p->use_qk_l2norm) {                         /* Step 3 */
            l2_normalise(qt, dk, p->eps);
            if (g_mutation != MUT_K_NOT_NORMED) l2_normalise(kt, dk, p->eps);
        }
        if (g_mutation != MUT_SCALE_BEFORE_NORM)        /* Step 4 */
            for (int i = 0; i < dk; ++i) qt[i] *= scale;
    }
}

/* ---- Step 5: the gated delta rule for one head ------------------------------
 * For t = 0..L-1 (S is dk x dv, row-major, S[i][j]):
 *   S      <- exp(g_t) * S
 *   v_pred  = S^T k_t                  (v_pred[j] = sum_i S[i][j] k_t[i])
 *   delta   = beta_t * (v_t - v_pred)
 *   S      <- S + k_t delta^T          (S[i][j] += k_t[i] delta[j])
 *   o_t     = S^T q_t                  (o_t[j] = sum_i S[i][j] q_t[i])
 * q, k: [L][dk]; v, o: [L][dv]; snap (optional): [L][dk][dv], state after each token. */
int orc_delta_rule(int L, int dk, int dv, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, double* S, double* o, double* snap) {
    if (L < 0 || dk <= 0 || dv <= 0 || !S) return ORC_ERR_ARG;
    double* vp = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
    double* dl = (double*)malloc(sizeof(double) * (size_t)dv);
    double* oo = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!vp || !dl || !oo) { free(vp); free(dl); free(oo); return ORC_ERR_NOMEM; }
    for (int t = 0; t < L; ++t) {
        const double* kt = k + (size_t)t * dk;
        const double* qt = q + (size_t)t * dk;
        const double* vt = v + (size_t)t * dv;
        const double a = exp(g[t]);
        const double b = beta[t];
        if (g_mutation != MUT_NO_DECAY_BEFORE_PREDICT && g_mutation != MUT_DECAY_AFTER_WRITE)
            for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] *= a;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            if (g_mutation == MUT_PREDICT_TRANSPOSED && dk == dv)
                for (int i = 0; i < dk; ++i) acc += S[(size_t)j * dv + i] * kt[i];
            else
                for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * kt[i];
            vp[j] = acc;
        }
        if (g_mutation == MUT_NO_DECAY_BEFORE_PREDICT)
            for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] *= a;
        for (int j = 0; j < dv; ++j) {
            double d = (g_mutation == MUT_DELTA_SIGN) ? (vp[j] - vt[j]) : (vt[j] - vp[j]);
            dl[j] = (g_mutation == MUT_NO_BETA) ? d : b * d;
        }
        if (g_mutation == MUT_OUT_PRE_WRITE) {
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qt[i];
                oo[j] = acc;
            }
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * dl[j];
        if (g_mutation == MUT_DECAY_AFTER_WRITE)
            for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] *= a;
        if (g_mutation != MUT_OUT_PRE_WRITE) {
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qt[i];
                oo[j] = acc;
            }
        }
        if (o) memcpy(o + (size_t)t * dv, oo, sizeof(double) * (size_t)dv);
        if (snap) memcpy(snap + (size_t)t * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    }
    free(vp); free(dl); free(oo);
    return ORC_OK;
}

/* Channel indices of the split (Step 2) under the [Q | K | V] head-major reading. */
static int64_t chan_q(const orc_params* p, int hk, int i) {
    int64_t base = (g_mutation == MUT_QK_SWAPPED) ? (int64_t)p->num_k_heads * p->head_k_dim : 0;
    return base + (int64_t)hk * p->head_k_dim + i;
}
static int64_t chan_k(const orc_params* p, int hk, int i) {
    int64_t base = (g_mutation == MUT_QK_SWAPPED) ? 0 : (int64_t)p->num_k_heads * p->head_k_dim;
    return base + (int64_t)hk * p->head_k_dim + i;
}
static int64_t chan_v(const orc_params* p, int h, int j) {
    return 2LL * p->num_k_heads * p->head_k_dim + (int64_t)h * p->head_v_dim + j;
}
/* Reverse GQA: repeat_interleave(factor) maps V head h to K/Q head h / factor. */
static int k_head_of(const orc_params* p, int h) {
    int factor = p->num_v_heads / p->num_k_heads;
    return (g_mutation == MUT_GQA_TILED) ? (h % p->num_k_heads) : (h / factor);
}

/* ---- a pool of threads over independent work units ------------------------- */
typedef struct {
    int64_t n_units;
    int64_t next;
    pthread_mutex_t mu;
    int (*fn)(void* ctx, int64_t unit);
    void* ctx;
    int status;
} pool_t;

static void* pool_worker(void* arg) {
    pool_t* pl = (pool_t*)arg;
    for (;;) {
        pthread_mutex_lock(&pl->mu);
        int64_t u = pl->next++;
        pthread_mutex_unlock(&pl->mu);
        if (u >= pl->n_units) break;
        int st = pl->fn(pl->ctx, u);
        if (st != ORC_OK) {
            pthread_mutex_lock(&pl->mu);
            pl->status = st;
            pthread_mutex_unlock(&pl->mu);
        }
    }
    return NULL;
}

static int run_pool(int64_t n_units, int nthreads, int (*fn)(void*, int64_t), void* ctx) {
    pool_t pl;
    pl.n_units = n_units; pl.next = 0; pl.fn = fn; pl.ctx = ctx; pl.status = ORC_OK;
    pthread_mutex_init(&pl.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads == 1 || n_units <= 1) {
        pool_worker(&pl);
    } else {
        pthread_t th[256];
        int started = 0;
        for (int i = 0; i < nthreads; ++i)
            if (pthread_create(&th[i], NULL, pool_worker, &pl) == 0) ++started;
        if (started == 0) pool_worker(&pl);
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    }
    pthread_mutex_destroy(&pl.mu);
    return pl.status;
}

/* ---- Step 1 on its own: conv1d + SiLU over every channel -------------------- */
typedef struct {
    const orc_params* p; int L; const int32_t* cu; int N;
    const double* x; const double* w; const double* conv_in; double* conv_out; double* y;
} conv_ctx;

static int conv_unit(void* vctx, int64_t u) {
    conv_ctx* c = (conv_ctx*)vctx;
    const int64_t D = dim_D(c->p);
    const int K = c->p->conv_k;
    int n = (int)(u / D);
    int64_t ch = u % D;
    int row, start, len;
    if (segment(n, c->L, c->cu, &row, &start, &len) != ORC_OK) return ORC_ERR_ARG;
    const double* x_c = c->x + ((size_t)row * D + ch) * c->L + start;
    double* y_c = c->y ? c->y + ((size_t)row * D + ch) * c->L + start : NULL;
    double* ybuf = y_c ? y_c : (double*)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
    if (!ybuf) return ORC_ERR_NOMEM;
    conv_channel(K, c->w + ch * K, c->conv_in + ((size_t)n * D + ch) * (K - 1), x_c, len, ybuf,
                 c->conv_out ? c->conv_out + ((size_t)n * D + ch) * (K - 1) : NULL);
    if (!y_c) free(ybuf);
    return ORC_OK;
}

/* y [B,D,L] = silu(conv(x)) per channel; conv_out [N,D,K-1] = new window (nullable). */
int orc_conv1d_silu(const orc_params* p, int B, int L, const double* x, const double* w,
                    const double* conv_in, double* conv_out, double* y,
                    const int32_t* cu_seqlens, int N, int nthreads) {
    if (check_params(p) != ORC_OK) return ORC_ERR_ARG;
    if (check_segments(B, L, cu_seqlens, N) != ORC_OK) return ORC_ERR_ARG;
    if (!x || !w || !conv_in) return ORC_ERR_ARG;
    conv_ctx c = {p, L, cu_seqlens, N, x, w, conv_in, conv_out, y};
    return run_pool((int64_t)N * dim_D(p), nthreads, conv_unit, &c);
}

/* ---- Steps 1-4 for one (sequence, V head) unit ------------------------------ */
static int unit_front_end(const orc_params* p, int L, const int32_t* cu, int n, int h,
                          const double* x, const double* w, const double* conv_in,
                          int* row_out, int* start_out, int* len_out,
                          double** q_out, double** k_out, double** v_out) {
    const int64_t D = dim_D(p);
    const int K = p->conv_k, dk = p->head_k_dim, dv = p->head_v_dim;
    int row, start, len;
    if (segment(n, L, cu, &row, &start, &len) != ORC_OK) return ORC_ERR_ARG;
    size_t lz = (size_t)(len > 0 ? len : 1);
    double* yq = (double*)malloc(sizeof(double) * lz * dk);
    double* yk = (double*)malloc(sizeof(double) * lz * dk);
    double* yv = (double*)malloc(sizeof(double) * lz * dv);
    double* q = (double*)malloc(sizeof(double) * lz * dk);
    double* k = (double*)malloc(sizeof(double) * lz * dk);
    double* v = (double*)malloc(sizeof(double) * lz * dv);
    if (!yq || !yk || !yv || !q || !k || !v) {
        free(yq); free(yk); free(yv); free(q); free(k); free(v);
        return ORC_ERR_NOMEM;
    }
    const int hk = k_head_of(p, h);
    for (int i = 0; i < dk; ++i) {
        int64_t cq = chan_q(p, hk, i), ck = chan_k(p, hk, i);
        conv_channel(K, w + cq * K, conv_in + ((size_t)n * D + cq) * (K - 1),
                     x + ((size_t)row * D + cq) * L + start, len, yq + (size_t)i * len, NULL);
        conv_channel(K, w + ck * K, conv_in + ((size_t)n * D + ck) * (K - 1),
                     x + ((size_t)row * D + ck) * L + start, len, yk + (size_t)i * len, NULL);
    }
    for (int j = 0; j < dv; ++j) {
        int64_t cv = chan_v(p, h, j);
        conv_channel(K, w + cv * K, conv_in + ((size_t)n * D + cv) * (K - 1),
                     x + ((size_t)row * D + cv) * L + start, len, yv + (size_t)j * len, NULL);
    }
    qkv_heads(p, len, yq, yk, yv, q, k, v);
    free(yq); free(yk); free(yv);
    *row_out = row; *start_out = start; *len_out = len;
    *q_out = q; *k_out = k; *v_out = v;
    return ORC_OK;
}

/* Steps 1-4 for every token and V head: q_hat, k_hat [B,L,Hv,dk], v [B,L,Hv,dv]
 * (K/Q already expanded to the V heads). */
int orc_front_end(const orc_params* p, int B, int L, const double* x, const double* w,
                  const double* conv_in, const int32_t* cu_seqlens, int N,
                  double* q_hat, double* k_hat, double* v_out) {
    if (check_params(p) != ORC_OK) return ORC_ERR_ARG;
    if (check_segments(B, L, cu_seqlens, N) != ORC_OK) return ORC_ERR_ARG;
    if (!x || !w || !conv_in || !q_hat || !k_hat || !v_out) return ORC_ERR_ARG;
    const int Hv = p->num_v_heads, dk = p->head_k_dim, dv = p->head_v_dim;
    for (int n = 0; n < N; ++n) {
        for (int h = 0; h < Hv; ++h) {
            int row, start, len;
            double *q, *k, *v;
            int st = unit_front_end(p, L, cu_seqlens, n, h, x, w, conv_in, &row, &start, &len, &q, &k, &v);
            if (st != ORC_OK) return st;
            for (int t = 0; t < len; ++t) {
                size_t tok = (size_t)row * L + start + t;
                memcpy(q_hat + (tok * Hv + h) * dk, q + (size_t)t * dk, sizeof(double) * dk);
                memcpy(k_hat + (tok * Hv + h) * dk, k + (size_t)t * dk, sizeof(double) * dk);
                memcpy(v_out + (tok * Hv + h) * dv, v + (size_t)t * dv, sizeof(double) * dv);
            }
            free(q); free(k); free(v);
        }
    }
    return ORC_OK;
}

/* ---- the whole layer ----------------------------------------------------------- */
typedef struct {
    const orc_params* p; int L; const int32_t* cu; int N;
    const double *x, *gate, *beta, *w, *conv_in;
    double *S, *o, *snap;
    const unsigned char* mask;
} fwd_ctx;

static int fwd_unit(void* vctx, int64_t u) {
    fwd_ctx* c = (fwd_ctx*)vctx;
    const orc_params* p = c->p;
    const int Hv = p->num_v_heads, dk = p->head_k_dim, dv = p->head_v_dim;
    const int n = (int)(u / Hv), h = (int)(u % Hv);
    if (c->mask && !c->mask[u]) return ORC_OK;
    int row, start, len;
    double *q, *k, *v;
    int st = unit_front_end(p, c->L, c->cu, n, h, c->x, c->w, c->conv_in, &row, &start, &len, &q, &k, &v);
    if (st != ORC_OK) return st;
    size_t lz = (size_t)(len > 0 ? len : 1);
    double* g = (double*)malloc(sizeof(double) * lz);
    double* b = (double*)malloc(sizeof(double) * lz);
    double* o = (double*)malloc(sizeof(double) * lz * dv);
    double* snap = c->snap ? (double*)malloc(sizeof(double) * lz * dk * dv) : NULL;
    if (!g || !b || !o || (c->snap && !snap)) {
        free(q); free(k); free(v); free(g); free(b); free(o); free(snap);
        return ORC_ERR_NOMEM;
    }
    for (int t = 0; t < len; ++t) {
        size_t tok = (size_t)row * c->L + start + t;
        g[t] = c->gate[tok * Hv + h];
        b[t] = c->beta[tok * Hv + h];
    }
    double* S = c->S + ((size_t)n * Hv + h) * dk * dv;
    st = orc_delta_rule(len, dk, dv, q, k, v, g, b, S, o, snap);
    if (st == ORC_OK) {
        for (int t = 0; t < len; ++t) {
            size_t tok = (size_t)row * c->L + start + t;
            if (c->o) memcpy(c->o + (tok * Hv + h) * dv, o + (size_t)t * dv, sizeof(double) * dv);
            if (snap)
                memcpy(c->snap + (tok * Hv + h) * dk * dv, snap + (size_t)t * dk * dv,
                       sizeof(double) * dk * dv);
        }
    }
    free(q); free(k); free(v); free(g); free(b); free(o); free(snap);
    return st;
}

/* Full layer over B rows of L tokens (or N ragged sequences packed in row 0).
 *   x [B,D,L], gate/beta [B,L,Hv], w [D,1,K], conv_in/conv_out [N,D,K-1]
 *   S [N,Hv,dk,dv] in/out; o [B,L,Hv,dv]; snap [B,L,Hv,dk,dv] (nullable): the
 *   state after every token; unit_mask [N*Hv] (nullable): units to compute
 *   (others leave S, o and snap untouched). conv_out is written for every
 *   sequence whatever the mask. */
int orc_gdn_forward(const orc_params* p, int B, int L, const double* x, const double* gate,
                    const double* beta, const double* w, const double* conv_in, double* conv_out,
                    double* S, double* o, double* snap, const int32_t* cu_seqlens, int N,
                    const unsigned char* unit_mask, int nthreads) {
    if (check_params(p) != ORC_OK) return ORC_ERR_ARG;
    if (check_segments(B, L, cu_seqlens, N) != ORC_OK) return ORC_ERR_ARG;
    if (!x || !gate || !beta || !w || !conv_in || !S) return ORC_ERR_ARG;
    fwd_ctx c = {p, L, cu_seqlens, N, x, gate, beta, w, conv_in, S, o, snap, unit_mask};
    int st = run_pool((int64_t)N * p->num_v_heads, nthreads, fwd_unit, &c);
    if (st != ORC_OK) return st;
    if (conv_out) {
        const int64_t D = dim_D(p);
        const int K = p->conv_k;
        for (int n = 0; n < N; ++n) {
            int row, start, len;
            segment(n, L, cu_seqlens, &row, &start, &len);
            for (int64_t ch = 0; ch < D; ++ch) {
                const double* st_c = conv_in + ((size_t)n * D + ch) * (K - 1);
                const double* x_c = x + ((size_t)row * D + ch) * L + start;
                double* out_c = conv_out + ((size_t)n * D + ch) * (K - 1);
                int shift = (g_mutation == MUT_CONV_STATE_SHIFT) ? 1 : 0;
                for (int q = 0; q < K - 1; ++q) {
                    int pos = len + q - shift;
                    if (pos < 0) pos = 0;
                    out_c[q] = (pos < K - 1) ? st_c[pos] : x_c[pos - (K - 1)];
                }
            }
        }
    }
    return ORC_OK;
}

/* ---- gate / beta parameterisation -----------------------------------------------
 * "MNN Model Support: Qwen3.5", §1.2, the paragraph after Step 5: beta is the
 * sigmoid of a raw projection b, and the log-decay is
 *   gate = -exp(A_log) * softplus(a + dt_bias)     (<= 0, so exp(gate) is in (0, 1])
 * with A_log and dt_bias learned per V head. softplus(x) = log(1 + e^x).
 * a, b: [n_tok, Hv]; A_log, dt_bias: [Hv]; outputs gate, beta: [n_tok, Hv]. */
static double softplus(double x) { return x > 0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

int orc_gate_beta(int64_t n_tok, int Hv, const double* a, const double* b, const double* A_log,
                  const double* dt_bias, double* gate, double* beta) {
    if (n_tok < 0 || Hv <= 0 || !a || !b || !A_log || !dt_bias || !gate || !beta) return ORC_ERR_ARG;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int h = 0; h < Hv; ++h) {
            const int64_t i = t * Hv + h;
            gate[i] = (g_mutation == MUT_GATE_SIGN ? 1.0 : -1.0) * exp(A_log[h]) * softplus(a[i] + dt_bias[h]);
            beta[i] = 1.0 / (1.0 + exp(-b[i]));
        }
    return ORC_OK;
}

/* ---- gated RMSNorm -----------------------------------------------------------------
 * "MNN Model Support: Qwen3.5", §2 "Gated RMSNorm": over the last dimension,
 *   h = x * rsqrt(mean(x^2) + eps);  h = weight * h;  h = h * silu(gate)
 * applied to the layer output per (token, V head) over d_v, the gate being z
 * from in_proj_z. x, z, out: [n_rows, dv]; weight: [dv]. */
int orc_gated_rmsnorm(int64_t n_rows, int dv, const double* x, const double* z, const double* weight,
                      double eps, double* out) {
    if (n_rows < 0 || dv <= 0 || !x || !z || !weight || !out) return ORC_ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        const double* xr = x + r * dv;
        const double* zr = z + r * dv;
        double ms = 0.0;
        for (int j = 0; j < dv; ++j) ms += xr[j] * xr[j];
        if (g_mutation != MUT_RMS_SUM) ms /= dv;
        const double inv = 1.0 / sqrt(ms + eps);
        for (int j = 0; j < dv; ++j) {
            const double gz = (g_mutation == MUT_RMS_SIGMOID_GATE) ? 1.0 / (1.0 + exp(-zr[j])) : silu(zr[j]);
            out[r * dv + j] = weight[j] * (xr[j] * inv) * gz;
        }
    }
    return ORC_OK;
}

/* ---- speculative commit ----------------------------------------------------------
 * For each row b with a = clamp(accept_len[b], 0, T-1):
 *   S_out[b]    = snap[b][a]  (state after 1 + a tokens of the block)
 *   conv_out[b] = the K-1 raw inputs that precede token a+1 in
 *                 concat(conv_in[b], x[b][:, 0..T-1]), oldest first. */
int orc_verify_commit(const orc_params* p, int B, int T, const int32_t* accept_len,
                      const double* x, const double* conv_in, const double* snap,
                      double* conv_out, double* S_out) {
    if (check_params(p) != ORC_OK) return ORC_ERR_ARG;
    if (B < 0 || T < 1 || !accept_len || !x || !conv_in || !snap || !conv_out || !S_out)
        return ORC_ERR_ARG;
    const int64_t D = dim_D(p);
    const int K = p->conv_k, Hv = p->num_v_heads;
    const size_t tile = (size_t)p->head_k_dim * p->head_v_dim;
    for (int b = 0; b < B; ++b) {
        int a = accept_len[b];
        if (a < 0) a = 0;
        if (a > T - 1) a = T - 1;
        for (int h = 0; h < Hv; ++h)
            memcpy(S_out + ((size_t)b * Hv + h) * tile, snap + (((size_t)b * T + a) * Hv + h) * tile,
                   sizeof(double) * tile);
        for (int64_t ch = 0; ch < D; ++ch) {
            const double* st_c = conv_in + ((size_t)b * D + ch) * (K - 1);
            const double* x_c = x + ((size_t)b * D + ch) * T;
            double* out_c = conv_out + ((size_t)b * D + ch) * (K - 1);
            for (int q = 0; q < K - 1; ++q) {
                int pos = a + 1 + q; /* window positions a+1 .. a+K-1 of the concat */
                out_c[q] = (pos < K - 1) ? st_c[pos] : x_c[pos - (K - 1)];
            }
        }
    }
    return ORC_OK;
}
