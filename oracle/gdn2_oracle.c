/*
 * Gated DeltaNet-2 forward recurrence: plain FP64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is slow on purpose and
 * written so that each step can be checked against the pages by eye.
 *
 * Sources (web pages; cited by title and section):
 *   [IPX]  "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention",
 *          analysis at iplexlaw.co.kr -- sections "Independent decisions on two
 *          axes" (the update equations) and "Token processing and parallel
 *          training" (64-token chunkwise WY form, FP32 decay / solve).
 *   [MP]   "DeltaNet" entity trail at mindpattern.ai -- finding "You Could Have
 *          Come Up With Kimi Delta Attention": per-key-channel decay with
 *          per-token transitions are a diagonal decay composed with a
 *          rank-one correction; the fused recurrent and chunkwise forms give
 *          the same result.
 *
 * The method, per head, per token t, with state S in R^{dk x dv} (keys index
 * rows) [IPX, "Independent decisions on two axes"]:
 *     e_t  = b_t (.) k_t                 erase vector on key channels
 *     z_t  = w_t (.) v_t                 write vector on value channels
 *     Sbar = Diag(alpha_t) S_{t-1}       channel-wise decay on key channels
 *     r_t  = Sbar^T e_t                  old read
 *     S_t  = Sbar + k_t (z_t - r_t)^T    delta update
 *     o_t  = S_t^T q_t                   output from the state AFTER the update
 *
 * Functions:
 *   gdn2_oracle_recurrent   O1  the definition, token by token  (THE oracle)
 *   gdn2_oracle_chunked     O2  chunkwise WY form, any chunk size C (pin)
 *   gdn2_oracle_transition  O3  explicit dk x dk transition products (pin)
 *   gdn2_oracle_kda         O4a Kimi-Delta-Attention form (pin for b=w=beta)
 *   gdn2_oracle_gdn         O4b Gated DeltaNet form (pin for scalar alpha)
 *   gdn2_oracle_backward    O5  gradients of O1 (reverse mode, token by token)
 *
 * Layouts (row-major, contiguous, FP64):
 *   q, k, b, alpha : [B, T, H, dk]        v, w, o : [B, T, H, dv]
 *   initial / final state : [N, H, dk, dv]
 *   With cu_seqlens (int32 [N+1], host memory) B must be 1 and sequence n
 *   occupies packed tokens [cu_seqlens[n], cu_seqlens[n+1]); otherwise N = B
 *   and sequence n is batch row n with T tokens.
 *   chains (optional, int32 [num_chains]) selects which (n*H + h) chains are
 *   evaluated; outputs of the other chains are left untouched.  NULL = all.
 *   initial_state NULL = zeros; final_state NULL = not written.
 * Return value: 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t B, T, H, dk, dv, N;
    const int32_t* cu;
} shape_t;

/* Token range and batch row of sequence n. */
static void seq_bounds(const shape_t* s, int32_t n, int64_t* bos, int64_t* eos, int64_t* brow)
{
    if (s->cu) {
        *bos = s->cu[n];
        *eos = s->cu[n + 1];
        *brow = 0;
    } else {
        *bos = 0;
        *eos = s->T;
        *brow = n;
    }
}

/* Offset of element 0 of token t (within batch row brow) for head h. */
static int64_t tok_off(const shape_t* s, int64_t brow, int64_t t, int32_t h, int32_t width)
{
    return ((brow * s->T + t) * s->H + h) * (int64_t)width;
}

static int check_shape(const shape_t* s)
{
    if (s->B <= 0 || s->T < 0 || s->H <= 0 || s->dk <= 0 || s->dv <= 0 || s->N <= 0) return -1;
    if (s->cu) {
        if (s->B != 1) return -1;
        if (s->cu[0] != 0) return -1;
        for (int32_t n = 0; n < s->N; ++n)
            if (s->cu[n + 1] < s->cu[n]) return -1;
        if (s->cu[s->N] > s->T) return -1;
    } else if (s->N != s->B) {
        return -1;
    }
    return 0;
}

static int pick_threads(int32_t nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * O1: the recurrence exactly as defined [IPX, "Independent decisions on two
 * axes"], one token at a time.  S is dk x dv, row c = key channel c.
 * ---------------------------------------------------------------------- */
static void recurrent_chain(const shape_t* s, int32_t n, int32_t h,
                            const double* q, const double* k, const double* v,
                            const double* alpha, const double* b, const double* w,
                            const double* S0, double* Sf, double* o)
{
    const int32_t dk = s->dk, dv = s->dv;
    double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* e = (double*)malloc(sizeof(double) * dk);
    double* z = (double*)malloc(sizeof(double) * dv);
    double* r = (double*)malloc(sizeof(double) * dv);
    const int64_t soff = ((int64_t)n * s->H + h) * dk * dv;
    if (S0) memcpy(S, S0 + soff, sizeof(double) * dk * dv);

    int64_t bos, eos, brow;
    seq_bounds(s, n, &bos, &eos, &brow);
    for (int64_t t = bos; t < eos; ++t) {
        const double* qt = q + tok_off(s, brow, t, h, dk);
        const double* kt = k + tok_off(s, brow, t, h, dk);
        const double* bt = b + tok_off(s, brow, t, h, dk);
        const double* at = alpha + tok_off(s, brow, t, h, dk);
        const double* vt = v + tok_off(s, brow, t, h, dv);
        const double* wt = w + tok_off(s, brow, t, h, dv);
        double* ot = o + tok_off(s, brow, t, h, dv);

        for (int32_t c = 0; c < dk; ++c) e[c] = bt[c] * kt[c];          /* e = b (.) k */
        for (int32_t j = 0; j < dv; ++j) z[j] = wt[j] * vt[j];          /* z = w (.) v */
        for (int32_t c = 0; c < dk; ++c)                                /* Sbar = Diag(alpha) S */
            for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= at[c];
        for (int32_t j = 0; j < dv; ++j) {                              /* r = Sbar^T e */
            double acc = 0.0;
            for (int32_t c = 0; c < dk; ++c) acc += S[c * dv + j] * e[c];
            r[j] = acc;
        }
        for (int32_t c = 0; c < dk; ++c)                                /* S = Sbar + k (z - r)^T */
            for (int32_t j = 0; j < dv; ++j) S[c * dv + j] += kt[c] * (z[j] - r[j]);
        for (int32_t j = 0; j < dv; ++j) {                              /* o = S^T q */
            double acc = 0.0;
            for (int32_t c = 0; c < dk; ++c) acc += S[c * dv + j] * qt[c];
            ot[j] = acc;
        }
    }
    if (Sf) memcpy(Sf + soff, S, sizeof(double) * dk * dv);
    free(S);
    free(e);
    free(z);
    free(r);
}

/* ------------------------------------------------------------------------
 * O2: the chunkwise form [IPX, "Token processing and parallel training"]:
 * within a chunk the running per-channel decay is folded into unequal row
 * and column factors (row side e * exp(+G), column side k * exp(-G)), which
 * leaves a unit-lower-triangular solve and dense products:
 *   G_i  = sum_{m<=i} log alpha_m                 (per key channel)
 *   Et_i = e_i exp(G_i),  Kh_j = k_j exp(-G_j),  Qt_i = q_i exp(G_i),
 *   Kb_j = k_j exp(G_last - G_j)
 *   A    = strict_lower(Et Kh^T),  P = lower_incl_diag(Qt Kh^T)
 *   Tm   = (I + A)^{-1}           (forward substitution)
 *   W    = Tm Et,   Ut = Tm Z,    U = Ut - W S0
 *   O    = Qt S0 + P U,           S_last = Diag(exp(G_last)) S0 + Kb^T U
 * Chunks restart at every sequence start; the last chunk may be short.
 * Requires alpha > 0 (log).  FP64; meant for small inputs.
 * ---------------------------------------------------------------------- */
static void chunked_chain(const shape_t* s, int32_t n, int32_t h, int32_t C,
                          const double* q, const double* k, const double* v,
                          const double* alpha, const double* b, const double* w,
                          const double* S0, double* Sf, double* o)
{
    const int32_t dk = s->dk, dv = s->dv;
    const size_t LK = (size_t)C * dk, LV = (size_t)C * dv, LL = (size_t)C * C;
    double* S  = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* G  = (double*)malloc(sizeof(double) * LK);
    double* Et = (double*)malloc(sizeof(double) * LK);
    double* Kh = (double*)malloc(sizeof(double) * LK);
    double* Qt = (double*)malloc(sizeof(double) * LK);
    double* Kb = (double*)malloc(sizeof(double) * LK);
    double* Z  = (double*)malloc(sizeof(double) * LV);
    double* A  = (double*)malloc(sizeof(double) * LL);
    double* P  = (double*)malloc(sizeof(double) * LL);
    double* Tm = (double*)malloc(sizeof(double) * LL);
    double* W  = (double*)malloc(sizeof(double) * LK);
    double* U  = (double*)malloc(sizeof(double) * LV);
    double* Sn = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    const int64_t soff = ((int64_t)n * s->H + h) * dk * dv;
    if (S0) memcpy(S, S0 + soff, sizeof(double) * dk * dv);

    int64_t bos, eos, brow;
    seq_bounds(s, n, &bos, &eos, &brow);
    for (int64_t t0 = bos; t0 < eos; t0 += C) {
        const int32_t L = (int32_t)((eos - t0) < C ? (eos - t0) : C);
        /* cumulative log decay and absorbed factors */
        for (int32_t i = 0; i < L; ++i) {
            const int64_t ok = tok_off(s, brow, t0 + i, h, dk);
            const int64_t ov = tok_off(s, brow, t0 + i, h, dv);
            for (int32_t c = 0; c < dk; ++c) {
                const double prev = i ? G[(size_t)(i - 1) * dk + c] : 0.0;
                G[(size_t)i * dk + c] = prev + log(alpha[ok + c]);
            }
            for (int32_t c = 0; c < dk; ++c) {
                const double g = G[(size_t)i * dk + c];
                Et[(size_t)i * dk + c] = b[ok + c] * k[ok + c] * exp(g);
                Kh[(size_t)i * dk + c] = k[ok + c] * exp(-g);
                Qt[(size_t)i * dk + c] = q[ok + c] * exp(g);
            }
            for (int32_t j = 0; j < dv; ++j) Z[(size_t)i * dv + j] = w[ov + j] * v[ov + j];
        }
        for (int32_t i = 0; i < L; ++i)
            for (int32_t c = 0; c < dk; ++c)
                Kb[(size_t)i * dk + c] = Kh[(size_t)i * dk + c] * exp(G[(size_t)(L - 1) * dk + c]);
        /* A (strictly lower) and P (lower including the diagonal) */
        for (int32_t i = 0; i < L; ++i)
            for (int32_t j = 0; j < L; ++j) {
                double a = 0.0, p = 0.0;
                for (int32_t c = 0; c < dk; ++c) {
                    a += Et[(size_t)i * dk + c] * Kh[(size_t)j * dk + c];
                    p += Qt[(size_t)i * dk + c] * Kh[(size_t)j * dk + c];
                }
                A[(size_t)i * C + j] = j < i ? a : 0.0;
                P[(size_t)i * C + j] = j <= i ? p : 0.0;
            }
        /* Tm = (I + A)^{-1}, unit lower triangular, column by column */
        for (int32_t j = 0; j < L; ++j)
            for (int32_t i = 0; i < L; ++i) {
                if (i < j) { Tm[(size_t)i * C + j] = 0.0; continue; }
                if (i == j) { Tm[(size_t)i * C + j] = 1.0; continue; }
                double acc = 0.0;
                for (int32_t m = j; m < i; ++m) acc += A[(size_t)i * C + m] * Tm[(size_t)m * C + j];
                Tm[(size_t)i * C + j] = -acc;
            }
        /* W = Tm Et ; U = Tm Z - W S */
        for (int32_t i = 0; i < L; ++i) {
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t m = 0; m <= i; ++m) acc += Tm[(size_t)i * C + m] * Et[(size_t)m * dk + c];
                W[(size_t)i * dk + c] = acc;
            }
            for (int32_t j = 0; j < dv; ++j) {
                double ut = 0.0, ws = 0.0;
                for (int32_t m = 0; m <= i; ++m) ut += Tm[(size_t)i * C + m] * Z[(size_t)m * dv + j];
                for (int32_t c = 0; c < dk; ++c) ws += W[(size_t)i * dk + c] * S[(size_t)c * dv + j];
                U[(size_t)i * dv + j] = ut - ws;
            }
        }
        /* O = Qt S + P U */
        for (int32_t i = 0; i < L; ++i) {
            double* ot = o + tok_off(s, brow, t0 + i, h, dv);
            for (int32_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int32_t c = 0; c < dk; ++c) acc += Qt[(size_t)i * dk + c] * S[(size_t)c * dv + j];
                for (int32_t m = 0; m <= i; ++m) acc += P[(size_t)i * C + m] * U[(size_t)m * dv + j];
                ot[j] = acc;
            }
        }
        /* S <- Diag(exp(G_last)) S + Kb^T U */
        for (int32_t c = 0; c < dk; ++c) {
            const double gl = exp(G[(size_t)(L - 1) * dk + c]);
            for (int32_t j = 0; j < dv; ++j) {
                double acc = gl * S[(size_t)c * dv + j];
                for (int32_t m = 0; m < L; ++m) acc += Kb[(size_t)m * dk + c] * U[(size_t)m * dv + j];
                Sn[(size_t)c * dv + j] = acc;
            }
        }
        memcpy(S, Sn, sizeof(double) * dk * dv);
    }
    if (Sf) memcpy(Sf + soff, S, sizeof(double) * dk * dv);
    free(S); free(G); free(Et); free(Kh); free(Qt); free(Kb); free(Z);
    free(A); free(P); free(Tm); free(W); free(U); free(Sn);
}

/* ------------------------------------------------------------------------
 * O3: the same recurrence written with explicit transition matrices
 * [MP: with per-channel gating each step's transition is a diagonal matrix
 * plus a rank-one term]:
 *     M_t = (I - k_t e_t^T) Diag(alpha_t)      (dk x dk)
 *     S_t = M_t S_{t-1} + k_t z_t^T,   o_t = S_t^T q_t
 * ---------------------------------------------------------------------- */
static void transition_chain(const shape_t* s, int32_t n, int32_t h,
                             const double* q, const double* k, const double* v,
                             const double* alpha, const double* b, const double* w,
                             const double* S0, double* Sf, double* o)
{
    const int32_t dk = s->dk, dv = s->dv;
    double* S  = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* Sn = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* M  = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    const int64_t soff = ((int64_t)n * s->H + h) * dk * dv;
    if (S0) memcpy(S, S0 + soff, sizeof(double) * dk * dv);

    int64_t bos, eos, brow;
    seq_bounds(s, n, &bos, &eos, &brow);
    for (int64_t t = bos; t < eos; ++t) {
        const int64_t ok = tok_off(s, brow, t, h, dk);
        const int64_t ov = tok_off(s, brow, t, h, dv);
        for (int32_t r = 0; r < dk; ++r)
            for (int32_t c = 0; c < dk; ++c) {
                const double id = r == c ? 1.0 : 0.0;
                M[(size_t)r * dk + c] = (id - k[ok + r] * b[ok + c] * k[ok + c]) * alpha[ok + c];
            }
        for (int32_t r = 0; r < dk; ++r)
            for (int32_t j = 0; j < dv; ++j) {
                double acc = k[ok + r] * w[ov + j] * v[ov + j];
                for (int32_t c = 0; c < dk; ++c) acc += M[(size_t)r * dk + c] * S[(size_t)c * dv + j];
                Sn[(size_t)r * dv + j] = acc;
            }
        memcpy(S, Sn, sizeof(double) * dk * dv);
        for (int32_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int32_t r = 0; r < dk; ++r) acc += S[(size_t)r * dv + j] * q[ok + r];
            o[ov + j] = acc;
        }
    }
    if (Sf) memcpy(Sf + soff, S, sizeof(double) * dk * dv);
    free(S);
    free(Sn);
    free(M);
}

/* ------------------------------------------------------------------------
 * O4: the two published relatives the method reduces to [IPX, "Independent
 * decisions on two axes": tying both gates to one scalar beta gives KDA, and
 * also making the decay scalar gives Gated DeltaNet; "From a growing cache to
 * a fixed state" for the roles of the gates].  Written in their own matrix
 * form with a scalar beta per token-head:
 *   KDA: S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   GDN: S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   both: o_t = S_t^T q_t
 * beta: [B, T, H];  KDA alpha: [B, T, H, dk];  GDN alpha: [B, T, H].
 * ---------------------------------------------------------------------- */
static void relative_chain(const shape_t* s, int32_t n, int32_t h, int scalar_alpha,
                           const double* q, const double* k, const double* v,
                           const double* alpha, const double* beta,
                           const double* S0, double* Sf, double* o)
{
    const int32_t dk = s->dk, dv = s->dv;
    double* S  = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* D  = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* M  = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    const int64_t soff = ((int64_t)n * s->H + h) * dk * dv;
    if (S0) memcpy(S, S0 + soff, sizeof(double) * dk * dv);

    int64_t bos, eos, brow;
    seq_bounds(s, n, &bos, &eos, &brow);
    for (int64_t t = bos; t < eos; ++t) {
        const int64_t ok = tok_off(s, brow, t, h, dk);
        const int64_t ov = tok_off(s, brow, t, h, dv);
        const int64_t os = tok_off(s, brow, t, h, 1);
        const double bt = beta[os];
        for (int32_t r = 0; r < dk; ++r)        /* D = decayed state */
            for (int32_t j = 0; j < dv; ++j)
                D[(size_t)r * dv + j] = (scalar_alpha ? alpha[os] : alpha[ok + r]) * S[(size_t)r * dv + j];
        for (int32_t r = 0; r < dk; ++r)        /* M = I - beta k k^T */
            for (int32_t c = 0; c < dk; ++c)
                M[(size_t)r * dk + c] = (r == c ? 1.0 : 0.0) - bt * k[ok + r] * k[ok + c];
        for (int32_t r = 0; r < dk; ++r)
            for (int32_t j = 0; j < dv; ++j) {
                double acc = bt * k[ok + r] * v[ov + j];
                for (int32_t c = 0; c < dk; ++c) acc += M[(size_t)r * dk + c] * D[(size_t)c * dv + j];
                S[(size_t)r * dv + j] = acc;
            }
        for (int32_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int32_t r = 0; r < dk; ++r) acc += S[(size_t)r * dv + j] * q[ok + r];
            o[ov + j] = acc;
        }
    }
    if (Sf) memcpy(Sf + soff, S, sizeof(double) * dk * dv);
    free(S);
    free(D);
    free(M);
}


/* ------------------------------------------------------------------------
 * O5: the gradients of O1 by reverse-mode differentiation, token by token.
 * The analysis page asks for a backward pass that accumulates gradients
 * through the gated keys and values and keeps the channel-wise factors
 * inside the sums [IPX, "Token processing and parallel training"]; this is
 * that adjoint written out for one token, applied from the last token back
 * to the first.  The scalar loss is
 *     L = sum_t <dO_t, o_t> + <dS_final, S_final>,
 * and the results are dL/dq, dL/dk, dL/dv, dL/dalpha, dL/db, dL/dw (same
 * layouts as the inputs) and dL/dS_initial.  Per token, with Sprev the state
 * before it and S the state after it (forward order of O1):
 *     o = S^T q               dq = S dO_t;        dS += q dO_t^T
 *     S = Sbar + k u^T        du = dS^T k;        dk = dS u;   dSbar = dS
 *     u = z - Sbar^T e        dz = du;            de = -Sbar du;  dSbar -= e du^T
 *     Sbar = Diag(alpha) Sprev  dalpha_c = sum_j dSbar[c][j] Sprev[c][j];
 *                              dS (for Sprev) = Diag(alpha) dSbar
 *     e = b (.) k, z = w (.) v  db = de (.) k;  dk += de (.) b;
 *                              dw = dz (.) v;  dv = dz (.) w
 * States are kept at every 64th token and the states inside a 64-token
 * segment are recomputed (forward, as in O1) before the segment is walked
 * backwards; this only bounds memory and changes no arithmetic.
 * ---------------------------------------------------------------------- */
#define O5_SEGMENT 64

/* One forward token of O1 on S in place (the same arithmetic, in order). */
static void o5_forward_token(int32_t dk, int32_t dv, double* S, const double* qt, const double* kt,
                             const double* vt, const double* at, const double* bt, const double* wt,
                             double* e, double* z, double* r)
{
    (void)qt;
    for (int32_t c = 0; c < dk; ++c) e[c] = bt[c] * kt[c];
    for (int32_t j = 0; j < dv; ++j) z[j] = wt[j] * vt[j];
    for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= at[c];
    for (int32_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int32_t c = 0; c < dk; ++c) acc += S[c * dv + j] * e[c];
        r[j] = acc;
    }
    for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) S[c * dv + j] += kt[c] * (z[j] - r[j]);
}

static void backward_chain(const shape_t* s, int32_t n, int32_t h,
                           const double* q, const double* k, const double* v,
                           const double* alpha, const double* b, const double* w,
                           const double* S0, const double* dO, const double* dSf,
                           double* dq, double* dk_out, double* dv_out, double* da,
                           double* db, double* dw, double* dS0)
{
    const int32_t dk = s->dk, dv = s->dv;
    const size_t sz = (size_t)dk * dv;
    const int64_t soff = ((int64_t)n * s->H + h) * dk * dv;
    int64_t bos, eos, brow;
    seq_bounds(s, n, &bos, &eos, &brow);
    const int64_t L = eos - bos;
    const int64_t nseg = (L + O5_SEGMENT - 1) / O5_SEGMENT;

    double* ckpt = (double*)calloc((size_t)(nseg + 1) * sz, sizeof(double)); /* state before segment i */
    double* seg = (double*)malloc((size_t)(O5_SEGMENT + 1) * sz * sizeof(double));
    double* dS = (double*)calloc(sz, sizeof(double));
    double* Sbar = (double*)malloc(sz * sizeof(double));
    double* e = (double*)malloc(sizeof(double) * dk);
    double* z = (double*)malloc(sizeof(double) * dv);
    double* r = (double*)malloc(sizeof(double) * dv);
    double* u = (double*)malloc(sizeof(double) * dv);
    double* du = (double*)malloc(sizeof(double) * dv);
    double* de = (double*)malloc(sizeof(double) * dk);

    /* forward: the state before every segment */
    if (S0) memcpy(ckpt, S0 + soff, sz * sizeof(double));
    {
        double* S = (double*)malloc(sz * sizeof(double));
        memcpy(S, ckpt, sz * sizeof(double));
        for (int64_t t = 0; t < L; ++t) {
            const int64_t T = bos + t;
            o5_forward_token(dk, dv, S, q + tok_off(s, brow, T, h, dk), k + tok_off(s, brow, T, h, dk),
                             v + tok_off(s, brow, T, h, dv), alpha + tok_off(s, brow, T, h, dk),
                             b + tok_off(s, brow, T, h, dk), w + tok_off(s, brow, T, h, dv), e, z, r);
            if ((t + 1) % O5_SEGMENT == 0) memcpy(ckpt + (size_t)((t + 1) / O5_SEGMENT) * sz, S, sz * sizeof(double));
        }
        free(S);
    }

    if (dSf) memcpy(dS, dSf + soff, sz * sizeof(double));
    for (int64_t sgi = nseg - 1; sgi >= 0; --sgi) {
        const int64_t t0 = sgi * O5_SEGMENT;
        const int64_t t1 = t0 + O5_SEGMENT < L ? t0 + O5_SEGMENT : L;
        /* recompute the states of this segment: seg[i] = state after token t0 + i - 1 */
        memcpy(seg, ckpt + (size_t)sgi * sz, sz * sizeof(double));
        for (int64_t t = t0; t < t1; ++t) {
            const int64_t T = bos + t;
            double* S = seg + (size_t)(t - t0 + 1) * sz;
            memcpy(S, seg + (size_t)(t - t0) * sz, sz * sizeof(double));
            o5_forward_token(dk, dv, S, q + tok_off(s, brow, T, h, dk), k + tok_off(s, brow, T, h, dk),
                             v + tok_off(s, brow, T, h, dv), alpha + tok_off(s, brow, T, h, dk),
                             b + tok_off(s, brow, T, h, dk), w + tok_off(s, brow, T, h, dv), e, z, r);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const int64_t T = bos + t;
            const double* Sprev = seg + (size_t)(t - t0) * sz;
            const double* S = seg + (size_t)(t - t0 + 1) * sz;
            const double* qt = q + tok_off(s, brow, T, h, dk);
            const double* kt = k + tok_off(s, brow, T, h, dk);
            const double* bt = b + tok_off(s, brow, T, h, dk);
            const double* at = alpha + tok_off(s, brow, T, h, dk);
            const double* vt = v + tok_off(s, brow, T, h, dv);
            const double* wt = w + tok_off(s, brow, T, h, dv);
            const double* gt = dO + tok_off(s, brow, T, h, dv);
            double* dqt = dq + tok_off(s, brow, T, h, dk);
            double* dkt = dk_out + tok_off(s, brow, T, h, dk);
            double* dbt = db + tok_off(s, brow, T, h, dk);
            double* dat = da + tok_off(s, brow, T, h, dk);
            double* dvt = dv_out + tok_off(s, brow, T, h, dv);
            double* dwt = dw + tok_off(s, brow, T, h, dv);

            /* the token's forward intermediates */
            for (int32_t c = 0; c < dk; ++c) e[c] = bt[c] * kt[c];
            for (int32_t j = 0; j < dv; ++j) z[j] = wt[j] * vt[j];
            for (int32_t c = 0; c < dk; ++c)
                for (int32_t j = 0; j < dv; ++j) Sbar[c * dv + j] = at[c] * Sprev[c * dv + j];
            for (int32_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int32_t c = 0; c < dk; ++c) acc += Sbar[c * dv + j] * e[c];
                u[j] = z[j] - acc;
            }
            /* o = S^T q */
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += S[c * dv + j] * gt[j];
                dqt[c] = acc;
            }
            for (int32_t c = 0; c < dk; ++c)
                for (int32_t j = 0; j < dv; ++j) dS[c * dv + j] += qt[c] * gt[j];
            /* S = Sbar + k u^T */
            for (int32_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int32_t c = 0; c < dk; ++c) acc += dS[c * dv + j] * kt[c];
                du[j] = acc;
            }
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += dS[c * dv + j] * u[j];
                dkt[c] = acc;
            }
            /* u = z - Sbar^T e  (dS now stands for dL/dSbar) */
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += Sbar[c * dv + j] * du[j];
                de[c] = -acc;
            }
            for (int32_t c = 0; c < dk; ++c)
                for (int32_t j = 0; j < dv; ++j) dS[c * dv + j] -= e[c] * du[j];
            /* Sbar = Diag(alpha) Sprev */
            for (int32_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += dS[c * dv + j] * Sprev[c * dv + j];
                dat[c] = acc;
            }
            for (int32_t c = 0; c < dk; ++c)
                for (int32_t j = 0; j < dv; ++j) dS[c * dv + j] *= at[c];
            /* e = b (.) k, z = w (.) v */
            for (int32_t c = 0; c < dk; ++c) {
                dbt[c] = de[c] * kt[c];
                dkt[c] += de[c] * bt[c];
            }
            for (int32_t j = 0; j < dv; ++j) {
                dwt[j] = du[j] * vt[j];
                dvt[j] = du[j] * wt[j];
            }
        }
    }
    if (dS0) memcpy(dS0 + soff, dS, sz * sizeof(double));
    free(ckpt);
    free(seg);
    free(dS);
    free(Sbar);
    free(e);
    free(z);
    free(r);
    free(u);
    free(du);
    free(de);
}

/* ---------------------------------------------------------------------- */

#define CHAIN_LOOP(BODY)                                                              \
    do {                                                                              \
        const int64_t total = chains ? (int64_t)num_chains : (int64_t)s.N * s.H;      \
        if (chains)                                                                   \
            for (int64_t i = 0; i < total; ++i)                                       \
                if (chains[i] < 0 || chains[i] >= s.N * s.H) return -1;               \
        _Pragma("omp parallel for schedule(dynamic, 1) num_threads(nt)")              \
        for (int64_t i = 0; i < total; ++i) {                                         \
            const int32_t id = chains ? chains[i] : (int32_t)i;                       \
            const int32_t n = id / s.H, h = id % s.H;                                 \
            BODY;                                                                     \
        }                                                                             \
    } while (0)

int gdn2_oracle_recurrent(const double* q, const double* k, const double* v,
                          const double* alpha, const double* b, const double* w,
                          const double* initial_state, double* final_state, double* o,
                          const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                          int32_t dk, int32_t dv, int32_t num_seqs,
                          const int32_t* chains, int32_t num_chains, int32_t nthreads)
{
    const shape_t s = {B, T, H, dk, dv, cu_seqlens ? num_seqs : B, cu_seqlens};
    if (check_shape(&s) || !q || !k || !v || !alpha || !b || !w || !o) return -1;
    const int nt = pick_threads(nthreads);
    CHAIN_LOOP(recurrent_chain(&s, n, h, q, k, v, alpha, b, w, initial_state, final_state, o));
    return 0;
}

int gdn2_oracle_chunked(const double* q, const double* k, const double* v,
                        const double* alpha, const double* b, const double* w,
                        const double* initial_state, double* final_state, double* o,
                        const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                        int32_t dk, int32_t dv, int32_t num_seqs, int32_t chunk,
                        const int32_t* chains, int32_t num_chains, int32_t nthreads)
{
    const shape_t s = {B, T, H, dk, dv, cu_seqlens ? num_seqs : B, cu_seqlens};
    if (check_shape(&s) || chunk <= 0 || !q || !k || !v || !alpha || !b || !w || !o) return -1;
    const int nt = pick_threads(nthreads);
    CHAIN_LOOP(chunked_chain(&s, n, h, chunk, q, k, v, alpha, b, w, initial_state, final_state, o));
    return 0;
}

int gdn2_oracle_transition(const double* q, const double* k, const double* v,
                           const double* alpha, const double* b, const double* w,
                           const double* initial_state, double* final_state, double* o,
                           const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                           int32_t dk, int32_t dv, int32_t num_seqs,
                           const int32_t* chains, int32_t num_chains, int32_t nthreads)
{
    const shape_t s = {B, T, H, dk, dv, cu_seqlens ? num_seqs : B, cu_seqlens};
    if (check_shape(&s) || !q || !k || !v || !alpha || !b || !w || !o) return -1;
    const int nt = pick_threads(nthreads);
    CHAIN_LOOP(transition_chain(&s, n, h, q, k, v, alpha, b, w, initial_state, final_state, o));
    return 0;
}

int gdn2_oracle_kda(const double* q, const double* k, const double* v,
                    const double* alpha, const double* beta,
                    const double* initial_state, double* final_state, double* o,
                    const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                    int32_t dk, int32_t dv, int32_t num_seqs,
                    const int32_t* chains, int32_t num_chains, int32_t nthreads)
{
    const shape_t s = {B, T, H, dk, dv, cu_seqlens ? num_seqs : B, cu_seqlens};
    if (check_shape(&s) || !q || !k || !v || !alpha || !beta || !o) return -1;
    const int nt = pick_threads(nthreads);
    CHAIN_LOOP(relative_chain(&s, n, h, 0, q, k, v, alpha, beta, initial_state, final_state, o));
    return 0;
}

int gdn2_oracle_gdn(const double* q, const double* k, const double* v,
                    const double* alpha, const double* beta,
                    const double* initial_state, double* final_state, double* o,
                    const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                    int32_t dk, int32_t dv, int32_t num_seqs,
                    const int32_t* chains, int32_t num_chains, int32_t nthreads)
{
    const shape_t s = {B, T, H, dk, dv, cu_seqlens ? num_seqs : B, cu_seqlens};
    if (check_shape(&s) || !q || !k || !v || !alpha || !beta || !o) return -1;
    const int nt = pick_threads(nthreads);
    CHAIN_LOOP(relative_chain(&s, n, h, 1, q, k, v, alpha, beta, initial_state, final_state, o));
    return 0;
}

int gdn2_oracle_backward(const double* q, const double* k, const double* v,
                         const double* alpha, const double* b, const double* w,
                         const double* initial_state, const double* d_o, const double* d_final_state,
                         double* dq, double* dk, double* dv, double* dalpha, double* db, double* dw,
                         double* d_initial_state,
                         const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                         int32_t dk_, int32_t dv_, int32_t num_seqs,
                         const int32_t* chains, int32_t num_chains, int32_t nthreads)
{
    const shape_t s = {B, T, H, dk_, dv_, cu_seqlens ? num_seqs : B, cu_seqlens};
    if (check_shape(&s) || !q || !k || !v || !alpha || !b || !w || !d_o) return -1;
    if (!dq || !dk || !dv || !dalpha || !db || !dw) return -1;
    const int nt = pick_threads(nthreads);
    CHAIN_LOOP(backward_chain(&s, n, h, q, k, v, alpha, b, w, initial_state, d_o, d_final_state,
                              dq, dk, dv, dalpha, db, dw, d_initial_state));
    return 0;
}

int gdn2_oracle_max_threads(void)
{
    return pick_threads(0);
}
