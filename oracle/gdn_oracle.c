/*
 * Reference oracle for the Gated DeltaNet gated-delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU product
 * path never calls it, and the two share no source.
 *
 * Everything here runs in IEEE double precision on the CPU, one plain loop
 * after another, with no blocking, fusion or reordering beyond what the
 * definitions below state.  Work is split over independent (sequence, v-head)
 * units with OpenMP.  That split does not change the arithmetic of any unit.
 *
 * Source of the method: "Optimizing on-device inference for Apple Silicon"
 * (Perplexity blog, 2026), section "Qwen creates three distinct workload
 * shapes".  It describes a Gated DeltaNet layer as a fixed-size recurrent
 * state.  A learned gate decides how much of the state to keep, and a delta
 * update writes in the current token.  The layer can be evaluated token by
 * token or reorganised into blocks.  The same post ("Keep the recurrent state
 * on chip") keeps that state in fp32.  The page prints no formula, so the
 * update written out here is the standard gated delta rule:
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with S_t a d_v x d_k matrix per (sequence, v-head), alpha_t = exp(g_t), and
 * q_t, k_t optionally L2-normalised per token and head:
 * x / sqrt(sum x^2 + 1e-6).  The query is then multiplied by `scale`.
 *
 * Conventions:
 *   - v-head h reads q/k head h / (h_v / h_k): consecutive v-heads share a
 *     k-head (grouped-query sharing).
 *   - Packed layout: q, k [T, h_k, d_k]; v, out [T, h_v, d_v];
 *     g, beta [T, h_v]; state [N, h_v, d_v, d_k], row-major, one row per
 *     value index.
 *   - cu_seqlens [N+1] gives the packed token range of each sequence.  NULL
 *     means one sequence covering all T tokens.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GDN_EPS 1e-6

/* L2 normalisation of one head's vector, as the layer description uses it
 * for queries and keys.  Off: the vector is copied through. */
static void prep_vec(const double *x, int d, int l2norm, double mul, double *out)
{
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += x[i] * x[i];
    double r = l2norm ? 1.0 / sqrt(ss + GDN_EPS) : 1.0;
    for (int i = 0; i < d; ++i) out[i] = x[i] * r * mul;
}

static void seq_range(const int32_t *cu, int n, int64_t T, int64_t *b, int64_t *e)
{
    if (!cu) { *b = 0; *e = T; return; }
    *b = cu[n];
    *e = cu[n + 1];
}

/*
 * The direct token scan: the definition of the recurrence, applied one token
 * at a time ("evaluate the recurrence directly" in the workload-shapes
 * section).  For every token, with the previous state S:
 *     S <- alpha S (I - beta k k^T) + beta v k^T,   o = S q
 * expanded without forming the d_k x d_k matrix:
 *     S k is formed first; S <- alpha S - alpha beta (S k) k^T + beta v k^T.
 */
int gdn_oracle_scan(int32_t num_seqs, int64_t total_tokens, const int32_t *cu_seqlens,
                    int32_t h_k, int32_t h_v, int32_t d_k, int32_t d_v,
                    int32_t qk_l2norm, double scale,
                    const double *q, const double *k, const double *v,
                    const double *g, const double *beta,
                    const double *state_in, double *out, double *state_out,
                    int32_t nthreads)
{
    if (num_seqs < 1 || h_k < 1 || h_v < 1 || h_v % h_k || d_k < 1 || d_v < 1) return 1;
    if (!cu_seqlens && num_seqs != 1) return 1;
    const int r = h_v / h_k;
    const int64_t units = (int64_t)num_seqs * h_v;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int n = (int)(unit / h_v), h = (int)(unit % h_v), hk = h / r;
        int64_t b, e;
        seq_range(cu_seqlens, n, total_tokens, &b, &e);
        if (b < 0 || e < b || e > total_tokens) { bad |= 1; continue; }
        double *S = (double *)malloc(sizeof(double) * (size_t)d_v * d_k);
        double *kh = (double *)malloc(sizeof(double) * (size_t)d_k);
        double *qh = (double *)malloc(sizeof(double) * (size_t)d_k);
        double *Sk = (double *)malloc(sizeof(double) * (size_t)d_v);
        const size_t soff = ((size_t)n * h_v + h) * (size_t)d_v * d_k;
        for (size_t i = 0; i < (size_t)d_v * d_k; ++i) S[i] = state_in ? state_in[soff + i] : 0.0;
        for (int64_t t = b; t < e; ++t) {
            prep_vec(k + ((size_t)t * h_k + hk) * d_k, d_k, qk_l2norm, 1.0, kh);
            prep_vec(q + ((size_t)t * h_k + hk) * d_k, d_k, qk_l2norm, scale, qh);
            const double alpha = exp(g[(size_t)t * h_v + h]);
            const double bt = beta[(size_t)t * h_v + h];
            const double *vt = v + ((size_t)t * h_v + h) * d_v;
            for (int i = 0; i < d_v; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d_k; ++j) acc += S[(size_t)i * d_k + j] * kh[j];
                Sk[i] = acc;
            }
            for (int i = 0; i < d_v; ++i)
                for (int j = 0; j < d_k; ++j) {
                    double *s = &S[(size_t)i * d_k + j];
                    *s = alpha * *s - alpha * bt * Sk[i] * kh[j] + bt * vt[i] * kh[j];
                }
            double *ot = out + ((size_t)t * h_v + h) * d_v;
            for (int i = 0; i < d_v; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d_k; ++j) acc += S[(size_t)i * d_k + j] * qh[j];
                ot[i] = acc;
            }
        }
        if (state_out)
            for (size_t i = 0; i < (size_t)d_v * d_k; ++i) state_out[soff + i] = S[i];
        free(S); free(kh); free(qh); free(Sk);
    }
    return bad ? 1 : 0;
}

/*
 * The blocked ("chunked") evaluation of the same recurrence.  The workload
 * section says the updates can be regrouped into blocks that expose matrix
 * work.  This is that regrouping, derived from the update above.  It is an
 * exact algebraic identity, so in exact arithmetic it equals the scan.
 * Here it serves only to check the identity the GPU kernels rely on.
 *
 * For one block of n tokens with block-initial state S (d_v x d_k), K and Q
 * hold the prepared keys and queries as rows (n x d_k), and V the values
 * (n x d_v):
 *   G_i  = g_1 + ... + g_i          (cumulative log-decay inside the block)
 *   A_ij = beta_i exp(G_i - G_j) k_i.k_j    for i > j, else 0
 *   T    = (I + A)^{-1} diag(beta)            (unit lower-triangular solve)
 *   W    = T diag(exp(G)) K,   Ut = T V
 *   U    = Ut - W S^T                          (the block's delta terms)
 *   P_ij = exp(G_i - G_j) q_i.k_j     for i >= j, else 0
 *   O    = diag(exp(G)) Q S^T + P U
 *   S'   = exp(G_n) S + U^T diag(exp(G_n - G)) K
 * Derivation: with u_t = beta_t (v_t - alpha_t S_{t-1} k_t), the update reads
 * S_t = alpha_t S_{t-1} + u_t k_t^T.  Unrolling inside the block gives
 * S_t = exp(G_t) S + sum_{j<=t} exp(G_t - G_j) u_j k_j^T.  Substituting this
 * into u_t gives the triangular system (I + A) U = diag(beta)(V - diag(exp G) K S^T).
 * The triangular solve is plain forward substitution.
 */
int gdn_oracle_chunked(int32_t num_seqs, int64_t total_tokens, const int32_t *cu_seqlens,
                       int32_t h_k, int32_t h_v, int32_t d_k, int32_t d_v,
                       int32_t qk_l2norm, double scale,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       const double *state_in, double *out, double *state_out,
                       int32_t chunk, int32_t nthreads)
{
    if (num_seqs < 1 || h_k < 1 || h_v < 1 || h_v % h_k || d_k < 1 || d_v < 1 || chunk < 1) return 1;
    if (!cu_seqlens && num_seqs != 1) return 1;
    const int r = h_v / h_k, C = chunk;
    const int64_t units = (int64_t)num_seqs * h_v;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int n = (int)(unit / h_v), h = (int)(unit % h_v), hk = h / r;
        int64_t b, e;
        seq_range(cu_seqlens, n, total_tokens, &b, &e);
        if (b < 0 || e < b || e > total_tokens) { bad |= 1; continue; }
        const size_t dd = (size_t)d_v * d_k;
        double *S = malloc(sizeof(double) * dd), *Sn = malloc(sizeof(double) * dd);
        double *K = malloc(sizeof(double) * (size_t)C * d_k), *Q = malloc(sizeof(double) * (size_t)C * d_k);
        double *V = malloc(sizeof(double) * (size_t)C * d_v);
        double *G = malloc(sizeof(double) * C), *bt = malloc(sizeof(double) * C);
        double *A = malloc(sizeof(double) * (size_t)C * C), *T = malloc(sizeof(double) * (size_t)C * C);
        double *W = malloc(sizeof(double) * (size_t)C * d_k), *Ut = malloc(sizeof(double) * (size_t)C * d_v);
        double *U = malloc(sizeof(double) * (size_t)C * d_v), *P = malloc(sizeof(double) * (size_t)C * C);
        const size_t soff = ((size_t)n * h_v + h) * dd;
        for (size_t i = 0; i < dd; ++i) S[i] = state_in ? state_in[soff + i] : 0.0;
        for (int64_t c0 = b; c0 < e; c0 += C) {
            const int nt = (int)((e - c0) < C ? (e - c0) : C);
            double acc = 0.0;
            for (int i = 0; i < nt; ++i) {
                const int64_t t = c0 + i;
                prep_vec(k + ((size_t)t * h_k + hk) * d_k, d_k, qk_l2norm, 1.0, K + (size_t)i * d_k);
                prep_vec(q + ((size_t)t * h_k + hk) * d_k, d_k, qk_l2norm, scale, Q + (size_t)i * d_k);
                for (int j = 0; j < d_v; ++j) V[(size_t)i * d_v + j] = v[((size_t)t * h_v + h) * d_v + j];
                acc += g[(size_t)t * h_v + h];
                G[i] = acc;
                bt[i] = beta[(size_t)t * h_v + h];
            }
            /* A and P */
            for (int i = 0; i < nt; ++i)
                for (int j = 0; j < nt; ++j) {
                    double kk = 0.0, qk = 0.0;
                    for (int x = 0; x < d_k; ++x) {
                        kk += K[(size_t)i * d_k + x] * K[(size_t)j * d_k + x];
                        qk += Q[(size_t)i * d_k + x] * K[(size_t)j * d_k + x];
                    }
                    const double dec = (j <= i) ? exp(G[i] - G[j]) : 0.0;
                    A[(size_t)i * C + j] = (j < i) ? bt[i] * dec * kk : 0.0;
                    P[(size_t)i * C + j] = (j <= i) ? dec * qk : 0.0;
                }
            /* T = (I + A)^{-1} diag(beta): forward substitution, column by column of the identity */
            for (int col = 0; col < nt; ++col)
                for (int i = 0; i < nt; ++i) {
                    double x = (i == col) ? 1.0 : 0.0;
                    for (int j = 0; j < i; ++j) x -= A[(size_t)i * C + j] * T[(size_t)j * C + col];
                    T[(size_t)i * C + col] = x;
                }
            for (int i = 0; i < nt; ++i)
                for (int col = 0; col < nt; ++col) T[(size_t)i * C + col] *= bt[col];
            /* W = T diag(exp G) K ; Ut = T V */
            for (int i = 0; i < nt; ++i) {
                for (int x = 0; x < d_k; ++x) {
                    double s = 0.0;
                    for (int j = 0; j < nt; ++j) s += T[(size_t)i * C + j] * exp(G[j]) * K[(size_t)j * d_k + x];
                    W[(size_t)i * d_k + x] = s;
                }
                for (int x = 0; x < d_v; ++x) {
                    double s = 0.0;
                    for (int j = 0; j < nt; ++j) s += T[(size_t)i * C + j] * V[(size_t)j * d_v + x];
                    Ut[(size_t)i * d_v + x] = s;
                }
            }
            /* U = Ut - W S^T */
            for (int i = 0; i < nt; ++i)
                for (int x = 0; x < d_v; ++x) {
                    double s = Ut[(size_t)i * d_v + x];
                    for (int y = 0; y < d_k; ++y) s -= W[(size_t)i * d_k + y] * S[(size_t)x * d_k + y];
                    U[(size_t)i * d_v + x] = s;
                }
            /* O = diag(exp G) Q S^T + P U */
            for (int i = 0; i < nt; ++i)
                for (int x = 0; x < d_v; ++x) {
                    double s1 = 0.0, s2 = 0.0;
                    for (int y = 0; y < d_k; ++y) s1 += Q[(size_t)i * d_k + y] * S[(size_t)x * d_k + y];
                    for (int j = 0; j < nt; ++j) s2 += P[(size_t)i * C + j] * U[(size_t)j * d_v + x];
                    out[((size_t)(c0 + i) * h_v + h) * d_v + x] = exp(G[i]) * s1 + s2;
                }
            /* S' = exp(G_n) S + U^T diag(exp(G_n - G)) K */
            const double gn = G[nt - 1];
            for (int x = 0; x < d_v; ++x)
                for (int y = 0; y < d_k; ++y) {
                    double s = exp(gn) * S[(size_t)x * d_k + y];
                    for (int j = 0; j < nt; ++j) s += U[(size_t)j * d_v + x] * exp(gn - G[j]) * K[(size_t)j * d_k + y];
                    Sn[(size_t)x * d_k + y] = s;
                }
            memcpy(S, Sn, sizeof(double) * dd);
        }
        if (state_out) memcpy(state_out + soff, S, sizeof(double) * dd);
        free(S); free(Sn); free(K); free(Q); free(V); free(G); free(bt); free(A); free(T);
        free(W); free(Ut); free(U); free(P);
    }
    return bad ? 1 : 0;
}
