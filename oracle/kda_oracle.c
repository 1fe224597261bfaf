/*
 * kda_oracle.c -- plain float64 CPU oracle for the Kimi Delta Attention (KDA)
 * forward pass.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * in __graft_entry__.py and the cpu_baseline leg of bench.py may load or call
 * this library.  The GPU library (libkda) never links, loads or calls it, and
 * the two share no source, header, table or helper.
 *
 * What it computes -- the KDA recurrence, per (sequence, head), token by token,
 * with the state S stored d_v x d_k (rows = value channels, columns = key
 * channels):
 *
 *   decay    S~_t  = S_{t-1} . Diag(alpha_t),   alpha_t = exp(log_alpha_t)
 *   predict  vh_t  = S~_t k_t
 *   error    e_t   = beta_t (v_t - vh_t)
 *   write    S_t   = S~_t + e_t k_t^T
 *   readout  o_t   = S_t q_t                      (post-write state, no scale)
 *
 * Sources:
 *   - "KDA derivation summary" page (hn.213312.xyz, article 49085909), sect. 3
 *     (predict / error / write of DeltaNet, state = sum of |v><k|, readout
 *     S_t|q_t>) and sect. 5 (KDA: the decay is S_{t-1} D_t, one forget rate per
 *     column = per key channel; the other steps as in Gated DeltaNet).
 *   - "Kimi K3 notes 1: KDA" page (jaimeyzzz.com), sect. 4 and the summary box
 *     of sect. 5 (same update in the transposed d_k x d_v orientation; q, k are
 *     L2-normalised by the caller).
 *
 * write_mode ADD replaces the error by the plain write e_t = beta_t v_t (linear
 * attention / GLA, "Linear/sparse attention tutorial" page, sect. 2.2 and 2.4);
 * it exists only so tests can pin the oracle against closed forms.
 *
 * Every step is written out as the definition states it: a full-matrix decay,
 * then the prediction vector, the error vector, the rank-1 write and the
 * readout.  No blocking, fusion or reordering.  Parallelism (OpenMP) is only
 * across independent (sequence, head) pairs.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { KDA_ORACLE_WRITE_DELTA = 0, KDA_ORACLE_WRITE_ADD = 1 };

/* Strides (in elements) of one head's token sequence inside a
 * [.., T, H, d] token-major tensor: consecutive tokens are H*d apart. */
typedef struct {
    const double *q, *k, *v, *log_alpha, *beta;
    double *out;
    long n_tokens;
    long tok_stride_k;   /* H * dk  (q, k, log_alpha) */
    long tok_stride_v;   /* H * dv  (v, out) */
    long tok_stride_b;   /* H       (beta) */
} head_view;

/* Runs the recurrence for one head over n_tokens tokens.  S (dv x dk,
 * row-major) holds the incoming state and receives the final state.
 * work must hold 2*dk + 2*dv doubles. */
static void head_recurrence(const head_view *hv, long dk, long dv, int write_mode,
                            double *S, double *work)
{
    double *alpha = work;           /* dk */
    double *vhat  = work + dk;      /* dv */
    double *err   = vhat + dv;      /* dv */
    for (long t = 0; t < hv->n_tokens; ++t) {
        const double *q  = hv->q + t * hv->tok_stride_k;
        const double *k  = hv->k + t * hv->tok_stride_k;
        const double *la = hv->log_alpha + t * hv->tok_stride_k;
        const double *v  = hv->v + t * hv->tok_stride_v;
        const double beta = hv->beta[t * hv->tok_stride_b];
        double *o = hv->out + t * hv->tok_stride_v;

        /* decay: S~ = S Diag(alpha) -- column c scaled by alpha_c */
        for (long c = 0; c < dk; ++c) alpha[c] = exp(la[c]);
        for (long i = 0; i < dv; ++i)
            for (long c = 0; c < dk; ++c) S[i * dk + c] *= alpha[c];

        /* predict: vh = S~ k */
        for (long i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (long c = 0; c < dk; ++c) acc += S[i * dk + c] * k[c];
            vhat[i] = acc;
        }

        /* error: e = beta (v - vh); plain write for the additive mode */
        for (long i = 0; i < dv; ++i)
            err[i] = (write_mode == KDA_ORACLE_WRITE_ADD) ? beta * v[i]
                                                          : beta * (v[i] - vhat[i]);

        /* write: S = S~ + e k^T */
        for (long i = 0; i < dv; ++i)
            for (long c = 0; c < dk; ++c) S[i * dk + c] += err[i] * k[c];

        /* readout: o = S q */
        for (long i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (long c = 0; c < dk; ++c) acc += S[i * dk + c] * q[c];
            o[i] = acc;
        }
    }
}

static int check_dims(long H, long dk, long dv, int write_mode)
{
    if (H <= 0 || dk <= 0 || dv <= 0) return 2;
    if (write_mode != KDA_ORACLE_WRITE_DELTA && write_mode != KDA_ORACLE_WRITE_ADD) return 3;
    return 0;
}

/*
 * Dense batch.  Layouts (row-major, d fastest):
 *   q, k, log_alpha [B, T, H, dk];  v, out [B, T, H, dv];  beta [B, T, H];
 *   S0, S_final [B, H, dv, dk].
 * S0 == NULL means a zero initial state; S_final == NULL means "not written".
 * S_final may alias S0.  Returns 0 on success, nonzero on bad arguments or
 * allocation failure.
 */
int kda_oracle_forward(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const double *S0, double *out, double *S_final,
                       long B, long T, long H, long dk, long dv, int write_mode)
{
    int rc = check_dims(H, dk, dv, write_mode);
    if (rc) return rc;
    if (B < 0 || T < 0) return 2;
    if (!q || !k || !v || !log_alpha || !beta || (!out && B * T > 0)) return 1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
    for (long bh = 0; bh < B * H; ++bh) {
        long b = bh / H, h = bh % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dv * dk + 2 * dk + 2 * dv));
        if (!S) { failed = 1; continue; }
        double *work = S + dv * dk;
        if (S0) memcpy(S, S0 + bh * dv * dk, sizeof(double) * (size_t)(dv * dk));
        else memset(S, 0, sizeof(double) * (size_t)(dv * dk));
        head_view hv;
        hv.q = q + (b * T * H + h) * dk;
        hv.k = k + (b * T * H + h) * dk;
        hv.log_alpha = log_alpha + (b * T * H + h) * dk;
        hv.v = v + (b * T * H + h) * dv;
        hv.out = out ? out + (b * T * H + h) * dv : NULL;
        hv.beta = beta + b * T * H + h;
        hv.n_tokens = T;
        hv.tok_stride_k = H * dk;
        hv.tok_stride_v = H * dv;
        hv.tok_stride_b = H;
        head_recurrence(&hv, dk, dv, write_mode, S, work);
        if (S_final) memcpy(S_final + bh * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        free(S);
    }
    return failed ? 4 : 0;
}

/*
 * Packed variable-length batch: N sequences concatenated along the token axis
 * of [1, T_total, H, d] tensors; sequence n owns tokens
 * [cu_seqlens[n], cu_seqlens[n+1]).  Each sequence starts from its own state
 * S0[n] (or zero) and writes S_final[n]; layouts [N, H, dv, dk].
 */
int kda_oracle_forward_varlen(const double *q, const double *k, const double *v,
                              const double *log_alpha, const double *beta,
                              const double *S0, double *out, double *S_final,
                              const int *cu_seqlens, long N, long T_total,
                              long H, long dk, long dv, int write_mode)
{
    int rc = check_dims(H, dk, dv, write_mode);
    if (rc) return rc;
    if (N < 0 || T_total < 0 || !cu_seqlens) return 2;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_total) return 2;
    for (long n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
    for (long nh = 0; nh < N * H; ++nh) {
        long n = nh / H, h = nh % H;
        long t0 = cu_seqlens[n];
        double *S = (double *)malloc(sizeof(double) * (size_t)(dv * dk + 2 * dk + 2 * dv));
        if (!S) { failed = 1; continue; }
        double *work = S + dv * dk;
        if (S0) memcpy(S, S0 + nh * dv * dk, sizeof(double) * (size_t)(dv * dk));
        else memset(S, 0, sizeof(double) * (size_t)(dv * dk));
        head_view hv;
        hv.q = q + (t0 * H + h) * dk;
        hv.k = k + (t0 * H + h) * dk;
        hv.log_alpha = log_alpha + (t0 * H + h) * dk;
        hv.v = v + (t0 * H + h) * dv;
        hv.out = out + (t0 * H + h) * dv;
        hv.beta = beta + t0 * H + h;
        hv.n_tokens = cu_seqlens[n + 1] - t0;
        hv.tok_stride_k = H * dk;
        hv.tok_stride_v = H * dv;
        hv.tok_stride_b = H;
        head_recurrence(&hv, dk, dv, write_mode, S, work);
        if (S_final) memcpy(S_final + nh * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        free(S);
    }
    return failed ? 4 : 0;
}

/* Threads an OpenMP parallel region of this library will use. */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void kda_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
