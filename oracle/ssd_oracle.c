/*
 * ssd_oracle.c -- plain, slow CPU oracle for the Mamba-2 SSD layer scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only tests/, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * Everything is double precision.  Inputs are the exact values handed to the
 * GPU (bf16 and fp32 widen to fp64 without rounding).  No blocking, no
 * chunking, no re-association: the recurrence is evaluated token by token.
 *
 * Sources (arXiv 2603.09555, C. Santoni, "Compiler-First State Space Duality
 * and Portable O(1) Autoregressive Caching for Inference"):
 *   - abstract: per-head diagonal dynamics; prefill and O(1) cached decode
 *     compute the same recurrence.
 *   - bqwf.cn article on the compiler-first Mamba-2 implementation:
 *       §1.1  diagonal state matrix, so the update splits into independent
 *             scalar operations per head; discretised decay exp(A*dt) (the
 *             printed formula lost the minus sign of A, see oracle_ssd_scan);
 *       §2.1  state h in R^{H x P x N} per layer and a (K-1)-token input
 *             window for the depthwise convolution;
 *       §2.2  the cache update: conv window rolled by one with the newest
 *             token written last; state = state * A_bar + B_bar * input.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Sequential SSD recurrence                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    int B, L, H, P, G, N;
    const double *x, *dt, *A_log, *Bm, *Cm, *D, *init_state;
    double *y, *final_state;
    int nthreads, tid;
} scan_args;

/*
 * One (b, h) pair, tokens in order.  For head h with A = -exp(A_log[h]):
 *   decay_t   = exp(dt[b,t,h] * A)                     (bqwf.cn §1.1, §4.1)
 *   S[p][n]  <- decay_t * S[p][n] + dt[b,t,h] * x[b,t,h,p] * Bm[b,t,g,n]
 *                                                     (bqwf.cn §2.2 update)
 *   y[b,t,h,p] = sum_n Cm[b,t,g,n] * S[p][n] + D[h] * x[b,t,h,p]
 * The state is laid out [P][N] (outer product x (x) B); the readout
 * contracts over N, as the intra-chunk einsum of bqwf.cn §1.2 contracts C
 * against B over the state index n.  g = h / (H / G).
 */
static void scan_one(const scan_args *a, int b, int h, double *S)
{
    const int L = a->L, H = a->H, P = a->P, G = a->G, N = a->N;
    const int g = h / (H / G);
    const double A = -exp(a->A_log[h]);
    const double Dh = a->D ? a->D[h] : 0.0;
    const size_t PN = (size_t)P * N;

    if (a->init_state)
        memcpy(S, a->init_state + ((size_t)b * H + h) * PN, PN * sizeof(double));
    else
        memset(S, 0, PN * sizeof(double));

    for (int t = 0; t < L; ++t) {
        const size_t bt = (size_t)b * L + t;
        const double dtv = a->dt[bt * H + h];
        const double decay = exp(dtv * A);
        const double *xv = a->x + (bt * H + h) * P;
        const double *Bv = a->Bm + (bt * G + g) * N;
        const double *Cv = a->Cm + (bt * G + g) * N;
        double *yv = a->y ? a->y + (bt * H + h) * P : NULL;
        for (int p = 0; p < P; ++p) {
            double *row = S + (size_t)p * N;
            const double coef = dtv * xv[p];
            for (int n = 0; n < N; ++n)
                row[n] = decay * row[n] + coef * Bv[n];
        }
        if (yv) {
            for (int p = 0; p < P; ++p) {
                const double *row = S + (size_t)p * N;
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += Cv[n] * row[n];
                yv[p] = acc + Dh * xv[p];
            }
        }
    }
    if (a->final_state)
        memcpy(a->final_state + ((size_t)b * a->H + h) * PN, S, PN * sizeof(double));
}

static void *scan_worker(void *arg)
{
    const scan_args *a = (const scan_args *)arg;
    double *S = (double *)malloc((size_t)a->P * a->N * sizeof(double));
    if (!S) return (void *)1;
    const int pairs = a->B * a->H;
    for (int i = a->tid; i < pairs; i += a->nthreads)
        scan_one(a, i / a->H, i % a->H, S);
    free(S);
    return NULL;
}

/*
 * y: [B,L,H,P] (nullable: state only), final_state: [B,H,P,N] (nullable).
 * x: [B,L,H,P], dt: [B,L,H], A_log: [H], Bm/Cm: [B,L,G,N], D: [H] (nullable
 * means 0), init_state: [B,H,P,N] (nullable means 0).  All row-major.
 * Threads split the independent (b, h) pairs, which cannot change any value.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_ssd_scan(int B, int L, int H, int P, int G, int N,
                    const double *x, const double *dt, const double *A_log,
                    const double *Bm, const double *Cm, const double *D,
                    const double *init_state, double *y, double *final_state,
                    int nthreads)
{
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G) return -1;
    if (!A_log || (L > 0 && (!x || !dt || !Bm || !Cm))) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B * H) nthreads = B * H > 0 ? B * H : 1;

    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    scan_args *args = (scan_args *)malloc(sizeof(scan_args) * nthreads);
    if (!th || !args) { free(th); free(args); return -1; }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        scan_args s = {B, L, H, P, G, N, x, dt, A_log, Bm, Cm, D, init_state,
                       y, final_state, nthreads, i};
        args[i] = s;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, scan_worker, &args[i]) != 0) { rc = -1; break; }
        started = i;
    }
    if (scan_worker(&args[0]) != NULL) rc = -1;
    for (int i = 1; i <= started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = -1;
    }
    if (rc == 0 && started != nthreads - 1) {
        /* thread creation failed part-way: finish the missing shares here */
        for (int i = started + 1; i < nthreads; ++i)
            if (scan_worker(&args[i]) != NULL) rc = -1;
    }
    free(th);
    free(args);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Depthwise causal convolution with a (K-1)-token window cache              */
/* ------------------------------------------------------------------------ */

/*
 * conv_state: [B,C,K-1], index 0 the oldest cached input, K-2 the newest
 * (bqwf.cn §2.2: roll by -1 along the last axis, then write the new token at
 * index -1).  For each channel c and each new token u_t:
 *   window   = (conv_state[b,c,0..K-2], u_t)
 *   v        = bias[c] + sum_k w[c,k] * window[k]      (window[K-1] newest)
 *   out[b,t,c] = silu(v) = v / (1 + exp(-v)) if activation, else v
 *   conv_state[b,c,:] = window[1..K-1]
 * conv_state is updated in place.  xBC/out: [B,T,C], w: [C,K], bias: [C]
 * (nullable).  out may be NULL (state only).
 */
int oracle_conv_update(int B, int T, int C, int K, double *conv_state,
                       const double *xBC, const double *w, const double *bias,
                       int activation, double *out)
{
    if (B < 0 || T < 0 || C <= 0 || K < 2 || !conv_state || !w) return -1;
    if (T > 0 && !xBC) return -1;
    double *win = (double *)malloc(sizeof(double) * K);
    if (!win) return -1;
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < C; ++c) {
            double *st = conv_state + ((size_t)b * C + c) * (K - 1);
            for (int t = 0; t < T; ++t) {
                const size_t idx = ((size_t)b * T + t) * C + c;
                for (int k = 0; k < K - 1; ++k) win[k] = st[k];
                win[K - 1] = xBC[idx];
                double v = bias ? bias[c] : 0.0;
                for (int k = 0; k < K; ++k) v += w[(size_t)c * K + k] * win[k];
                if (activation) v = v / (1.0 + exp(-v));
                if (out) out[idx] = v;
                for (int k = 0; k < K - 1; ++k) st[k] = win[k + 1];
            }
        }
    }
    free(win);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Step-size preprocessing                                                   */
/* ------------------------------------------------------------------------ */

/*
 * The chain that bqwf.cn §1.2 names before the decay (softplus, then clip,
 * then exp), as the step size is formed from a raw projection:
 *   u        = dt_raw[i] + dt_bias[h]          (bias 0 when absent)
 *   dt[i]    = min(max(softplus(u), dt_min), dt_max)
 *   softplus(u) = log(1 + exp(u)), written max(u, 0) + log1p(exp(-|u|)) so
 *   that it neither overflows nor loses the small tail for large |u|.
 * dt_raw and dt are [n, H] (h = i % H).  dt_max may be +inf.
 */
int oracle_dt_from_raw(long n, int H, const double *dt_raw, const double *dt_bias,
                       double dt_min, double dt_max, double *dt)
{
    if (n < 0 || H <= 0 || !dt_raw || !dt || !(dt_min <= dt_max)) return -1;
    for (long i = 0; i < n * H; ++i) {
        const double u = dt_raw[i] + (dt_bias ? dt_bias[i % H] : 0.0);
        const double sp = (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u)));
        dt[i] = fmin(fmax(sp, dt_min), dt_max);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Output side of the mixer: gated RMS normalisation                        */
/* ------------------------------------------------------------------------ */

/*
 * The normalisation that closes the layer (bqwf.cn §3.2 fuses it into its
 * neighbours; §4.1 asks for its variance in at least fp32), in the gated
 * RMS form of the Mamba-2 mixer: the scan output is gated by the z branch,
 * then each group of `group` consecutive channels is scaled to unit RMS and
 * by a per-channel weight.  For row r and channel c of group k:
 *   g[c]     = y[r,c] * silu(z[r,c])        (g = y when z is NULL)
 *   ms_k     = (1/group) * sum over the group of g[c]^2
 *   out[r,c] = g[c] / sqrt(ms_k + eps) * w[c]        (w = 1 when NULL)
 * y, z, out: [rows, D] (z with row stride z_stride); w: [D].
 */
int oracle_gated_rmsnorm(long rows, int D, int group, const double *y, const double *z, long z_stride,
                         const double *w, double eps, double *out)
{
    if (rows < 0 || D <= 0 || group <= 0 || D % group != 0 || !y || !out || !(eps >= 0.0)) return -1;
    double *g = (double *)malloc(sizeof(double) * group);
    if (!g) return -1;
    for (long r = 0; r < rows; ++r) {
        for (int k0 = 0; k0 < D; k0 += group) {
            double ss = 0.0;
            for (int j = 0; j < group; ++j) {
                const int c = k0 + j;
                double v = y[r * D + c];
                if (z) {
                    const double zz = z[r * z_stride + c];
                    v *= zz / (1.0 + exp(-zz));
                }
                g[j] = v;
                ss += v * v;
            }
            const double inv = 1.0 / sqrt(ss / group + eps);
            for (int j = 0; j < group; ++j)
                out[r * D + k0 + j] = g[j] * inv * (w ? w[k0 + j] : 1.0);
        }
    }
    free(g);
    return 0;
}
