/*
 * Finch WKV recurrence -- plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  The GPU
 * library shares no code, header or constant with it.
 *
 * What it computes (GoldFinch architecture summary page, section 3.4
 * "Finch-C2 Time Mixing", paragraph "Recurrent state update and output"):
 *
 *   wkv_t = sum_{i<t} diag( prod_{j=i+1}^{t-1} w_j ) k_i^T v_i
 *
 * a D x D state per (sequence, head) whose ROWS are key channels (the decay
 * acts on the rows of the outer product through the diagonal matrix) and
 * whose columns are value channels.  Evaluated as the equivalent recurrence
 *
 *   S_t = diag(w_t) S_{t-1} + k_t^T v_t ,     wkv_t = S_{t-1},
 *
 * with a carried-in state S_0 (zeros when none is given).  The read-out is
 * base Finch's (the static per-channel bonus u that section 3.4 lists as
 * modification (4), i.e. the term Finch-C2 later replaces):
 *
 *   o_t[j] = sum_i r_t[i] * ( S_{t-1}[i][j] + u[i] * k_t[i] * v_t[j] ).
 *
 * Two further forms from the same section are selectable:
 *
 * - decay given as d_t (paragraph "Data-dependent decay"): the caller passes
 *   d_t and the weight is w_t = exp(-exp(d_t)), formed here in double;
 * - the Finch-C2 time mixer (paragraphs "Key computation with normalization
 *   property", "Receptance, value, and the new second value" and the output
 *   equation): the key that enters the state is the given key times
 *   (1 - w_t); there is no static bonus; the data-dependent second value u'_t
 *   is added to the read-out,
 *
 *     o_t[j] = sum_i r_t[i] * S_{t-1}[i][j] + u'_t[j],
 *     S_t    = diag(w_t) S_{t-1} + (k_t * (1 - w_t))^T v_t .
 *
 *   With no u' given the term is absent (the pages' ablation "Finch-C2
 *   without second value").
 *
 * Every input value is the exact value the GPU receives (bf16 bit patterns or
 * fp32), widened exactly to double.  No blocking, no reordering: one token at
 * a time, in order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_DECAY_W = 0, ORACLE_DECAY_LOG = 1 };   /* w_t given, or d_t with w_t = exp(-exp(d_t)) */
enum { ORACLE_FINCH = 0, ORACLE_FINCH_C2 = 1 };

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t x = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &x, sizeof f);
    return (double)f;
}

static double load_value(int kind, const void *base, int64_t idx)
{
    if (kind == ORACLE_BF16)
        return bf16_bits_to_double(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/*
 * One (sequence n, head h) slice: tokens [t0, t1) of the packed [tokens, H, D]
 * tensors.  S is D x D, row = key channel i, column = value channel j.
 */
static void scan_slice(int kind, int decay_kind, int variant,
                       const void *r, const void *k, const void *v,
                       const void *w, const float *u, const void *u2,
                       const double *state_in,
                       int64_t t0, int64_t t1, int64_t n, int h, int H, int D,
                       double *o, double *state_out)
{
    double *S = (double *)calloc((size_t)D * D, sizeof(double));
    double *rt = (double *)malloc((size_t)D * sizeof(double));
    double *kt = (double *)malloc((size_t)D * sizeof(double));
    double *vt = (double *)malloc((size_t)D * sizeof(double));
    double *wt = (double *)malloc((size_t)D * sizeof(double));
    double *ud = (double *)malloc((size_t)D * sizeof(double));
    if (!S || !rt || !kt || !vt || !wt || !ud) abort();

    for (int i = 0; i < D; ++i) ud[i] = variant == ORACLE_FINCH ? (double)u[(int64_t)h * D + i] : 0.0;
    if (state_in) {
        const double *s0 = state_in + ((n * H + h) * (int64_t)D * D);
        memcpy(S, s0, (size_t)D * D * sizeof(double));
    }

    for (int64_t t = t0; t < t1; ++t) {
        int64_t base = (t * H + h) * (int64_t)D;
        for (int i = 0; i < D; ++i) {
            rt[i] = load_value(kind, r, base + i);
            kt[i] = load_value(kind, k, base + i);
            vt[i] = load_value(kind, v, base + i);
            wt[i] = load_value(kind, w, base + i);
        }
        if (decay_kind == ORACLE_DECAY_LOG)          /* the input holds d_t */
            for (int i = 0; i < D; ++i) wt[i] = exp(-exp(wt[i]));
        if (variant == ORACLE_FINCH_C2)              /* key-decay multiplication */
            for (int i = 0; i < D; ++i) kt[i] = kt[i] * (1.0 - wt[i]);
        /* read-out from the state before this token, plus the bonus term */
        if (o && variant == ORACLE_FINCH_C2) {
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int i = 0; i < D; ++i)
                    acc += rt[i] * S[i * D + j];
                if (u2) acc += load_value(kind, u2, base + j);   /* second value u'_t */
                o[base + j] = acc;
            }
        } else if (o) {
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int i = 0; i < D; ++i)
                    acc += rt[i] * (S[i * D + j] + ud[i] * kt[i] * vt[j]);
                o[base + j] = acc;
            }
        }
        /* state update: decay rows by w_t, add the outer product k_t^T v_t */
        for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j)
                S[i * D + j] = wt[i] * S[i * D + j] + kt[i] * vt[j];
    }

    if (state_out) {
        double *so = state_out + ((n * H + h) * (int64_t)D * D);
        memcpy(so, S, (size_t)D * D * sizeof(double));
    }
    free(S); free(rt); free(kt); free(vt); free(wt); free(ud);
}

/*
 * Packed-sequence entry point.
 *   kind        ORACLE_F32 or ORACLE_BF16 (r, k, v, w, u2 element type)
 *   decay_kind  ORACLE_DECAY_W (w holds w_t) or ORACLE_DECAY_LOG (w holds d_t)
 *   variant     ORACLE_FINCH (bonus u) or ORACLE_FINCH_C2 (u unused, may be
 *               NULL; u2 = second value u'_t [total_tokens, H, D] or NULL)
 *   r,k,v,w     [total_tokens, H, D] packed rows of all N sequences
 *   u           [H, D] fp32 bonus
 *   state_in    [N, H, D, D] fp64 or NULL (zeros); callers widen fp32
 *               states exactly, and a carried fp64 state stays exact
 *   cu_seqlens  [N + 1] token offsets, cu_seqlens[0] == 0, non-decreasing
 *   slice_mask  [N * H] bytes, non-zero = compute this (n, h); NULL = all
 *   o           [total_tokens, H, D] fp64 output or NULL (only masked slices
 *               are written)
 *   state_out   [N, H, D, D] fp64 output or NULL
 *   threads     OpenMP threads (<= 0: library default)
 * Returns 0, or -1 on an inconsistent offsets array.
 */
int oracle_wkv_f64_ex(int kind, int decay_kind, int variant,
                      const void *r, const void *k, const void *v,
                      const void *w, const float *u, const void *u2,
                      const double *state_in,
                      const int64_t *cu_seqlens, int64_t N, int H, int D,
                      const uint8_t *slice_mask, double *o, double *state_out,
                      int threads)
{
    if (decay_kind != ORACLE_DECAY_W && decay_kind != ORACLE_DECAY_LOG) return -1;
    if (variant != ORACLE_FINCH && variant != ORACLE_FINCH_C2) return -1;
    if (cu_seqlens[0] != 0) return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

    int64_t slices = N * (int64_t)H;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t s = 0; s < slices; ++s) {
        if (slice_mask && !slice_mask[s]) continue;
        int64_t n = s / H;
        int h = (int)(s % H);
        scan_slice(kind, decay_kind, variant, r, k, v, w, u, u2, state_in,
                   cu_seqlens[n], cu_seqlens[n + 1], n, h, H, D, o, state_out);
    }
    (void)threads;
    return 0;
}

/* base Finch with w_t given: oracle_wkv_f64_ex(kind, ORACLE_DECAY_W, ORACLE_FINCH, ..., u2 = NULL, ...) */
int oracle_wkv_f64(int kind, const void *r, const void *k, const void *v,
                   const void *w, const float *u, const double *state_in,
                   const int64_t *cu_seqlens, int64_t N, int H, int D,
                   const uint8_t *slice_mask, double *o, double *state_out,
                   int threads)
{
    return oracle_wkv_f64_ex(kind, ORACLE_DECAY_W, ORACLE_FINCH, r, k, v, w, u, NULL,
                             state_in, cu_seqlens, N, H, D, slice_mask, o, state_out,
                             threads);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
