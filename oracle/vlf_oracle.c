/*
 * TEST INFRASTRUCTURE ONLY — the float64 CPU oracle for packed variable-length attention.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load or call this
 * file's library. It shares no code, header, table or helper with the HIP path, and the HIP
 * path never calls it.
 *
 * What it computes (hanzo-kernel 0.2.42, src/packed.rs: the module contract at the top of the
 * page, and the f64 composite `attend_ref` near its end):
 *
 *   qkv [T, 3*H*64]: row t holds token t's queries, then keys, then values, heads contiguous.
 *   cu  [S+1]:       sequence s owns tokens cu[s] .. cu[s+1]-1; L_s = cu[s+1]-cu[s].
 *   cos, sin [P,32]: rotary tables indexed by position within a sequence.
 *
 * For a token t in sequence s at position i = t - cu[s], head h:
 *   rot(x, p)[m]    = x[m] c[p][m] - x[m+32] s[p][m]          (m < 32, half-split pairs)
 *   rot(x, p)[m+32] = x[m] s[p][m] + x[m+32] c[p][m]
 *   q_i = rot(Q row, i),  k_j = rot(K row, j),  v_j = V row        (all within head h)
 *   visible j:  0 <= j < L_s  and (W == 0 or |i - j| < W)
 *   score s_ij  = scale * <q_i, k_j>
 *   lse_i = m_i + ln(sum_j exp(s_ij - m_i)),  m_i = max_j s_ij        (natural log)
 *   out_i = sum_j exp(s_ij - lse_i) v_j
 *
 * W is the window value the kernel receives: 0 means every key of the sequence, W >= 1 means
 * |i - j| < W (the page passes its window option w as w + 1; its composite's |i-j| <= w is the
 * same set). With the flag CAUSAL_FLAG set in the window value, key j is visible to row i when
 * j <= i and, for W >= 1, i - j < W: the causal sliding window of the array library page.
 *
 * Two modes:
 *   mode A (0): the definition above, exactly, in float64.
 *   mode B (1): the operands rounded the way the page's kernel rounds them before its matrix
 *     products (the query-tile and key-tile loads of `attend`): each rotated element is formed
 *     in float32, the query element multiplied by `scale` in float32, and the result rounded
 *     to the storage type (bf16 or fp16, round-to-nearest-even). Scores are then the float64
 *     dot products of those rounded operands; everything after that is float64 as in mode A.
 *     Probabilities are not rounded: where the kernel rounds them depends on its key blocking.
 *
 * Inputs arrive as float32 arrays holding bf16/fp16 values (the widening is exact).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define HD 64   /* head dimension (the page fixes D = 64) */
#define HALF 32 /* rotation pairs (m, m + 32) */

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_MODE_A = 0, ORACLE_MODE_B = 1 };
#define CAUSAL_FLAG 0x40000000 /* set in the window value: the causal sliding window */

/*
 * Round a finite double to the nearest value with `p` significand bits and minimum normal
 * exponent `emin` (subnormals below it), ties to even; values at or beyond `max_finite` plus
 * half an ulp become infinity. This is IEEE round-to-nearest-even for a binary format, written
 * from the definition: scale the value so its ulp is 1, round to an integer with ties to even,
 * scale back.
 */
static double round_binary(double x, int p, int emin, double max_finite, int emax)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);    /* ax = f * 2^e with f in [0.5, 1): unbiased exponent is e - 1 */
    int ue = e - 1;
    if (ue < emin)
        ue = emin;    /* subnormal range: fixed ulp */
    double ulp = ldexp(1.0, ue - (p - 1));
    double q = ax / ulp; /* exact: a power-of-two scaling */
    double r = floor(q);
    double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    double y = r * ulp;
    /* overflow: anything that rounds above the largest finite value is infinite */
    double top = max_finite + 0.5 * ldexp(1.0, emax - (p - 1));
    if (ax >= top)
        y = INFINITY;
    else if (y > max_finite)
        y = max_finite;
    return x < 0 ? -y : y;
}

static double round_storage(double x, int dtype)
{
    if (dtype == ORACLE_BF16) /* 8 significand bits, float32's exponent range */
        return round_binary(x, 8, -126, 0x1.fep127, 127);
    /* fp16: 11 significand bits, exponents -14 .. 15 */
    return round_binary(x, 11, -14, 65504.0, 15);
}

/* Exposed so the tests can pin the rounding against library conversions. */
int vlf_oracle_round(const double *x, int64_t n, int32_t dtype, double *y)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        y[i] = round_storage(x[i], dtype);
    return 0;
}

/*
 * One head's 64-element row rotated to position `pos`.
 * Mode A: exact float64.
 * Mode B: each output formed as a single float32 rounding of x1*c -/+ x2*s (the two products of
 * storage-type values are exact, so fmaf over an exact product rounds once), then times
 * `scale` in float32 (pass 1 for keys), then rounded to the storage type.
 */
static void rotate_row(const float *x, const float *c, const float *s, int mode, int dtype,
                       float scale, double *y)
{
    for (int m = 0; m < HALF; ++m) {
        if (mode == ORACLE_MODE_A) {
            double x1 = x[m], x2 = x[m + HALF], cm = c[m], sm = s[m];
            y[m] = x1 * cm - x2 * sm;
            y[m + HALF] = x1 * sm + x2 * cm;
        } else {
            float a = fmaf(x[m], c[m], -(x[m + HALF] * s[m]));
            float b = fmaf(x[m], s[m], x[m + HALF] * c[m]);
            a = a * scale;
            b = b * scale;
            y[m] = round_storage((double)a, dtype);
            y[m + HALF] = round_storage((double)b, dtype);
        }
    }
}

/*
 * The score operands of every token and head, as the scores above use them: q_out [T, H*64] the
 * query rows rotated to their positions and scaled (mode A: scale * rot(q) in float64; mode B: the
 * rounded operand of rotate_row), k_out [T, H*64] the key rows rotated (mode B: rounded). The
 * gradient (oracle/__init__.py, attend_backward) is taken with respect to these. Returns 0, or -1
 * on malformed arguments.
 */
int vlf_oracle_operands(const float *qkv, const float *cos_t, const float *sin_t, int64_t P,
                        const int32_t *cu, int32_t S, int64_t T, int32_t H, double scale,
                        int32_t mode, int32_t dtype, double *q_out, double *k_out)
{
    if (S < 0 || T < 0 || H < 1 || P < 0)
        return -1;
    if (mode != ORACLE_MODE_A && mode != ORACLE_MODE_B)
        return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return -1;
    if (cu[0] != 0 || cu[S] != T)
        return -1;
    for (int32_t s = 0; s < S; ++s)
        if (cu[s + 1] < cu[s] || cu[s + 1] - cu[s] > P)
            return -1;
    const int64_t hd = (int64_t)H * HD, ld = 3 * hd;
    for (int32_t s = 0; s < S; ++s) {
        for (int64_t i = 0; i < cu[s + 1] - cu[s]; ++i) {
            int64_t t = cu[s] + i;
            for (int32_t h = 0; h < H; ++h) {
                double *q = q_out + t * hd + (int64_t)h * HD;
                rotate_row(qkv + t * ld + (int64_t)h * HD, cos_t + i * HALF, sin_t + i * HALF,
                           mode, dtype, mode == ORACLE_MODE_B ? (float)scale : 1.0f, q);
                if (mode == ORACLE_MODE_A)
                    for (int m = 0; m < HD; ++m)
                        q[m] *= scale;
                rotate_row(qkv + t * ld + hd + (int64_t)h * HD, cos_t + i * HALF,
                           sin_t + i * HALF, mode, dtype, 1.0f, k_out + t * hd + (int64_t)h * HD);
            }
        }
    }
    return 0;
}

/* The sequence holding token t: the s with cu[s] <= t < cu[s+1] (zero-length sequences skipped). */
static int32_t sequence_of(const int32_t *cu, int32_t S, int64_t t)
{
    int32_t lo = 0, hi = S; /* invariant: cu[lo] <= t < cu[hi] */
    while (hi - lo > 1) {
        int32_t mid = lo + (hi - lo) / 2;
        if (cu[mid] <= t)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

/*
 * out [n_rows, H*64] and lse [n_rows, H] for the tokens rows[0..n_rows) (all T tokens in order
 * when rows is NULL). Returns 0, or -1 on malformed arguments.
 */
int vlf_oracle_attend(const float *qkv, const float *cos_t, const float *sin_t, int64_t P,
                      const int32_t *cu, int32_t S, int64_t T, int32_t H, int32_t window,
                      double scale, int32_t mode, int32_t dtype, const int64_t *rows,
                      int64_t n_rows, int32_t threads, double *out, double *lse)
{
    if (S < 0 || T < 0 || H < 1 || window < 0 || P < 0)
        return -1;
    if (mode != ORACLE_MODE_A && mode != ORACLE_MODE_B)
        return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return -1;
    if (cu[0] != 0 || cu[S] != T)
        return -1;
    const int causal = (window & CAUSAL_FLAG) != 0;
    const int32_t w = window & ~CAUSAL_FLAG;
    int64_t max_len = 0;
    for (int32_t s = 0; s < S; ++s) {
        if (cu[s + 1] < cu[s])
            return -1;
        if (cu[s + 1] - cu[s] > max_len)
            max_len = cu[s + 1] - cu[s];
    }
    if (max_len > P)
        return -1;
    if (rows == NULL && n_rows != T)
        return -1;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= T)
            return -1;
    if (n_rows == 0)
        return 0;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif

    const int64_t hd = (int64_t)H * HD, ld = 3 * hd;

    /* which sequences hold a requested row: only their keys are rotated */
    unsigned char *need = calloc((size_t)S + 1, 1);
    double *krot = malloc(sizeof(double) * (size_t)(T ? T : 1) * (size_t)hd);
    if (!need || !krot) {
        free(need);
        free(krot);
        return -2;
    }
    for (int64_t r = 0; r < n_rows; ++r)
        need[sequence_of(cu, S, rows ? rows[r] : r)] = 1;

    /* rotated keys of every needed (sequence, head): k_j = rot(K row of token cu[s]+j, j) */
    const float one = 1.0f;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sh = 0; sh < (int64_t)S * H; ++sh) {
        int32_t s = (int32_t)(sh / H), h = (int32_t)(sh % H);
        if (!need[s])
            continue;
        for (int64_t j = 0; j < cu[s + 1] - cu[s]; ++j) {
            int64_t t = cu[s] + j;
            rotate_row(qkv + t * ld + hd + (int64_t)h * HD, cos_t + j * HALF, sin_t + j * HALF,
                       mode, dtype, one, krot + t * hd + (int64_t)h * HD);
        }
    }

#pragma omp parallel
    {
        double *sc = malloc(sizeof(double) * (size_t)(max_len ? max_len : 1));
        double q[HD];
#pragma omp for schedule(dynamic, 16)
        for (int64_t rh = 0; rh < n_rows * H; ++rh) {
            int64_t r = rh / H;
            int32_t h = (int32_t)(rh % H);
            int64_t t = rows ? rows[r] : r;
            int32_t s = sequence_of(cu, S, t);
            int64_t start = cu[s], L = cu[s + 1] - cu[s], i = t - start;
            rotate_row(qkv + t * ld + (int64_t)h * HD, cos_t + i * HALF, sin_t + i * HALF, mode,
                       dtype, mode == ORACLE_MODE_B ? (float)scale : 1.0f, q);
            /* scores of the visible keys */
            double m = -INFINITY;
            for (int64_t j = 0; j < L; ++j) {
                int64_t gap = i > j ? i - j : j - i;
                if ((w > 0 && gap >= w) || (causal && j > i)) {
                    sc[j] = -INFINITY;
                    continue;
                }
                const double *k = krot + (start + j) * hd + (int64_t)h * HD;
                double dot = 0.0;
                for (int d = 0; d < HD; ++d)
                    dot += q[d] * k[d];
                sc[j] = mode == ORACLE_MODE_A ? scale * dot : dot;
                if (sc[j] > m)
                    m = sc[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j < L; ++j)
                if (sc[j] != -INFINITY)
                    sum += exp(sc[j] - m);
            double lz = m + log(sum);
            lse[r * H + h] = lz;
            double *o = out + r * hd + (int64_t)h * HD;
            for (int d = 0; d < HD; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                if (sc[j] == -INFINITY)
                    continue;
                double p = exp(sc[j] - lz);
                const float *v = qkv + (start + j) * ld + 2 * hd + (int64_t)h * HD;
                for (int d = 0; d < HD; ++d)
                    o[d] += p * (double)v[d];
            }
        }
        free(sc);
    }
    free(need);
    free(krot);
    return 0;
}

/* The number of threads a parallel region of this library uses. */
int32_t vlf_oracle_threads(int32_t threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
    return (int32_t)omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}
