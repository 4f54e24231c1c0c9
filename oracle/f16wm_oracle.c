/*
 * f16wm oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of what the F16-weight matrix products
 * compute, written from the bankML documentation page "bankML/f16.rs -- F16
 * weights, multiplied as the shipped ggml b11192 multiplies them" (cited below
 * as "f16 page"; its sections: Summary, Technical usage, Matrix products,
 * How it is verified, Design notes).  It shares no code, header or table with
 * the HIP library under f16_weight_matrix_amd/; only tests/, the smoke check
 * and the benchmark's CPU-baseline leg may load it.
 *
 * Floating point: every f32 operation below is one IEEE binary32 operation
 * with round-to-nearest-even (built with -ffp-contract=off, no fast-math);
 * fmaf is the fused multiply-add with a single rounding; the tail of vec_dot
 * is binary64 as the page states.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py to
 * something other than itself (exhaustive library conversions, exact integer
 * sums, one-hot rows, hand-derived tree cases, invariance groups, error bounds
 * against an exact fixed-point sum).  One claim stays "parity unpinned": that
 * these orders reproduce the bits of the shipped ggml b11192 CPU library.
 * That library is not available here, so the orders are the page's text under
 * the readings stated at each function.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------ */
/* f16 <-> f32 conversions, written from the IEEE 754 binary16 format   */
/* ------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }
static float bits_f32(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }

/*
 * to_f16: binary32 -> binary16, round to nearest, ties to even.
 * f16 page, Design notes ("Activation"): the activation is rounded to f16
 * (F16C vcvtps2ph with immediate 0, i.e. round to nearest even) before any
 * product.  The page says nothing of NaN, overflow or subnormals; we take the
 * IEEE definition with the x86 F16C conventions: overflow to +-inf, gradual
 * underflow into f16 subnormals, NaN -> quiet NaN keeping the sign and the
 * top ten payload bits.
 *
 * Method: |x| = M * 2^E exactly (M integer).  The f16 quantum at |x| is
 * 2^(max(floor(log2|x|), -14) - 10).  Divide by the quantum, round the integer
 * quotient to nearest-even, and re-encode; a quotient that reaches the next
 * binade carries into the exponent field by plain addition.
 */
uint16_t oracle_to_f16_one(float x)
{
    uint32_t b = f32_bits(x);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t ef = (b >> 23) & 0xffu;
    uint32_t m = b & 0x7fffffu;

    if (ef == 0xffu) {
        if (m == 0) return sign | 0x7c00u;                     /* +-inf */
        return sign | 0x7c00u | 0x0200u | (uint16_t)(m >> 13); /* quiet NaN */
    }
    if (ef == 0 && m == 0) return sign;                        /* +-0 */

    uint64_t M;
    int E;       /* |x| = M * 2^E */
    int e2;      /* floor(log2 |x|) */
    if (ef != 0) {
        M = (uint64_t)(m | 0x800000u);
        E = (int)ef - 150;
        e2 = (int)ef - 127;
    } else {
        M = m;
        E = -149;
        int top = 31 - __builtin_clz(m);
        e2 = top - 149;
    }
    int qexp = (e2 < -14 ? -14 : e2) - 10;   /* f16 quantum = 2^qexp */
    int shift = qexp - E;                     /* >= 13 for every f32 */

    uint64_t N;
    if (shift >= 40) {
        N = 0;                                /* M < 2^24: below half a quantum */
    } else {
        N = M >> shift;
        uint64_t rem = M & ((1ull << shift) - 1);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (N & 1u))) N += 1;
    }
    /* value = N * 2^qexp.  Subnormal range (qexp = -24): the encoding is N
       itself (N = 1024 is the smallest normal).  Normal range: exponent field
       qexp + 25 and significand N - 1024; N = 2048 carries into the field. */
    uint64_t enc;
    if (qexp == -24 && N <= 1024)
        enc = N;
    else
        enc = ((uint64_t)(qexp + 25) << 10) + (N - 1024);
    if (enc >= 0x7c00u) return sign | 0x7c00u;                /* overflow */
    return sign | (uint16_t)enc;
}

void oracle_to_f16(const float *x, uint16_t *y, int64_t count)
{
    for (int64_t i = 0; i < count; i++) y[i] = oracle_to_f16_one(x[i]);
}

/* widen: exact binary16 -> binary32 (f16 page, Technical usage: "exact").
   Subnormal: f * 2^-24; normal: (1024 + f) * 2^(e - 25); both representable
   in binary32, so ldexpf is exact.  NaN keeps sign and payload, quieted. */
float oracle_widen_one(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t f = h & 0x3ffu;
    if (e == 31) {
        if (f == 0) return bits_f32(sign | 0x7f800000u);
        return bits_f32(sign | 0x7f800000u | 0x00400000u | (f << 13));
    }
    float mag = (e == 0) ? ldexpf((float)f, -24) : ldexpf((float)(1024u + f), (int)e - 25);
    return (sign ? -mag : mag);
}

void oracle_widen(const uint16_t *h, float *y, int64_t count)
{
    for (int64_t i = 0; i < count; i++) y[i] = oracle_widen_one(h[i]);
}

/* The products call widen on every element; the values are memoised once
   in a 65536-entry table filled by oracle_widen_one itself. */
static float g_widen[65536];
static pthread_once_t g_widen_once = PTHREAD_ONCE_INIT;
static void fill_widen(void)
{
    for (uint32_t i = 0; i < 65536u; i++) g_widen[i] = oracle_widen_one((uint16_t)i);
}
static inline float W16(uint16_t h) { return g_widen[h]; }
static void need_widen(void) { pthread_once(&g_widen_once, fill_widen); }

/* ------------------------------------------------------------------ */
/* The two reductions                                                  */
/* ------------------------------------------------------------------ */

/*
 * vec_dot: ggml_vec_dot_f16, f16 page, Design notes ("vec_dot") and Summary
 * (one column).  Four accumulators of eight f32 lanes each are fed by FMAs
 * over 32-element steps: accumulator j, lane l takes elements 32t + 8j + l.
 * They are reduced as (a0 + a2) + (a1 + a3) lane by lane, then the low four
 * lanes are added to the high four, then two horizontal adds combine adjacent
 * pairs (our reading of "horizontal add": pairs (0,1) and (2,3), then the two
 * sums).  The reduced value is an f32; the k % 32 tail is added to it in
 * binary64, element by element in ascending order; the result is that double
 * rounded to f32.
 */
float oracle_vec_dot(const uint16_t *x, const uint16_t *y, int64_t k)
{
    need_widen();
    float acc[4][8];
    for (int j = 0; j < 4; j++)
        for (int l = 0; l < 8; l++) acc[j][l] = 0.0f;

    int64_t np = k - k % 32;
    for (int64_t i = 0; i < np; i += 32)
        for (int j = 0; j < 4; j++)
            for (int l = 0; l < 8; l++) {
                int64_t e = i + 8 * j + l;
                acc[j][l] = fmaf(W16(x[e]), W16(y[e]), acc[j][l]);
            }

    float s[8];
    for (int l = 0; l < 8; l++) s[l] = (acc[0][l] + acc[2][l]) + (acc[1][l] + acc[3][l]);
    float u[4];
    for (int i = 0; i < 4; i++) u[i] = s[i] + s[i + 4];
    float v = (u[0] + u[1]) + (u[2] + u[3]);

    double d = (double)v;
    for (int64_t i = np; i < k; i++) {
        float p = W16(x[i]) * W16(y[i]);   /* exact: an f16 x f16 product fits in f32 */
        d = d + (double)p;
    }
    return (float)d;
}

/*
 * sgemm_dot: one tinyBLAS element, f16 page, Design notes ("sgemm_dot").
 * One chain of eight f32 lanes: lane l takes elements 8t + l in ascending t,
 * each step an FMA; then hsum ((l0 + l4) + (l2 + l6)) + ((l1 + l5) + (l3 + l7)).
 * Requires k % 8 == 0 (Technical usage: y.len() % 8 == 0); the caller checks.
 */
float oracle_sgemm_dot(const uint16_t *x, const uint16_t *y, int64_t k)
{
    need_widen();
    float acc[8];
    for (int l = 0; l < 8; l++) acc[l] = 0.0f;
    for (int64_t i = 0; i + 8 <= k; i += 8)
        for (int l = 0; l < 8; l++)
            acc[l] = fmaf(W16(x[i + l]), W16(y[i + l]), acc[l]);
    return ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));
}

/* takes_sgemm: f16 page, Technical usage: n >= 2 && rows % 4 == 0 && k % 8 == 0.
   rows = weight rows (outputs), k = row length, n = activation columns. */
int oracle_takes_sgemm(int64_t rows, int64_t k, int64_t n)
{
    return n >= 2 && rows % 4 == 0 && k % 8 == 0;
}

/* ------------------------------------------------------------------ */
/* Products (f16 page, Matrix products)                                 */
/* ------------------------------------------------------------------ */

/* Element (r, c) of a product of W [rows][k] with A [n][k], by the shape's
   path: tinyBLAS when takes_sgemm(rows, k, n), else vec_dot. */
static float element(const uint16_t *w, int64_t rows, int64_t k,
                     const uint16_t *a, int64_t n, int64_t r, int64_t c)
{
    const uint16_t *x = w + r * k;
    const uint16_t *y = a + c * k;
    return oracle_takes_sgemm(rows, k, n) ? oracle_sgemm_dot(x, y, k) : oracle_vec_dot(x, y, k);
}

typedef struct {
    const uint16_t *w; int64_t rows, k; const uint16_t *a; int64_t n; float *out;
    int64_t r0, r1;
} job_t;

static void *run_rows(void *p)
{
    job_t *j = (job_t *)p;
    for (int64_t c = 0; c < j->n; c++)
        for (int64_t r = j->r0; r < j->r1; r++)
            j->out[c * j->rows + r] = element(j->w, j->rows, j->k, j->a, j->n, r, c);
    return NULL;
}

static int pick_threads(int nthreads)
{
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* mat_mul: out[c * rows + r] for every r < rows, c < n (f16 page, Matrix
   products: "writes out[c*rows + r]").  With n == 1 this is mat_vec.
   Rows are split over threads in contiguous blocks; each element is computed
   whole by one thread, so the bits cannot depend on the thread count. */
void oracle_mat_mul(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                    float *out, int nthreads)
{
    need_widen();
    int T = pick_threads(nthreads);
    if (T > rows) T = rows > 0 ? (int)rows : 1;
    job_t *jobs = (job_t *)calloc((size_t)T, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)T, sizeof(pthread_t));
    for (int t = 0; t < T; t++) {
        jobs[t] = (job_t){w, rows, k, a, n, out, rows * t / T, rows * (t + 1) / T};
        if (T == 1) run_rows(&jobs[t]);
        else pthread_create(&th[t], NULL, run_rows, &jobs[t]);
    }
    if (T > 1)
        for (int t = 0; t < T; t++) pthread_join(th[t], NULL);
    free(jobs);
    free(th);
}

/* mat_vec: out[r] = vec_dot(W[r], a) (f16 page, Matrix products). */
void oracle_mat_vec(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, float *out,
                    int nthreads)
{
    oracle_mat_mul(w, rows, k, a, 1, out, nthreads);
}

/* Selected elements of a product (for parity on samples of full-size
   products): out[i] = element (rr[i], cc[i]) of W x A with the path that the
   full shape (rows, k, n) takes. */
void oracle_mat_mul_at(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                       const int64_t *rr, const int64_t *cc, int64_t count, float *out)
{
    need_widen();
    for (int64_t i = 0; i < count; i++) out[i] = element(w, rows, k, a, n, rr[i], cc[i]);
}

/* ------------------------------------------------------------------ */
/* Exact and binary64 references (for the error bounds and the MFMA path) */
/* ------------------------------------------------------------------ */

/* Every f16 value is an integer multiple of 2^-24 below 2^16 in magnitude,
   so every product is an integer multiple of 2^-48 below 2^32 and a sum of
   up to 2^40 of them fits in a signed 128-bit integer exactly. */
static __int128 f16_units(uint16_t h)   /* h = units * 2^-24, h finite */
{
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t f = h & 0x3ffu;
    __int128 mag = (e == 0) ? (__int128)f : ((__int128)(1024u + f) << (e - 1));
    return (h & 0x8000u) ? -mag : mag;
}

/* The exact sum of x[i]*y[i], rounded once to binary64; *abs_sum receives
   sum |x[i]*y[i]| the same way.  Inputs must be finite. */
double oracle_exact_dot(const uint16_t *x, const uint16_t *y, int64_t k, double *abs_sum)
{
    __int128 s = 0, sa = 0;
    for (int64_t i = 0; i < k; i++) {
        __int128 p = f16_units(x[i]) * f16_units(y[i]);
        s += p;
        sa += (p < 0 ? -p : p);
    }
    if (abs_sum) *abs_sum = ldexp((double)sa, -48);
    return ldexp((double)s, -48);
}

/* The binary64 reference of a product used to judge the MFMA fast path:
   ref[i] = sum_j widen(W[rr[i]][j]) * widen(A[cc[i]][j]) accumulated in
   binary64 in ascending j, and scale[i] = sum_j |...| the same way. */
void oracle_fp64_at(const uint16_t *w, int64_t k, const uint16_t *a,
                    const int64_t *rr, const int64_t *cc, int64_t count,
                    double *ref, double *scale)
{
    need_widen();
    for (int64_t i = 0; i < count; i++) {
        const uint16_t *x = w + rr[i] * k;
        const uint16_t *y = a + cc[i] * k;
        double s = 0.0, sa = 0.0;
        for (int64_t j = 0; j < k; j++) {
            double p = (double)W16(x[j]) * (double)W16(y[j]);
            s += p;
            sa += fabs(p);
        }
        ref[i] = s;
        scale[i] = sa;
    }
}

/* ------------------------------------------------------------------ */
/* The last layer's output columns (forward page)                       */
/* ------------------------------------------------------------------ */

/*
 * mat_mul_out: bankML page "bankML/forward.rs", section "Why only the output
 * rows leave the last layer": on the last layer of a prompt only the rows
 * llama.cpp outputs (its inp_out_ids: none, the last, or all) go through the
 * feed-forward block, and for F16 weights the number of those rows decides
 * the float order (one column: vec_dot; two or more: tinyBLAS when
 * takes_sgemm holds).  mode 0 = none (nothing written), 1 = the last column
 * (out: rows f32), 2 = all n columns (out: n x rows f32).
 */
void oracle_mat_mul_out(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                        int mode, float *out, int nthreads)
{
    if (mode == 1 && n >= 1) oracle_mat_mul(w, rows, k, a + (n - 1) * k, 1, out, nthreads);
    else if (mode == 2) oracle_mat_mul(w, rows, k, a, n, out, nthreads);
}

/* ------------------------------------------------------------------ */
/* The attention helpers over an f16 KV cache (f16 page)                */
/* ------------------------------------------------------------------ */

/*
 * kq: attention scores against an f16 K cache.  f16 page, Technical usage:
 * vec_dot_u16 is vec_dot with the first operand given as f16 values (a K
 * cache row); Summary: the attention code uses it for K-cache rows.  Cache
 * layout per layer: kc[p][j][0..d) for position p < n_kv and KV head
 * j < n_kv_head (position-major, as llama.cpp stores a layer's K); query
 * head h uses KV head h / (n_head / n_kv_head) (grouped-query attention).
 * out[h * n_kv + p] = vec_dot(kc[p][h / G], q[h]), q: n_head x d f16.
 */
void oracle_kq(const uint16_t *kc, int64_t n_kv, int64_t n_kv_head, int64_t d, const uint16_t *q,
               int64_t n_head, float *out)
{
    const int64_t G = n_head / n_kv_head;
    for (int64_t h = 0; h < n_head; h++)
        for (int64_t p = 0; p < n_kv; p++)
            out[h * n_kv + p] = oracle_vec_dot(kc + (p * n_kv_head + h / G) * d, q + h * d, d);
}

/*
 * mad: ggml_vec_mad_f16, the flash-attention V accumulator (f16 page,
 * Technical usage `mad(acc, v, w)`; How it is verified: checked against the
 * scalar definition, odd tails included).  The page names the function but
 * not its arithmetic; our reading (parity partly unpinned): every element is
 * acc[i] = to_f16(fma(widen(v[i]), w, widen(acc[i]))), one fused multiply-add
 * in f32 (the F16C + FMA vector body; the scalar tail contracts to the same
 * FMA), then rounded to f16.  Here for nvec vectors of n elements with one
 * weight per vector: acc[b][i] with w[b].
 */
void oracle_mad(uint16_t *acc, const uint16_t *v, const float *w, int64_t nvec, int64_t n)
{
    need_widen();
    for (int64_t b = 0; b < nvec; b++)
        for (int64_t i = 0; i < n; i++) {
            const int64_t e = b * n + i;
            acc[e] = oracle_to_f16_one(fmaf(W16(v[e]), w[b], W16(acc[e])));
        }
}

/*
 * scale: ggml_vec_scale_f16 (f16 page, Technical usage `scale(acc, s)`):
 * acc[i] = to_f16(widen(acc[i]) * s), one f32 multiply, then rounded to f16.
 * For nvec vectors of n elements with one factor per vector: acc[b][i], s[b].
 */
void oracle_scale(uint16_t *acc, const float *s, int64_t nvec, int64_t n)
{
    need_widen();
    for (int64_t b = 0; b < nvec; b++)
        for (int64_t i = 0; i < n; i++) {
            const int64_t e = b * n + i;
            acc[e] = oracle_to_f16_one(W16(acc[e]) * s[b]);
        }
}
