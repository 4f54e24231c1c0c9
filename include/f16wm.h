/*
 * f16wm -- F16-weight matrix products on AMD MI355X (gfx950), C ABI.
 *
 * The operations are those of the bankML documentation page "bankML/f16.rs --
 * F16 weights, multiplied as the shipped ggml b11192 multiplies them" (cited
 * as "f16 page" with its section names).  An F16 weight matrix W is rows x k
 * IEEE binary16 values, row-major, k contiguous (little-endian, as the page
 * requires).  Activations are f32 columns rounded to f16 by f16wm_to_f16 and
 * then shared by every product that reads them (bankML page "bankML/forward.rs",
 * Advantages and efficiency: one rounded activation feeds Q, K and V, another
 * feeds gate and up).
 *
 * Conventions for every entry point below:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    reads/writes them in stream order during the call's kernels and keeps no
 *    reference afterwards; it never frees them and allocates no device memory.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are
 *    asynchronous: they enqueue kernels and return without synchronising.
 *  - Validation happens on the host before any launch.  On failure nothing is
 *    launched, a negative F16WM_E* code is returned and f16wm_last_error()
 *    gives the reason (per calling thread).
 *  - Sizes are element counts (int64_t).  Zero-sized products are no-ops that
 *    return F16WM_OK.  Outputs may not overlap inputs (F16WM_EINVAL).
 *  - Every f16 pointer must be 2-byte aligned and every f32 pointer 4-byte
 *    aligned.  Greater alignment (16 bytes, with k % 8 == 0) selects the
 *    vectorised kernels; the bits are the same either way.
 */
#ifndef F16WM_H
#define F16WM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define F16WM_OK 0
#define F16WM_EINVAL (-1)      /* bad argument: null, negative, overflow, alignment, overlap */
#define F16WM_ENODEV (-2)      /* no usable gfx950 device is current */
#define F16WM_ELAUNCH (-3)     /* the HIP runtime refused a launch */
#define F16WM_EUNSUPPORTED (-4) /* a valid shape this entry point does not take */

#define F16WM_MAX_MULTI 8      /* matrices per f16wm_mat_vec_multi call */

/* One matrix of a grouped product: W (rows x k, f16) and its output (rows f32). */
typedef struct {
    const uint16_t *w;
    int64_t rows;
    float *out;
} f16wm_mat;

/*
 * f16wm_to_f16: y[i] = f16(x[i]), binary32 -> binary16, round to nearest,
 * ties to even; overflow gives +-inf, results below 2^-14 become f16
 * subnormals, NaN gives a quiet NaN with the sign and top ten payload bits.
 * f16 page, Design notes ("Activation"): the activation is rounded this way
 * before every product.  x: count f32, y: count f16 (bit patterns).
 */
int f16wm_to_f16(const float *x, uint16_t *y, int64_t count, void *stream);

/*
 * f16wm_widen: y[i] = f32(h[i]), exact (every f16, subnormals included, is an
 * f32; NaN stays NaN).  f16 page, Technical usage (`widen`).  h: count f16,
 * y: count f32.
 */
int f16wm_widen(const uint16_t *h, float *y, int64_t count, void *stream);

/*
 * f16wm_get_rows: out[i][j] = f32(W[ids[i]][j]) for i < nids, j < k: F16
 * weight rows widened to f32, ggml's get_rows (f16 page, Technical usage
 * `dequantize_row`; the embedding lookup, which reads the tied token_embd
 * matrix, bankML page "bankML/forward.rs", Summary).  w: rows x k f16; ids:
 * nids int64 row indices in DEVICE memory; out: nids x k f32.  The ids are
 * not visible to the host: an id outside [0, rows) is not an error, its
 * output row is filled with quiet NaN.
 */
int f16wm_get_rows(const uint16_t *w, int64_t rows, int64_t k, const int64_t *ids, int64_t nids,
                   float *out, void *stream);

/*
 * f16wm_mat_vec: out[r] = vec_dot(W[r], a) for r < rows.
 * f16 page, Matrix products (mat_vec_par) and Design notes ("vec_dot"): each
 * row is four 8-lane f32 FMA accumulators over 32-element steps (accumulator
 * j lane l takes elements 32t + 8j + l), reduced (a0+a2)+(a1+a3), then low four
 * lanes + high four, then two horizontal adds of adjacent pairs; the k % 32
 * tail is added to that f32 in binary64, ascending, and the sum is rounded to
 * f32.  w: rows x k f16, a: k f16, out: rows f32.  k = 0 writes +0.0.
 * The page's vec_dot_u16 (the same order with the first operand given as
 * f16 values, e.g. K-cache rows) is this call: W is f16 values here too.
 */
int f16wm_mat_vec(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, float *out,
                  void *stream);

/*
 * f16wm_mat_vec_multi: for each of `count` matrices (1..F16WM_MAX_MULTI, all
 * with the same k) mats[m].out[r] = vec_dot(mats[m].w[r], a), in ONE launch.
 * f16 page, Matrix products (mat_vec_multi_par): Q, K and V, or gate and up,
 * by one column in one pass; every row is still one vec_dot.  `mats` is a
 * HOST array of `count` descriptors (read during the call only); the
 * pointers inside are device pointers.  Outputs may not overlap each other.
 */
int f16wm_mat_vec_multi(const f16wm_mat *mats, int32_t count, int64_t k, const uint16_t *a,
                        void *stream);

/* One product of a table launch (f16wm_mat_vec_table): out = W x column. */
typedef struct {
    const uint16_t *w;   /* rows x k f16, row-major (k contiguous), device */
    const void *a;       /* the column, k values, device: f16 bit patterns (a_f32 = 0), or f32 (a_f32 = 1) */
    float *out;          /* rows f32, device */
    int64_t rows;
    int64_t k;
    int32_t a_f32;       /* 0 or 1 */
} f16wm_gemv;

#define F16WM_MAX_TABLE 4096   /* products per f16wm_mat_vec_table call */

/*
 * f16wm_mat_vec_table: `count` (0..F16WM_MAX_TABLE) independent one-column
 * products, prods[p].out[r] = vec_dot(W_p[r], column_p) for r < rows_p, each
 * with its own weight, k, column and output; an f32 column is rounded to f16
 * as f16wm_to_f16 rounds it, inside the launch.  Every element is the
 * f16wm_mat_vec (or f16wm_mat_vec_f32) result bit for bit: the grouping
 * decides only which block computes a row, never its order.
 * f16 page, Matrix products (mat_vec_par per row; mat_vec_multi_par: several
 * matrices in one pass) and Advantages and efficiency (grouped matrices are
 * handed to the pool as one job instead of one per matrix); here the job
 * table generalises the grouping to products that share nothing, such as
 * every product of a decode step whose columns are already known, or the
 * same layer for several sequences.
 * Launches: products with k % 8 == 0 and 16-byte aligned w and a run in one
 * launch per kernel class (k <= 576: rows in registers; longer rows: staged
 * in LDS; f16 or f32 columns) and per 96 products of a class, longest k
 * first; any other product takes its own f16wm_mat_vec launch.  Nothing runs
 * in between, so the products may not depend on each other: every output
 * must be disjoint from every other output and from every weight and column
 * (F16WM_EINVAL); columns and weights may be shared.  `prods` is a HOST
 * array read during the call.  rows_p = 0 is a no-op for that product and
 * k_p = 0 writes +0.0.  Errors as for f16wm_mat_vec, reported with the
 * product's index; nothing is launched if any product is invalid.
 */
int f16wm_mat_vec_table(const f16wm_gemv *prods, int32_t count, void *stream);

/*
 * f16wm_mat_vec_f32 / f16wm_mat_vec_multi_f32: the same products taking the
 * activation column as k f32 values: each value is rounded to f16 exactly as
 * f16wm_to_f16 rounds it (same code) inside the product's staging, so the
 * result equals f16wm_to_f16 followed by f16wm_mat_vec / f16wm_mat_vec_multi,
 * bit for bit, in one launch and without writing the rounded column out.
 * f16 page, Design notes ("Activation": the activation is rounded before any
 * product) and Matrix products; bankML page "bankML/forward.rs", Advantages
 * and efficiency (one rounded activation feeds Q, K and V, another feeds gate
 * and up).  x: k f32 (4-byte aligned; 16-byte alignment with k % 8 == 0
 * selects the vectorised kernels).
 */
int f16wm_mat_vec_f32(const uint16_t *w, int64_t rows, int64_t k, const float *x, float *out,
                      void *stream);
int f16wm_mat_vec_multi_f32(const f16wm_mat *mats, int32_t count, int64_t k, const float *x,
                            void *stream);

/*
 * f16wm_mat_mul: out[c*rows + r] = dot(W[r], A[c]) for r < rows, c < n, with
 * the float order ggml picks by shape (f16 page, Matrix products mat_mul_par
 * and Design notes "sgemm_dot"): when f16wm_takes_sgemm(rows, k, n), every
 * element is one 8-lane FMA chain (lane l takes elements 8t + l, ascending t)
 * reduced ((l0+l4)+(l2+l6))+((l1+l5)+(l3+l7)); otherwise every element is
 * vec_dot as in f16wm_mat_vec.  Bit-exact: the kernel tiling never changes an
 * element's order.  w: rows x k f16; a: n x k f16 (column c at a + c*k);
 * out: n x rows f32.  n = 1 equals f16wm_mat_vec.
 */
int f16wm_mat_mul(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                  float *out, void *stream);

/*
 * f16wm_mat_mul_multi: f16wm_mat_mul for each of `count` matrices
 * (1..F16WM_MAX_MULTI) that share k and the activation block a [n][k]:
 * mats[m].out is n x mats[m].rows f32.  Each matrix takes the order its own
 * shape picks (f16wm_takes_sgemm(mats[m].rows, k, n)); when every matrix takes
 * the tinyBLAS order the whole group is one launch.  The grouping follows the
 * shared activations of bankML page "bankML/forward.rs" (Advantages and
 * efficiency: one rounded activation feeds Q, K and V, another gate and up)
 * for prefill micro-batches.  `mats` is a HOST array read during the call.
 */
int f16wm_mat_mul_multi(const f16wm_mat *mats, int32_t count, int64_t k, const uint16_t *a, int64_t n,
                        void *stream);

/*
 * f16wm_mat_mul_f32 / f16wm_mat_mul_multi_f32: f16wm_mat_mul /
 * f16wm_mat_mul_multi taking the activation block as f32 values x [n][k]
 * (column c at x + c*k): each value is rounded to f16 exactly as f16wm_to_f16
 * rounds it (same code) while the product stages it, so the result equals
 * f16wm_to_f16 on the block followed by the f16 entry point, bit for bit, in
 * one launch and without writing the rounded block out.  f16 page, Design
 * notes ("Activation": the activation is rounded before any product) and
 * Matrix products (mat_mul_par); bankML page "bankML/forward.rs", Advantages
 * and efficiency (one rounded activation feeds Q, K and V, another gate and
 * up).  x: 4-byte aligned; 16-byte alignment selects the vectorised kernels
 * (the bits are the same).  Errors and the other arguments as for the f16
 * entry points.
 */
int f16wm_mat_mul_f32(const uint16_t *w, int64_t rows, int64_t k, const float *x, int64_t n, float *out,
                      void *stream);
int f16wm_mat_mul_multi_f32(const f16wm_mat *mats, int32_t count, int64_t k, const float *x, int64_t n,
                            void *stream);

/*
 * f16wm_mat_mul_mfma: the same product and layout as f16wm_mat_mul computed on
 * the fp16 matrix cores (MFMA, f16 x f16 products, f32 accumulation).  An
 * approximate fast path for prefill micro-batches (bankML page
 * "bankML/forward.rs", Technical usage: prompts run in micro-batches of up to
 * 512 columns): its summation order is the hardware's, so it is NOT bit-equal
 * to either ggml order; its error against a binary64 sum is bounded instead.
 * Requires k % 8 == 0 and 16-byte aligned w and a (F16WM_EUNSUPPORTED else).
 */
int f16wm_mat_mul_mfma(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                       float *out, void *stream);

/* f16wm_mat_mul_mfma_multi: f16wm_mat_mul_mfma for a group of matrices that
   share k and a (as f16wm_mat_mul_multi), in one launch. */
int f16wm_mat_mul_mfma_multi(const f16wm_mat *mats, int32_t count, int64_t k, const uint16_t *a,
                             int64_t n, void *stream);

/* Which columns of a micro-batch leave the last layer (f16wm_mat_mul_out). */
#define F16WM_OUT_NONE 0
#define F16WM_OUT_LAST 1
#define F16WM_OUT_ALL 2

/*
 * f16wm_mat_mul_out: the last layer's product of a micro-batch of n columns
 * (a: n x k f16) over only the columns that leave the model.  bankML page
 * "bankML/forward.rs", section "Why only the output rows leave the last
 * layer": llama.cpp sends through the last feed-forward block only the rows
 * it outputs (its inp_out_ids: none, the last, or all), and for F16 weights
 * that count decides the float order.  mode F16WM_OUT_NONE computes nothing;
 * F16WM_OUT_LAST computes the last column alone (n >= 1), i.e. vec_dot
 * (out: rows f32, the bits of f16wm_mat_vec on a + (n-1)*k, which differ
 * from that column of the full product wherever the full product takes the
 * tinyBLAS order); F16WM_OUT_ALL is f16wm_mat_mul (out: n x rows f32).
 * Another mode is F16WM_EINVAL.
 */
int f16wm_mat_mul_out(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n, int32_t mode,
                      float *out, void *stream);

/*
 * f16wm_kq: attention scores against an f16 K cache in the vec_dot order.
 * f16 page, Technical usage (vec_dot_u16: vec_dot with the first operand
 * given as f16 values) and Summary (the attention code uses it for K-cache
 * rows).  kc: n_kv x n_kv_head x d f16, position-major (one layer's K cache);
 * q: n_head x d f16 (the rounded queries); out: n_head x n_kv f32 with
 * out[h * n_kv + p] = vec_dot(kc[p][h / (n_head / n_kv_head)], q[h]).
 * Requires n_head % n_kv_head == 0 (grouped-query attention, else
 * F16WM_EINVAL) and n_kv_head <= 65535 (else F16WM_EUNSUPPORTED); out may
 * not overlap kc or q.  d of 64 or 128 with 16-byte aligned kc and q, at
 * most 512 query heads, a position row (n_kv_head * d halves) of at most
 * 32 KB and a cache below 2 GB takes the LDS-tiled kernel; any other case
 * the lane-per-chain kernel (same bits).  Empty outputs are a no-op.
 */
int f16wm_kq(const uint16_t *kc, int64_t n_kv, int64_t n_kv_head, int64_t d, const uint16_t *q, int64_t n_head,
             float *out, void *stream);

/*
 * f16wm_mad / f16wm_scale: the f16 V-accumulator updates of the attention
 * code (f16 page, Technical usage: mad is ggml_vec_mad_f16, scale is
 * ggml_vec_scale_f16), for nvec vectors of n elements with one f32 weight
 * (factor) per vector, in place on acc (nvec x n f16, device):
 *   mad:   acc[b][i] = f16(fma(f32(v[b][i]), w[b], f32(acc[b][i])))
 *   scale: acc[b][i] = f16(f32(acc[b][i]) * s[b])
 * each f32 result rounded to f16 as f16wm_to_f16 rounds.  The page names mad
 * but not its arithmetic: the single fused multiply-add is our reading.
 * v: nvec x n f16; w, s: nvec f32 in DEVICE memory.  v may not overlap acc.
 */
int f16wm_mad(uint16_t *acc, const uint16_t *v, const float *w, int64_t nvec, int64_t n, void *stream);
int f16wm_scale(uint16_t *acc, const float *s, int64_t nvec, int64_t n, void *stream);

/*
 * f16wm_takes_sgemm: 1 when n >= 2 && rows % 4 == 0 && k % 8 == 0, else 0
 * (f16 page, Technical usage).  Pure host function, no device needed.
 * Negative arguments give 0.
 */
int f16wm_takes_sgemm(int64_t rows, int64_t k, int64_t n);

/* The reason for the calling thread's last failed call ("" if none). */
const char *f16wm_last_error(void);

/* Library version string. */
const char *f16wm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* F16WM_H */
