// The f16wm C ABI: host-side validation, the shape-based choice of float
// order, and the kernel launches.  No entry point allocates memory or
// synchronises; every launch goes to the caller's stream.
//
// Path choice: bankML f16 page, Technical usage and Design notes.  One column
// (and every shape for which takes_sgemm is false) uses the vec_dot order;
// n >= 2 with rows % 4 == 0 and k % 8 == 0 uses the tinyBLAS order.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return F16WM_OK;
}

// Largest element count accepted for one array (keeps every byte offset and
// grid computation far inside int64 / uint32 ranges).
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool mul_ok(int64_t a, int64_t b, int64_t *r)
{
    if (a < 0 || b < 0) return false;
    if (__builtin_mul_overflow(a, b, r)) return false;
    return *r <= kMaxElems;
}

struct Span {
    uintptr_t lo, hi;   // [lo, hi)
};
Span span(const void *p, int64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }
bool overlap(Span x, Span y) { return x.lo < y.hi && y.lo < x.hi && x.lo != x.hi && y.lo != y.hi; }

// Device admission: the current device must be a gfx950.  Cached per device.
std::atomic<int> g_dev_state[64];   // 0 unknown, 1 ok, 2 refused

int check_device(const char *fn)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0)
        return fail(F16WM_ENODEV, "%s: no HIP device is current (%s)", fn,
                    e != hipSuccess ? hipGetErrorString(e) : "none");
    if (dev < 64) {
        int st = g_dev_state[dev].load(std::memory_order_relaxed);
        if (st == 1) return F16WM_OK;
        if (st == 2) return fail(F16WM_ENODEV, "%s: device %d is not a gfx950", fn, dev);
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
        return fail(F16WM_ENODEV, "%s: hipGetDeviceProperties(%d) failed: %s", fn, dev,
                    hipGetErrorString(e));
    const bool good = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_state[dev].store(good ? 1 : 2, std::memory_order_relaxed);
    if (!good)
        return fail(F16WM_ENODEV, "%s: device %d is %s, this library is built for gfx950", fn, dev,
                    prop.gcnArchName);
    return F16WM_OK;
}

int launched(const char *fn, hipError_t e)
{
    if (e != hipSuccess) return fail(F16WM_ELAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// Checks common to the products: sizes, overflow, null pointers, alignment
// and overlap.  The activation has n*k elements of a_es bytes (2: f16 bit
// patterns, 4: f32 values).
int check_product(const char *fn, const uint16_t *w, int64_t rows, int64_t k, const void *a, int a_es,
                  int64_t n, const float *out, int64_t *w_elems, int64_t *a_elems, int64_t *o_elems)
{
    if (rows < 0 || k < 0 || n < 0)
        return fail(F16WM_EINVAL, "%s: negative size (rows=%lld k=%lld n=%lld)", fn, (long long)rows,
                    (long long)k, (long long)n);
    if (!mul_ok(rows, k, w_elems) || !mul_ok(n, k, a_elems) || !mul_ok(n, rows, o_elems))
        return fail(F16WM_EINVAL, "%s: size too large (rows=%lld k=%lld n=%lld; limit 2^40 elements)",
                    fn, (long long)rows, (long long)k, (long long)n);
    if ((*w_elems > 0 && !w) || (*a_elems > 0 && !a) || (*o_elems > 0 && !out))
        return fail(F16WM_EINVAL, "%s: null pointer for a non-empty array", fn);
    if (!aligned(w, 2) || !aligned(a, (uintptr_t)a_es) || !aligned(out, 4))
        return fail(F16WM_EINVAL, "%s: misaligned pointer (f16 arrays need 2 bytes, f32 arrays 4)", fn);
    const Span so = span(out, *o_elems * 4);
    if (overlap(so, span(w, *w_elems * 2)) || overlap(so, span(a, *a_elems * a_es)))
        return fail(F16WM_EINVAL, "%s: output overlaps an input", fn);
    return F16WM_OK;
}

}  // namespace

extern "C" {

const char *f16wm_last_error(void) { return g_err.c_str(); }

const char *f16wm_version(void) { return "f16wm 0.1 (gfx950)"; }

int f16wm_takes_sgemm(int64_t rows, int64_t k, int64_t n)
{
    if (rows < 0 || k < 0 || n < 0) return 0;
    return (n >= 2 && rows % 4 == 0 && k % 8 == 0) ? 1 : 0;
}

int f16wm_to_f16(const float *x, uint16_t *y, int64_t count, void *stream)
{
    const char *fn = "f16wm_to_f16";
    if (count < 0 || count > kMaxElems)
        return fail(F16WM_EINVAL, "%s: bad count %lld", fn, (long long)count);
    if (count == 0) return ok();
    if (!x || !y) return fail(F16WM_EINVAL, "%s: null pointer", fn);
    if (!aligned(x, 4) || !aligned(y, 2)) return fail(F16WM_EINVAL, "%s: misaligned pointer", fn);
    if (overlap(span(x, count * 4), span(y, count * 2)))
        return fail(F16WM_EINVAL, "%s: output overlaps the input", fn);
    if (int rc = check_device(fn)) return rc;
    return launched(fn, f16wm::launch_to_f16(x, y, count, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// mat_vec with an f16 (f32act = false) or f32 (rounded in the kernel)
// activation column.
int mat_vec_impl(const char *fn, const uint16_t *w, int64_t rows, int64_t k, const void *a, bool f32act,
                 float *out, void *stream)
{
    int64_t we, ae, oe;
    if (int rc = check_product(fn, w, rows, k, a, f32act ? 4 : 2, 1, out, &we, &ae, &oe)) return rc;
    if (rows == 0) return ok();
    if (int rc = check_device(fn)) return rc;
    f16wm::RowTable t = {};
    t.count = 1;
    t.w[0] = w;
    t.out[0] = out;
    t.row0[0] = 0;
    t.row0[1] = rows;
    const bool vec8 = k % 8 == 0 && aligned(w, 16) && aligned(a, 16);
    return launched(fn, f16wm::launch_vec_dot(t, k, a, f32act, 1, vec8, (hipStream_t)stream));
}

int mat_vec_multi_impl(const char *fn, const f16wm_mat *mats, int32_t count, int64_t k, const void *a,
                       bool f32act, void *stream)
{
    if (count < 1 || count > F16WM_MAX_MULTI)
        return fail(F16WM_EINVAL, "%s: count %d outside 1..%d", fn, (int)count, F16WM_MAX_MULTI);
    if (!mats) return fail(F16WM_EINVAL, "%s: null descriptor array", fn);
    if (k < 0) return fail(F16WM_EINVAL, "%s: negative size (k=%lld)", fn, (long long)k);
    f16wm::RowTable t = {};
    t.count = count;
    bool vec8 = k % 8 == 0 && aligned(a, 16);
    int64_t total = 0;
    for (int m = 0; m < count; m++) {
        int64_t we, ae, oe;
        char name[64];
        snprintf(name, sizeof name, "%s[%d]", fn, m);
        if (int rc = check_product(name, mats[m].w, mats[m].rows, k, a, f32act ? 4 : 2, 1, mats[m].out, &we,
                                   &ae, &oe))
            return rc;
        for (int j = 0; j < m; j++) {
            // no output may overlap another matrix or another output
            const Span sm = span(mats[m].out, mats[m].rows * 4);
            if (overlap(sm, span(mats[j].out, mats[j].rows * 4)) ||
                overlap(sm, span(mats[j].w, mats[j].rows * k * 2)) ||
                overlap(span(mats[j].out, mats[j].rows * 4), span(mats[m].w, mats[m].rows * k * 2)))
                return fail(F16WM_EINVAL, "%s: outputs of matrices %d and %d overlap another array", fn,
                            j, m);
        }
        t.w[m] = mats[m].w;
        t.out[m] = mats[m].out;
        t.row0[m] = total;
        total += mats[m].rows;
        if (total > kMaxElems) return fail(F16WM_EINVAL, "%s: too many rows", fn);
        vec8 = vec8 && aligned(mats[m].w, 16);
    }
    t.row0[count] = total;
    if (total == 0) return ok();
    if (int rc = check_device(fn)) return rc;
    return launched(fn, f16wm::launch_vec_dot(t, k, a, f32act, 1, vec8, (hipStream_t)stream));
}

// Products of `count` matrices sharing k and the activation block a [n][k]
// (out of matrix m: [n][rows_m]).  Exact: each matrix in the order its own
// shape picks (tinyBLAS when takes_sgemm(rows_m, k, n), else vec_dot); one
// launch when every matrix takes the tinyBLAS order.  mfma: the matrix-core
// product of every matrix in one launch.
int mat_mul_impl(const char *fn, const f16wm_mat *mats, int32_t count, int64_t k, const void *a,
                 bool f32act, int64_t n, bool mfma, void *stream)
{
    if (count < 1 || count > F16WM_MAX_MULTI)
        return fail(F16WM_EINVAL, "%s: count %d outside 1..%d", fn, (int)count, F16WM_MAX_MULTI);
    if (!mats) return fail(F16WM_EINVAL, "%s: null descriptor array", fn);
    int64_t total = 0;
    for (int m = 0; m < count; m++) {
        int64_t we, ae, oe;
        char name[80];
        if (count == 1)
            snprintf(name, sizeof name, "%s", fn);
        else
            snprintf(name, sizeof name, "%s[%d]", fn, m);
        if (int rc = check_product(name, mats[m].w, mats[m].rows, k, a, f32act ? 4 : 2, n, mats[m].out, &we, &ae,
                                   &oe))
            return rc;
        for (int j = 0; j < m; j++) {
            const Span sm = span(mats[m].out, mats[m].rows * n * 4);
            if (overlap(sm, span(mats[j].out, mats[j].rows * n * 4)) ||
                overlap(sm, span(mats[j].w, mats[j].rows * k * 2)) ||
                overlap(span(mats[j].out, mats[j].rows * n * 4), span(mats[m].w, mats[m].rows * k * 2)))
                return fail(F16WM_EINVAL, "%s: outputs of matrices %d and %d overlap another array", fn,
                            j, m);
        }
        total += mats[m].rows;
    }
    bool al16 = aligned(a, 16);
    for (int m = 0; m < count; m++) al16 = al16 && aligned(mats[m].w, 16);
    if (mfma && (k % 8 != 0 || !al16))
        return fail(F16WM_EUNSUPPORTED, "%s: needs k %% 8 == 0 and 16-byte aligned w and a (k=%lld)", fn,
                    (long long)k);
    if (total == 0 || n == 0) return ok();
    if (int rc = check_device(fn)) return rc;

    f16wm::GemmTable g = {};
    bool all_sgemm = true;
    for (int m = 0; m < count; m++) {
        if (mats[m].rows == 0) continue;
        g.w[g.count] = mats[m].w;
        g.rows[g.count] = mats[m].rows;
        g.out[g.count] = mats[m].out;
        g.count++;
        all_sgemm = all_sgemm && f16wm_takes_sgemm(mats[m].rows, k, n);
    }
    if (mfma)
        return launched(fn, f16wm::launch_mfma(g, k, static_cast<const uint16_t *>(a), n, (hipStream_t)stream));
    if (all_sgemm) return launched(fn, f16wm::launch_sgemm(g, k, a, n, al16, f32act, (hipStream_t)stream));
    // other orders: one launch per matrix, each in its own order
    for (int m = 0; m < g.count; m++) {
        hipError_t e;
        if (f16wm_takes_sgemm(g.rows[m], k, n)) {
            f16wm::GemmTable one = {};
            one.count = 1;
            one.w[0] = g.w[m];
            one.rows[0] = g.rows[m];
            one.out[0] = g.out[m];
            e = f16wm::launch_sgemm(one, k, a, n, al16, f32act, (hipStream_t)stream);
        } else {
            f16wm::RowTable t = {};
            t.count = 1;
            t.w[0] = g.w[m];
            t.out[0] = g.out[m];
            t.row0[0] = 0;
            t.row0[1] = g.rows[m];
            e = f16wm::launch_vec_dot(t, k, a, f32act, n, k % 8 == 0 && al16, (hipStream_t)stream);
        }
        if (e != hipSuccess) return launched(fn, e);
    }
    return ok();
}

}  // namespace

extern "C" {

int f16wm_widen(const uint16_t *h, float *y, int64_t count, void *stream)
{
    const char *fn = "f16wm_widen";
    if (count < 0 || count > kMaxElems)
        return fail(F16WM_EINVAL, "%s: bad count %lld", fn, (long long)count);
    if (count == 0) return ok();
    if (!h || !y) return fail(F16WM_EINVAL, "%s: null pointer", fn);
    if (!aligned(h, 2) || !aligned(y, 4)) return fail(F16WM_EINVAL, "%s: misaligned pointer", fn);
    if (overlap(span(h, count * 2), span(y, count * 4)))
        return fail(F16WM_EINVAL, "%s: output overlaps the input", fn);
    if (int rc = check_device(fn)) return rc;
    return launched(fn, f16wm::launch_widen(h, y, count, (hipStream_t)stream));
}

int f16wm_get_rows(const uint16_t *w, int64_t rows, int64_t k, const int64_t *ids, int64_t nids,
                   float *out, void *stream)
{
    const char *fn = "f16wm_get_rows";
    int64_t we, oe;
    if (rows < 0 || k < 0 || nids < 0)
        return fail(F16WM_EINVAL, "%s: negative size (rows=%lld k=%lld nids=%lld)", fn, (long long)rows,
                    (long long)k, (long long)nids);
    if (!mul_ok(rows, k, &we) || !mul_ok(nids, k, &oe))
        return fail(F16WM_EINVAL, "%s: size too large", fn);
    if ((we > 0 && !w) || (nids > 0 && !ids) || (oe > 0 && !out))
        return fail(F16WM_EINVAL, "%s: null pointer for a non-empty array", fn);
    if (!aligned(w, 2) || !aligned(ids, 8) || !aligned(out, 4))
        return fail(F16WM_EINVAL, "%s: misaligned pointer", fn);
    const Span so = span(out, oe * 4);
    if (overlap(so, span(w, we * 2)) || overlap(so, span(ids, nids * 8)))
        return fail(F16WM_EINVAL, "%s: output overlaps an input", fn);
    if (nids == 0 || k == 0) return ok();
    if (int rc = check_device(fn)) return rc;
    return launched(fn, f16wm::launch_get_rows(w, rows, k, ids, nids, out, (hipStream_t)stream));
}

int f16wm_mat_vec(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, float *out,
                  void *stream)
{
    return mat_vec_impl("f16wm_mat_vec", w, rows, k, a, false, out, stream);
}

int f16wm_mat_vec_f32(const uint16_t *w, int64_t rows, int64_t k, const float *x, float *out,
                      void *stream)
{
    return mat_vec_impl("f16wm_mat_vec_f32", w, rows, k, x, true, out, stream);
}

int f16wm_mat_vec_multi(const f16wm_mat *mats, int32_t count, int64_t k, const uint16_t *a,
                        void *stream)
{
    return mat_vec_multi_impl("f16wm_mat_vec_multi", mats, count, k, a, false, stream);
}

int f16wm_mat_vec_multi_f32(const f16wm_mat *mats, int32_t count, int64_t k, const float *x,
                            void *stream)
{
    return mat_vec_multi_impl("f16wm_mat_vec_multi_f32", mats, count, k, x, true, stream);
}

int f16wm_mat_mul(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                  float *out, void *stream)
{
    const f16wm_mat m = {w, rows, out};
    return mat_mul_impl("f16wm_mat_mul", &m, 1, k, a, false, n, false, stream);
}

int f16wm_mat_mul_f32(const uint16_t *w, int64_t rows, int64_t k, const float *x, int64_t n, float *out,
                      void *stream)
{
    const f16wm_mat m = {w, rows, out};
    return mat_mul_impl("f16wm_mat_mul_f32", &m, 1, k, x, true, n, false, stream);
}

int f16wm_mat_mul_multi(const f16wm_mat *mats, int32_t count, int64_t k, const uint16_t *a, int64_t n,
                        void *stream)
{
    return mat_mul_impl("f16wm_mat_mul_multi", mats, count, k, a, false, n, false, stream);
}

int f16wm_mat_mul_multi_f32(const f16wm_mat *mats, int32_t count, int64_t k, const float *x, int64_t n,
                            void *stream)
{
    return mat_mul_impl("f16wm_mat_mul_multi_f32", mats, count, k, x, true, n, false, stream);
}

int f16wm_mat_mul_mfma(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                       float *out, void *stream)
{
    const f16wm_mat m = {w, rows, out};
    return mat_mul_impl("f16wm_mat_mul_mfma", &m, 1, k, a, false, n, true, stream);
}

int f16wm_mat_mul_mfma_multi(const f16wm_mat *mats, int32_t count, int64_t k, const uint16_t *a,
                             int64_t n, void *stream)
{
    return mat_mul_impl("f16wm_mat_mul_mfma_multi", mats, count, k, a, false, n, true, stream);
}

int f16wm_mat_mul_out(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n, int32_t mode,
                      float *out, void *stream)
{
    const char *fn = "f16wm_mat_mul_out";
    if (mode != F16WM_OUT_NONE && mode != F16WM_OUT_LAST && mode != F16WM_OUT_ALL)
        return fail(F16WM_EINVAL, "%s: mode %d is not none (0), last (1) or all (2)", fn, (int)mode);
    if (rows < 0 || k < 0 || n < 0)
        return fail(F16WM_EINVAL, "%s: negative size (rows=%lld k=%lld n=%lld)", fn, (long long)rows,
                    (long long)k, (long long)n);
    if (mode == F16WM_OUT_NONE) return ok();
    if (mode == F16WM_OUT_ALL) {
        const f16wm_mat m = {w, rows, out};
        return mat_mul_impl(fn, &m, 1, k, a, false, n, false, stream);
    }
    if (n < 1) return fail(F16WM_EINVAL, "%s: the last column of an empty micro-batch", fn);
    int64_t off;
    if (!mul_ok(n - 1, k, &off)) return fail(F16WM_EINVAL, "%s: size too large", fn);
    if (k > 0 && !a) return fail(F16WM_EINVAL, "%s: null activation", fn);
    // one column: the vec_dot order of f16wm_mat_vec
    return mat_vec_impl(fn, w, rows, k, a ? a + off : a, false, out, stream);
}

int f16wm_mat_vec_table(const f16wm_gemv *prods, int32_t count, void *stream)
{
    const char *fn = "f16wm_mat_vec_table";
    if (count < 0 || count > F16WM_MAX_TABLE)
        return fail(F16WM_EINVAL, "%s: count %d outside 0..%d", fn, (int)count, F16WM_MAX_TABLE);
    if (count == 0) return ok();
    if (!prods) return fail(F16WM_EINVAL, "%s: null table", fn);
    // Every product as f16wm_mat_vec checks it; then outputs pairwise
    // disjoint, and disjoint from every weight and column (sorted sweep).
    std::vector<Span> outs, ins;
    outs.reserve(count);
    ins.reserve(2 * (size_t)count);
    for (int p = 0; p < count; p++) {
        const f16wm_gemv &g = prods[p];
        char name[64];
        snprintf(name, sizeof name, "%s[%d]", fn, p);
        if (g.a_f32 != 0 && g.a_f32 != 1) return fail(F16WM_EINVAL, "%s: a_f32 is %d, not 0 or 1", name, (int)g.a_f32);
        const int esz = g.a_f32 ? 4 : 2;
        int64_t we, ae, oe;
        if (int rc = check_product(name, g.w, g.rows, g.k, g.a, esz, 1, g.out, &we, &ae, &oe)) return rc;
        if (oe > 0) outs.push_back(span(g.out, oe * 4));
        if (oe > 0 && we > 0) ins.push_back(span(g.w, we * 2));
        if (oe > 0 && ae > 0) ins.push_back(span(g.a, ae * esz));
    }
    std::sort(outs.begin(), outs.end(), [](const Span &x, const Span &y) { return x.lo < y.lo; });
    for (size_t i = 1; i < outs.size(); i++)
        if (outs[i].lo < outs[i - 1].hi) return fail(F16WM_EINVAL, "%s: two outputs overlap", fn);
    for (const Span &in : ins) {
        // the output with the largest start below the input's end is the only
        // one that can overlap it (outputs are disjoint and sorted)
        auto it = std::lower_bound(outs.begin(), outs.end(), in.hi,
                                   [](const Span &o, uintptr_t hi) { return o.lo < hi; });
        if (it != outs.begin() && std::prev(it)->hi > in.lo)
            return fail(F16WM_EINVAL, "%s: an output overlaps a weight or column", fn);
    }
    if (outs.empty()) return ok();
    if (int rc = check_device(fn)) return rc;

    // Kernel classes: [direct? 1 : 0][f32 column? 1 : 0]; products that take
    // no vectorised kernel launch one by one.
    std::vector<int> cls[2][2];
    for (int p = 0; p < count; p++) {
        const f16wm_gemv &g = prods[p];
        if (g.rows == 0) continue;
        const bool vec8 = g.k % 8 == 0 && aligned(g.w, 16) && aligned(g.a, 16) && g.rows <= 0x7fffffff &&
                          16 * 2 * g.k + 65536 <= 0x7fff0000;
        if (!vec8) {
            f16wm::RowTable t = {};
            t.count = 1;
            t.w[0] = g.w;
            t.out[0] = g.out;
            t.row0[1] = g.rows;
            const bool v8 = g.k % 8 == 0 && aligned(g.w, 16) && aligned(g.a, 16);
            const hipError_t e = f16wm::launch_vec_dot(t, g.k, g.a, g.a_f32 != 0, 1, v8, (hipStream_t)stream);
            if (e != hipSuccess) return launched(fn, e);
            continue;
        }
        cls[g.k <= f16wm::kDirectMaxKTable ? 1 : 0][g.a_f32 ? 1 : 0].push_back(p);
    }
    for (int d = 0; d < 2; d++)
        for (int f = 0; f < 2; f++) {
            std::vector<int> &v = cls[d][f];
            // longest rows first, so the blocks that take longest start first
            std::stable_sort(v.begin(), v.end(), [&](int x, int y) { return prods[x].k > prods[y].k; });
            // Chunks of at most kTableChunk products and 2^31 - 1 row tiles
            // (the grid's limit; a product has at most 2^27 tiles of 16 rows).
            const int64_t per = d == 1 ? f16wm::kTableRowsDirect : f16wm::kTableRowsLds;
            size_t i = 0;
            while (i < v.size()) {
                f16wm::ProdTable t = {};
                int64_t tiles = 0;
                while (i < v.size() && t.count < f16wm::kTableChunk) {
                    const f16wm_gemv &g = prods[v[i]];
                    const int64_t pt = (g.rows + per - 1) / per;
                    if (t.count > 0 && tiles + pt > 0x7fffffff) break;
                    tiles += pt;
                    t.w[t.count] = g.w;
                    t.a[t.count] = g.a;
                    t.out[t.count] = g.out;
                    t.rows[t.count] = (int32_t)g.rows;
                    t.k[t.count] = (int32_t)g.k;
                    t.count++;
                    i++;
                }
                const hipError_t e = f16wm::launch_vec_dot_table(t, d == 1, f == 1, (hipStream_t)stream);
                if (e != hipSuccess) return launched(fn, e);
            }
        }
    return ok();
}

int f16wm_kq(const uint16_t *kc, int64_t n_kv, int64_t n_kv_head, int64_t d, const uint16_t *q, int64_t n_head,
             float *out, void *stream)
{
    const char *fn = "f16wm_kq";
    if (n_kv < 0 || n_kv_head < 0 || d < 0 || n_head < 0)
        return fail(F16WM_EINVAL, "%s: negative size", fn);
    if (n_kv_head == 0 || n_head % n_kv_head != 0)
        return fail(F16WM_EINVAL, "%s: n_head (%lld) must be a multiple of n_kv_head (%lld) > 0", fn,
                    (long long)n_head, (long long)n_kv_head);
    if (n_kv_head > 65535) return fail(F16WM_EUNSUPPORTED, "%s: more than 65535 KV heads", fn);
    int64_t rows, ke, qe, oe;
    if (!mul_ok(n_kv, n_kv_head, &rows) || !mul_ok(rows, d, &ke) || !mul_ok(n_head, d, &qe) ||
        !mul_ok(n_head, n_kv, &oe))
        return fail(F16WM_EINVAL, "%s: size too large", fn);
    if ((ke > 0 && !kc) || (qe > 0 && !q) || (oe > 0 && !out))
        return fail(F16WM_EINVAL, "%s: null pointer for a non-empty array", fn);
    if (!aligned(kc, 2) || !aligned(q, 2) || !aligned(out, 4))
        return fail(F16WM_EINVAL, "%s: misaligned pointer", fn);
    const Span so = span(out, oe * 4);
    if (overlap(so, span(kc, ke * 2)) || overlap(so, span(q, qe * 2)))
        return fail(F16WM_EINVAL, "%s: output overlaps an input", fn);
    if (oe == 0) return ok();
    if (int rc = check_device(fn)) return rc;
    const bool vec8 = d % 8 == 0 && aligned(kc, 16) && aligned(q, 16);
    return launched(fn, f16wm::launch_kq(kc, n_kv, n_kv_head, d, q, n_head, vec8, out, (hipStream_t)stream));
}

int f16wm_mad(uint16_t *acc, const uint16_t *v, const float *w, int64_t nvec, int64_t n, void *stream)
{
    const char *fn = "f16wm_mad";
    int64_t e;
    if (nvec < 0 || n < 0 || !mul_ok(nvec, n, &e)) return fail(F16WM_EINVAL, "%s: bad size", fn);
    if (e == 0) return ok();
    if (!acc || !v || !w) return fail(F16WM_EINVAL, "%s: null pointer", fn);
    if (!aligned(acc, 2) || !aligned(v, 2) || !aligned(w, 4)) return fail(F16WM_EINVAL, "%s: misaligned pointer", fn);
    if (overlap(span(acc, e * 2), span(v, e * 2)) || overlap(span(acc, e * 2), span(w, nvec * 4)))
        return fail(F16WM_EINVAL, "%s: acc overlaps an input", fn);
    if (int rc = check_device(fn)) return rc;
    const bool vec8 = n % 8 == 0 && aligned(acc, 16) && aligned(v, 16);
    return launched(fn, f16wm::launch_mad(acc, v, w, nvec, n, vec8, (hipStream_t)stream));
}

int f16wm_scale(uint16_t *acc, const float *s, int64_t nvec, int64_t n, void *stream)
{
    const char *fn = "f16wm_scale";
    int64_t e;
    if (nvec < 0 || n < 0 || !mul_ok(nvec, n, &e)) return fail(F16WM_EINVAL, "%s: bad size", fn);
    if (e == 0) return ok();
    if (!acc || !s) return fail(F16WM_EINVAL, "%s: null pointer", fn);
    if (!aligned(acc, 2) || !aligned(s, 4)) return fail(F16WM_EINVAL, "%s: misaligned pointer", fn);
    if (overlap(span(acc, e * 2), span(s, nvec * 4))) return fail(F16WM_EINVAL, "%s: acc overlaps s", fn);
    if (int rc = check_device(fn)) return rc;
    const bool vec8 = n % 8 == 0 && aligned(acc, 16);
    return launched(fn, f16wm::launch_scale(acc, s, nvec, n, vec8, (hipStream_t)stream));
}

}  // extern "C"
