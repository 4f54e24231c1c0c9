// fp16 matrix-core product for prefill micro-batches (approximate fast path).
//
// The same product and output layout as the exact paths, out[c*rows + r] =
// sum_i W[r][i] * A[c][i], computed by v_mfma_f32_32x32x16_f16 (f16 inputs,
// f32 accumulation).  Its summation order is the matrix core's, so it is not
// either ggml order; it is judged against a binary64 sum instead.  bankML page
// "bankML/forward.rs" (Technical usage): prompts are processed in
// micro-batches of up to 512 columns, which makes this a dense contraction.
//
// Layout: the MFMA's A operand is the activation block (M = columns c), its B
// operand the weight block (N = rows r), both k-contiguous, so each lane
// fetches 8 consecutive k values of one row with a 16-byte LDS read, and the
// 32 lanes holding one output register cover 32 consecutive r: the stores to
// out[c*rows + r] are coalesced.
//
// 256-thread block, 128 (c) x 128 (r) tile, 2 x 2 waves of 64 x 64 (2 x 2 MFMA
// 32x32 tiles each), k staged 32 at a time through padded LDS rows (80-byte
// stride: conflict-free 16-byte reads), next stage prefetched into registers.
#include "kernels.h"

namespace f16wm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMB = 128;         // activation columns per block
constexpr int kNB = 128;         // weight rows per block
constexpr int kKB = 32;          // k per stage
constexpr int kLD = kKB + 8;     // padded LDS row, in halves

__global__ __launch_bounds__(256) void mfma_kernel(const uint16_t *__restrict__ w, int64_t rows,
                                                   int64_t k, const uint16_t *__restrict__ a,
                                                   int64_t n, float *__restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[kMB][kLD];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[kNB][kLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;        // columns wm*64 .. +63 of the tile
    const int wn = wave & 1;         // rows    wn*64 .. +63 of the tile
    const int64_t r0 = (int64_t)blockIdx.x * kNB;
    const int64_t c0 = (int64_t)blockIdx.y * kMB;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    u32x4 areg[2], wreg[2];
#define F16WM_MFMA_FETCH(K0)                                                                  \
    do {                                                                                      \
        _Pragma("unroll") for (int p = 0; p < 2; p++) {                                       \
            const int idx = tid + 256 * p;                                                    \
            const int row = idx >> 2, kv = idx & 3;                                           \
            const int64_t gk = (K0) + kv * 8;                                                 \
            const int64_t gc = c0 + row, gr = r0 + row;                                       \
            u32x4 av = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};                               \
            if (gc < n && gk < k) av = *reinterpret_cast<const u32x4 *>(a + gc * k + gk);     \
            if (gr < rows && gk < k) wv = *reinterpret_cast<const u32x4 *>(w + gr * k + gk);  \
            areg[p] = av;                                                                     \
            wreg[p] = wv;                                                                     \
        }                                                                                     \
    } while (0)

    const int lr = lane & 31;         // operand row within a 32-row block
    const int lk = (lane >> 5) * 8;   // k offset of the lane's 8 values

    if (k > 0) F16WM_MFMA_FETCH(0);
    for (int64_t k0 = 0; k0 < k; k0 += kKB) {
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const int idx = tid + 256 * p;
            const int row = idx >> 2, kv = idx & 3;
            *reinterpret_cast<u32x4 *>(&As[row][kv * 8]) = areg[p];
            *reinterpret_cast<u32x4 *>(&Ws[row][kv * 8]) = wreg[p];
        }
        __syncthreads();
        if (k0 + kKB < k) F16WM_MFMA_FETCH(k0 + kKB);
#pragma unroll
        for (int kk = 0; kk < kKB; kk += 16) {
            half8 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; i++)
                af[i] = *reinterpret_cast<const half8 *>(&As[wm * 64 + i * 32 + lr][kk + lk]);
#pragma unroll
            for (int j = 0; j < 2; j++)
                bf[j] = *reinterpret_cast<const half8 *>(&Ws[wn * 64 + j * 32 + lr][kk + lk]);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }

    // D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8).
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t r = r0 + wn * 64 + j * 32 + lr;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t c = c0 + wm * 64 + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
                if (r < rows && c < n) out[c * rows + r] = acc[i][j][v];
            }
        }
#undef F16WM_MFMA_FETCH
}

}  // namespace

hipError_t launch_mfma(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                       float *out, hipStream_t stream)
{
    const int64_t bx = (rows + kNB - 1) / kNB;
    const int64_t by_all = (n + kMB - 1) / kMB;
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    for (int64_t b0 = 0; b0 < by_all; b0 += 65535) {
        const int64_t by = by_all - b0 < 65535 ? by_all - b0 : 65535;
        const int64_t c0 = b0 * kMB;
        const int64_t nc = n - c0 < by * kMB ? n - c0 : by * kMB;
        mfma_kernel<<<dim3((uint32_t)bx, (uint32_t)by), dim3(256), 0, stream>>>(
            w, rows, k, a + c0 * k, nc, out + c0 * rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace f16wm
