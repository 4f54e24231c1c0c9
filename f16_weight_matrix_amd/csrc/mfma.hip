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
// Tiling: a 256-thread block computes BM columns x BN rows as 2 x 2 waves;
// each wave owns (BM/2) x (BN/2) = TM x TN MFMA tiles of 32 x 32.  With
// 128 x 128 per wave (16 tiles, 256 accumulators in AGPRs) every 16-byte LDS
// fragment feeds four MFMAs, which keeps LDS reads at half the LDS bandwidth.
// k is staged 32 at a time through two LDS buffers with 80-byte rows (a
// stride that puts the 16 rows of one LDS read phase in 16 different bank
// groups); the global loads of the next three stages are in flight during
// the MFMAs (weights come from HBM with microseconds of latency).
// Block b runs on XCD b % 8; tiles are handed out so each XCD walks a
// contiguous range, and consecutive tiles share one weight-row block, so its
// weights are read from HBM once and re-read from that XCD's L2.
#include "kernels.h"

namespace f16wm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKS = 32;          // k per stage
constexpr int kLD = kKS + 8;     // padded LDS row, in halves (80 bytes)

template <int BM, int BN>
__global__ __launch_bounds__(256) void mfma_generic(GemmTable g, int64_t k, const uint16_t *__restrict__ a,
                                                    int64_t n, int nct)
{
    constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
    constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 MFMA tiles per wave
    constexpr int AUPT = BM * kKS / 8 / 256;      // 16-byte activation units per thread
    constexpr int WUPT = BN * kKS / 8 / 256;      // 16-byte weight units per thread
    static_assert(AUPT >= 1 && WUPT >= 1, "tile too small for 256 threads");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][kLD];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN][kLD];

    // XCD-aware tile index (blocks are dispatched round-robin over 8 XCDs),
    // then this tile's matrix.
    int mi, rt, ct;
    gemm_tile(g, xcd_tile(blockIdx.x, g.tile0[g.count]), nct, mi, rt, ct);
    const uint16_t *__restrict__ w = g.w[mi];
    const int64_t rows = g.rows[mi];
    float *__restrict__ out = g.out[mi];
    const int64_t r0 = (int64_t)rt * BN;
    const int64_t c0 = (int64_t)ct * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;         // columns wm*WM .. of the tile
    const int wn = wave & 1;          // rows    wn*WN .. of the tile
    const int lr = lane & 31;         // operand row within a 32-row block
    const int lk = (lane >> 5) * 8;   // k offset of the lane's 8 values

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    // Global loads are issued for stage s + 3 while stage s computes; stage s
    // waits in register set s % 3 until it is copied into LDS buffer s % 2.
    // Every load is issued unconditionally from a clamped, valid address and
    // out-of-range values are replaced by zero when copied to LDS, so the loop
    // has no branches and the compiler can wait for exactly the oldest stage.
    // The stage count is rounded up to a multiple of 3; the extra stages are
    // all zeros and add nothing.
    u32x4 areg[3][AUPT], wreg[3][WUPT];
    const int64_t nstages = (k + kKS - 1) / kKS;
    const int64_t last_k = k >= 8 ? k - 8 : 0;
    auto fetch = [&](int64_t s, int set) {
        const int64_t k0 = s * kKS;
#pragma unroll
        for (int p = 0; p < AUPT; p++) {
            const int idx = p * 256 + tid;
            const int64_t gk = k0 + (idx & 3) * 8, gc = c0 + (idx >> 2);
            const int64_t ck = gk < k ? gk : last_k, cc = gc < n ? gc : n - 1;
            areg[set][p] = *reinterpret_cast<const u32x4 *>(a + cc * k + ck);
        }
#pragma unroll
        for (int p = 0; p < WUPT; p++) {
            const int idx = p * 256 + tid;
            const int64_t gk = k0 + (idx & 3) * 8, gr = r0 + (idx >> 2);
            const int64_t ck = gk < k ? gk : last_k, cr = gr < rows ? gr : rows - 1;
            wreg[set][p] = *reinterpret_cast<const u32x4 *>(w + cr * k + ck);
        }
    };
    auto stash = [&](int64_t s, int set, int buf) {
        const int64_t k0 = s * kKS;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int p = 0; p < AUPT; p++) {
            const int idx = p * 256 + tid;
            const bool ok = k0 + (idx & 3) * 8 < k && c0 + (idx >> 2) < n;
            *reinterpret_cast<u32x4 *>(&As[buf][idx >> 2][(idx & 3) * 8]) = ok ? areg[set][p] : zero;
        }
#pragma unroll
        for (int p = 0; p < WUPT; p++) {
            const int idx = p * 256 + tid;
            const bool ok = k0 + (idx & 3) * 8 < k && r0 + (idx >> 2) < rows;
            *reinterpret_cast<u32x4 *>(&Ws[buf][idx >> 2][(idx & 3) * 8]) = ok ? wreg[set][p] : zero;
        }
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < kKS; kk += 16) {
            half8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[i] = *reinterpret_cast<const half8 *>(&As[buf][wm * WM + i * 32 + lr][kk + lk]);
#pragma unroll
            for (int j = 0; j < TN; j++)
                bf[j] = *reinterpret_cast<const half8 *>(&Ws[buf][wn * WN + j * 32 + lr][kk + lk]);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    };

    if (nstages > 0) {
        const int64_t S = (nstages + 2) / 3 * 3;
        fetch(0, 0);
        fetch(1, 1);
        fetch(2, 2);
        stash(0, 0, 0);
        __syncthreads();
        for (int64_t s = 0; s < S; s += 3) {
            const int b0 = (int)(s & 1);     // LDS buffer of stage s
            fetch(s + 3, 0);
            compute(b0);
            stash(s + 1, 1, b0 ^ 1);
            __syncthreads();
            fetch(s + 4, 1);
            compute(b0 ^ 1);
            stash(s + 2, 2, b0);
            __syncthreads();
            fetch(s + 5, 2);
            compute(b0);
            stash(s + 3, 0, b0 ^ 1);
            __syncthreads();
        }
    }

    // D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8).
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t r = r0 + wn * WN + j * 32 + lr;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t c = c0 + wm * WM + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
                if (r < rows && c < n) out[c * rows + r] = acc[i][j][v];
            }
        }
}

// Fast path: k % 64 == 0.  Same tiling and MFMA order as mfma_generic, with
//  - buffer loads: each block addresses its activation and weight tiles
//    through buffer resources whose size ends at the tile's last valid row,
//    so rows past the matrix read as zero without a branch, and the prefetch
//    running past the last stage reads zero (offset past the resource end);
//  - 64-element k stages, two register sets (stages s+1 and s+2 in flight);
//  - unpadded 128-byte LDS rows with the 16-byte chunk index XORed by
//    (row / 2) % 8, which keeps both the row-wise stores and the 16-rows-per-
//    phase fragment reads free of bank conflicts.
constexpr int kFKS = 64;   // k per stage

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base, int64_t bytes)
{
    // raw buffer: stride 0, num_records = bytes, gfx9 dword3
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void mfma_fast(GemmTable g, int64_t k, const uint16_t *__restrict__ a,
                                                 int64_t n, int nct)
{
    constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
    constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 MFMA tiles per wave
    constexpr int AU = BM / 32;                   // activation units per thread per stage
    constexpr int WU = BN / 32;                   // weight units per thread per stage
    constexpr int ROWH = kFKS;                    // halves per LDS row (128 bytes)
    constexpr int BUFH = (BM + BN) * ROWH;        // halves per LDS buffer
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUFH];

    // XCD-aware tile index (blocks are dispatched round-robin over 8 XCDs),
    // then this tile's matrix.
    int mi, rt, ct;
    gemm_tile(g, xcd_tile(blockIdx.x, g.tile0[g.count]), nct, mi, rt, ct);
    const uint16_t *__restrict__ w = g.w[mi];
    const int64_t rows = g.rows[mi];
    float *__restrict__ out = g.out[mi];
    const int64_t r0 = (int64_t)rt * BN;
    const int64_t c0 = (int64_t)ct * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31;
    const int hi = lane >> 5;

    // Tile resources (bytes of the valid rows of this tile).
    const int64_t arows = n - c0 < BM ? n - c0 : BM;
    const int64_t wrows = rows - r0 < BN ? rows - r0 : BN;
    const __amdgpu_buffer_rsrc_t ar = tile_rsrc(a + c0 * k, arows * k * 2);
    const __amdgpu_buffer_rsrc_t wr = tile_rsrc(w + r0 * k, wrows * k * 2);
    // This thread's units: rows (tid >> 3) + 32 p, 16-byte chunk tid & 7.  All
    // of a load's offset is in the VGPR offset, which the buffer range check
    // covers; an offset at or past the resource size reads as zero.
    const int urow = tid >> 3, uch = tid & 7;
    const int voff = (int)(urow * k * 2 + uch * 16);
    const int rstride = (int)(32 * k * 2);          // bytes between p and p + 1
    const int past_end = 256 * (int)k * 2;          // >= every tile's resource size
    const int64_t nstages = k / kFKS;
    // LDS byte offsets of this thread's unit stores (row urow + 32 p, swizzled chunk)
    const int st_off = urow * (ROWH * 2) + 16 * (uch ^ ((urow >> 1) & 7));

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    u32x4 areg[2][AU], wreg[2][WU];
    auto fetch = [&](int64_t s, int set) {
        const bool live = s < nstages;
        const int so = (int)(s * kFKS * 2);
#pragma unroll
        for (int p = 0; p < AU; p++)
            areg[set][p] = __builtin_amdgcn_raw_buffer_load_b128(ar, live ? voff + p * rstride + so : past_end, 0, 0);
#pragma unroll
        for (int p = 0; p < WU; p++)
            wreg[set][p] = __builtin_amdgcn_raw_buffer_load_b128(wr, live ? voff + p * rstride + so : past_end, 0, 0);
    };
    auto stash = [&](int set, int buf) {
        unsigned char *base = reinterpret_cast<unsigned char *>(smem + buf * BUFH);
#pragma unroll
        for (int p = 0; p < AU; p++)
            *reinterpret_cast<u32x4 *>(base + st_off + p * 32 * ROWH * 2) = areg[set][p];
#pragma unroll
        for (int p = 0; p < WU; p++)
            *reinterpret_cast<u32x4 *>(base + BM * ROWH * 2 + st_off + p * 32 * ROWH * 2) = wreg[set][p];
    };
    // Fragment rows of this lane: wm*WM + i*32 + lr (activations) and
    // wn*WN + j*32 + lr (weights); all are lr modulo 16, so the swizzle is
    // the same (lr >> 1) & 7 for every fragment.
    const int sw = (lr >> 1) & 7;
    auto compute = [&](int buf) {
        const unsigned char *base = reinterpret_cast<const unsigned char *>(smem + buf * BUFH);
        const unsigned char *abase = base + (wm * WM + lr) * (ROWH * 2);
        const unsigned char *wbase = base + BM * ROWH * 2 + (wn * WN + lr) * (ROWH * 2);
#pragma unroll
        for (int kk = 0; kk < kFKS / 16; kk++) {
            const int ch = 16 * ((2 * kk + hi) ^ sw);
            // let the scheduler interleave the fragment reads with the MFMAs
            __builtin_amdgcn_iglp_opt(0);
            half8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[i] = *reinterpret_cast<const half8 *>(abase + i * 32 * ROWH * 2 + ch);
#pragma unroll
            for (int j = 0; j < TN; j++)
                bf[j] = *reinterpret_cast<const half8 *>(wbase + j * 32 * ROWH * 2 + ch);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    };

    // Stage s waits in register set s % 2 and is computed from LDS buffer s % 2.
    fetch(0, 0);
    fetch(1, 1);
    stash(0, 0);
    __syncthreads();
    for (int64_t s = 0; s < nstages; s += 2) {
        fetch(s + 2, 0);
        compute(0);
        stash(1, 1);
        __syncthreads();
        fetch(s + 3, 1);
        compute(1);
        stash(0, 0);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t r = r0 + wn * WN + j * 32 + lr;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t c = c0 + wm * WM + i * 32 + 8 * (v / 4) + 4 * hi + (v % 4);
                if (r < rows && c < n) out[c * rows + r] = acc[i][j][v];
            }
        }
}

// Tile offsets of every matrix for a B x B tiling; false past grid.x.
bool fill_tiles(GemmTable &g, int64_t n, int B, int64_t *nct_out)
{
    const int64_t nct = (n + B - 1) / B;
    int64_t tiles = 0;
    for (int i = 0; i < g.count; i++) {
        g.tile0[i] = (int32_t)tiles;
        tiles += (g.rows[i] + B - 1) / B * nct;
        if (tiles > 0x7fffffff) return false;
    }
    g.tile0[g.count] = (int32_t)tiles;
    *nct_out = nct;
    return true;
}

}  // namespace

hipError_t launch_mfma(GemmTable g, int64_t k, const uint16_t *a, int64_t n, hipStream_t stream)
{
    // 256 x 256 tiles when they still give at least one block per CU,
    // 128 x 128 otherwise.  The fast kernel needs k % 64 == 0 and 32-bit
    // byte offsets inside one 256-row tile.
    int64_t big = 0;
    for (int i = 0; i < g.count; i++) big += ((g.rows[i] + 255) / 256) * ((n + 255) / 256);
    const bool fast = k % kFKS == 0 && k > 0 && 256 * k * 2 < ((int64_t)1 << 31);
    const int B = fast && big >= 256 ? 256 : 128;
    int64_t nct = 0;
    if (!fill_tiles(g, n, B, &nct)) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)g.tile0[g.count]);
    if (!fast)
        mfma_generic<128, 128><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    else if (B == 256)
        mfma_fast<256, 256><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    else
        mfma_fast<128, 128><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    return hipGetLastError();
}

}  // namespace f16wm
