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
// Tiling: a block computes BM columns x BN rows as GM x GN waves (2 x 2 by
// default); each wave owns (BM/GM) x (BN/GN) = TM x TN MFMA tiles of 32 x 32,
// and each 16-byte LDS fragment it reads feeds TN (activation) or TM
// (weight) MFMAs: 64 x 128 per wave in the 256 x 256 tiles (eight waves, 128
// accumulators each), 64 x 64 or 64 x 32 in the smaller ones.  Block b runs
// on XCD b % 8; tiles are handed out so each XCD walks a contiguous range,
// and consecutive tiles share one weight-row block, so its weights are read
// from HBM once and re-read from that XCD's L2.
//
// Two kernels: mfma_fast (k % 64 == 0) stages k 64 at a time with direct
// global-to-LDS loads (see there); mfma_generic (any k % 8 == 0) stages k 32
// at a time through registers into LDS rows padded to 80 bytes (a stride that
// puts the 16 rows of one LDS read phase in 16 different bank groups), with
// the loads of the next three stages in flight.
//
// What bounds it: on this GPU the matrix cores alone, fed random f16
// operands, sustain about 1.66 PFLOP/s (the clock drops to about 1.7 GHz at
// the board's power limit); the 8B-shaped n = 512 products reach roughly
// half of that, limited by keeping the operand stream from L2/HBM ahead of
// the matrix cores.
#include "buffer_rsrc.h"
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

// Fast path: k % 64 == 0.  Same MFMA and wave tiling as mfma_generic, fed
// by direct global-to-LDS loads:
//  - each operand tile is addressed through a buffer resource whose size
//    ends at the tile's last valid row: rows past the matrix read as zero
//    without a branch (their outputs are not stored);
//  - buffer_load_dwordx4 with the lds bit writes a wave's 64 x 16 bytes to
//    M0 + 16 * lane in LDS, with no trip through VGPRs and no ds_write: lane
//    l of a load covers LDS row (l / 8) of its 8-row group and 16-byte slot
//    l % 8, and fetches the global chunk that belongs in that slot, chunk =
//    slot ^ ((row / 2) % 8).  That XOR swizzle keeps the 16-rows-per-phase
//    fragment reads free of bank conflicts (128-byte LDS rows, unpadded);
//  - k is staged 64 at a time through NBUF LDS buffers: while stage s is
//    multiplied, stages s + 1 .. s + NBUF - 1 are in flight; a wave waits
//    for its own loads of stage s (vmcnt) and a plain s_barrier makes every
//    wave's loads visible and frees the buffer the next loads overwrite.
//    The loads of the stage that refills it are issued a quarter before
//    each of the four 16-deep k steps, not all at once after the barrier:
//    a burst of every wave's loads fills the texture-address queue and
//    stalls the waves' MFMA issue behind it (5-12 % slower per shape).
//    Launches with fewer 128 x 128 tiles than CUs (q/k/v, o, down at
//    n = 512) are bound by that wait: one memory round trip per stage
//    unless several stages are in flight, so they use NBUF = 4 (one block
//    per CU), and 128 x 64 tiles when 128 x 128 would fill at most half the
//    CUs; the others use NBUF = 2.
// Measured on this GPU against a register-staged version of the same tiling
// (three stages in flight through VGPRs, ds_write into LDS): 5-15 % faster,
// 72 instead of 186 VGPRs, no LDS data-FIFO stalls.  The 256 x 256 tiles run
// as 4 x 2 waves of 64 x 128 (two waves per SIMD): with one wave per SIMD the
// LDS round trips of the fragment reads were exposed (one 4-wave block per CU
// reaches about half the LDS read bandwidth two blocks reach); eight waves
// read 1.5 times the fragment bytes per MFMA and were 12-15 % faster.
constexpr int kFKS = 64;   // k per stage

typedef __attribute__((address_space(3))) void lds_void;

template <int BM, int BN, int NBUF, int GM = 2, int GN = 2>
__global__ __launch_bounds__(64 * GM * GN) void mfma_fast(GemmTable g, int64_t k, const uint16_t *__restrict__ a,
                                                          int64_t n, int nct)
{
    constexpr int NW = GM * GN;                   // waves: GM over the columns, GN over the rows
    constexpr int WM = BM / GM, WN = BN / GN;     // wave tile
    constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 MFMA tiles per wave
    constexpr int ROWB = kFKS * 2;                // bytes per LDS row (8 chunks)
    constexpr int STAGEB = (BM + BN) * ROWB;      // bytes per stage: [A rows | W rows]
    constexpr int LA = BM / (8 * NW), LW = BN / (8 * NW);   // 8-row loads per wave per stage
    constexpr int PAST_END = 0x7ffffff0;          // an offset past every tile: reads zero
    __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * STAGEB];

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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / GN, wn = wave % GN;
    const int lr = lane & 31;
    const int hi = lane >> 5;

    const int64_t arows = n - c0 < BM ? n - c0 : BM;
    const int64_t wrows = rows - r0 < BN ? rows - r0 : BN;
    const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(a + c0 * k, arows * k * 2);
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(w + r0 * k, wrows * k * 2);

    // Load j < LA of this wave fills activation rows (wave * LA + j) * 8 .. +8
    // of a stage, load LA + j weight rows (wave * LW + j) * 8 .. +8.  Byte
    // offsets of stage 0; stage s adds 128 * s.
    int voff[LA + LW];
#pragma unroll
    for (int j = 0; j < LA + LW; j++) {
        const int trow = (j < LA ? wave * LA + j : wave * LW + j - LA) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ ((trow >> 1) & 7);
        voff[j] = (int)(trow * k * 2 + chunk * 16);
    }
    const int64_t nstages = k / kFKS;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    // Stage s goes to LDS buffer s % NBUF; this issues loads j0 .. j1 - 1 of
    // this wave's LA + LW.  Every stage issues the same loads (a stage past
    // the last reads zero and moves no data), so the waits below can count
    // them.
    auto issue = [&](int64_t s, int j0, int j1) {
        unsigned char *buf = smem + (int)(s % NBUF) * STAGEB;
        const bool live = s < nstages;
        const int so = (int)(s * ROWB);
#pragma unroll
        for (int j = 0; j < LA + LW; j++) {
            if (j < j0 || j >= j1) continue;
            const int row0 = j < LA ? (wave * LA + j) * 8 : BM + (wave * LW + j - LA) * 8;
            lds_void *dst = (lds_void *)(buf + row0 * ROWB);
            const int off = live ? voff[j] + so : PAST_END;
            if (j < LA)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, off, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, off, 0, 0, 0);
        }
    };
    // Fragment rows of this lane: wm*WM + i*32 + lr (activations) and
    // BM + wn*WN + j*32 + lr (weights); their swizzle is (lr >> 1) & 7.
    const int sw = (lr >> 1) & 7;
    // Multiplies stage s; the loads of stage s + NBUF - 1 are issued a
    // quarter at a time, one quarter before each 16-deep k step.
    constexpr int NL = LA + LW, NKK = kFKS / 16;
    auto compute = [&](int64_t s) {
        const unsigned char *base = smem + (int)(s % NBUF) * STAGEB;
        const unsigned char *abase = base + (wm * WM + lr) * ROWB;
        const unsigned char *wbase = base + (BM + wn * WN + lr) * ROWB;
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) {
            issue(s + NBUF - 1, kk * NL / NKK, (kk + 1) * NL / NKK);
            const int ch = 16 * ((2 * kk + hi) ^ sw);
            // let the scheduler interleave the next fragment reads with the MFMAs
            __builtin_amdgcn_iglp_opt(0);
            half8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[i] = *reinterpret_cast<const half8 *>(abase + i * 32 * ROWB + ch);
#pragma unroll
            for (int j = 0; j < TN; j++)
                bf[j] = *reinterpret_cast<const half8 *>(wbase + j * 32 * ROWB + ch);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    };

    // vmcnt(N) with N = the loads of the NBUF - 2 younger stages; expcnt and
    // lgkmcnt untouched (simm16: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
    // vmcnt[5:4] << 14).
    constexpr int YOUNG = (NBUF - 2) * (LA + LW);
    static_assert(YOUNG < 64, "vmcnt range");
    constexpr int WAIT = (YOUNG & 15) | 0x0F70 | ((YOUNG >> 4) << 14);
#pragma unroll
    for (int s = 0; s < NBUF - 1; s++) issue(s, 0, NL);
    for (int64_t s = 0; s < nstages; s++) {
        // This wave's loads of stage s are in LDS; the barrier makes every
        // wave's loads visible and guarantees stage s - 1 (whose buffer the
        // loads issued during compute(s) fill) is done.  A plain s_barrier:
        // a compiler fence would also wait for the younger stages.
        __builtin_amdgcn_s_waitcnt(WAIT);
        asm volatile("s_barrier" ::: "memory");
        compute(s);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // the zero loads past the end have landed

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

// Tile offsets of every matrix for BM activation columns x BN weight rows
// per tile; false past grid.x.
bool fill_tiles(GemmTable &g, int64_t n, int BM, int BN, int64_t *nct_out)
{
    const int64_t nct = (n + BM - 1) / BM;
    int64_t tiles = 0;
    for (int i = 0; i < g.count; i++) {
        g.tile0[i] = (int32_t)tiles;
        tiles += (g.rows[i] + BN - 1) / BN * nct;
        if (tiles > 0x7fffffff) return false;
    }
    g.tile0[g.count] = (int32_t)tiles;
    *nct_out = nct;
    return true;
}

}  // namespace

hipError_t launch_mfma(GemmTable g, int64_t k, const uint16_t *a, int64_t n, hipStream_t stream)
{
    // Tile size, measured on the 8B-shaped products at n = 512: 256 x 256
    // tiles (one block per CU, eight waves) once there are at least 192 of
    // them (the logits and the grouped gate/up product); 128 x 128 tiles (two
    // blocks per CU) below that, where 256-tiles would leave CUs idle, with
    // four LDS stages when even the 128-tiles are fewer than the CUs (q/k/v),
    // and 128 x 64 tiles with four stages when they would fill at most half
    // of the CUs (o, down).  The fast kernel needs
    // k % 64 == 0 and 32-bit byte offsets inside one 256-row tile.
    int64_t big = 0;
    for (int i = 0; i < g.count; i++) big += ((g.rows[i] + 255) / 256) * ((n + 255) / 256);
    const bool fast = k % kFKS == 0 && k > 0 && 256 * k * 2 < ((int64_t)1 << 31);
    const int B = fast && big >= 192 ? 256 : 128;
    int64_t nct = 0;
    if (!fill_tiles(g, n, B, B, &nct)) return hipErrorInvalidConfiguration;
    int64_t tiles = g.tile0[g.count];
    if (fast && B == 128 && tiles <= 128) {
        // at most half the CUs would get a 128 x 128 tile (o, down at
        // n = 512): 128 columns x 64 rows per tile doubles the blocks
        if (!fill_tiles(g, n, 128, 64, &nct)) return hipErrorInvalidConfiguration;
        tiles = g.tile0[g.count];
        mfma_fast<128, 64, 4><<<dim3((uint32_t)tiles), dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
        return hipGetLastError();
    }
    const dim3 grid((uint32_t)tiles);
    if (!fast)
        mfma_generic<128, 128><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    else if (B == 256)
        mfma_fast<256, 256, 2, 4, 2><<<grid, dim3(64 * 4 * 2), 0, stream>>>(g, k, a, n, (int)nct);
    else if (tiles < 256)   // fewer tiles than CUs: more stages in flight per tile
        mfma_fast<128, 128, 4><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    else
        mfma_fast<128, 128, 2><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    return hipGetLastError();
}

}  // namespace f16wm
