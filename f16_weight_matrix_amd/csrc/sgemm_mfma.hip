// tinyBLAS order on the fp32 matrix cores: the exact product for n >= 2
// columns when rows % 4 == 0 and k % 8 == 0.
//
// bankML f16 page, Design notes ("sgemm_dot" and "Blocking"): every output
// element is ONE chain of eight f32 lanes, lane l taking elements 8t + l in
// ascending t, each step an FMA; the element is then reduced
// ((l0 + l4) + (l2 + l6)) + ((l1 + l5) + (l3 + l7)).  Matrix products
// (mat_mul_par): out[c*rows + r].
//
// gfx950 design.  v_mfma_f32_32x32x1_2b_f32 computes, for two independent
// blocks, D[i][j] = C[i][j] + A[i] * B[j] over a 32 x 32 tile: one rank-1
// update per instruction, i.e. one chain step for 1024 elements of a block.
// On this GPU that update is the IEEE binary32 sum of C and the product,
// rounded to nearest even (an f16 x f16 product is exact in binary32, so
// this is the FMA step of the chain bit for bit; signed zeros, infinities,
// NaNs and subnormal accumulators behave as IEEE says).  So:
//  - block 0 of instruction p (p = 0..3) holds chain lane p and block 1 holds
//    chain lane p + 4: for step t the A operand is W[row][8t + p] in lanes
//    0..31 and W[row][8t + 4 + p] in lanes 32..63, the B operand the same
//    elements of the activation columns.  Each thread therefore needs four
//    consecutive values of its row (or column) per step: one 16-byte LDS
//    read once they are f32.
//  - The eight lanes of an element end in the same thread (instruction p,
//    registers v and v + 16), so the hsum is four in-thread adds in the
//    page's order, no shuffles.
//  - A 256-thread block computes 64 weight rows x 64 columns; each wave
//    one 32 x 32 tile x four instructions x 32 accumulators = 128
//    accumulators, and two blocks share a CU (two waves per SIMD, at most
//    256 registers each).  Per step a wave issues four MFMAs from two
//    16-byte LDS reads, read two steps ahead so their latency hides behind
//    the matrix core (one step ahead was 0.4-3 % slower per shape).
//    Measured against 64 x 128 blocks with one wave per
//    SIMD (32 x 64 per wave, 256 accumulators): 11 % faster on the 8B-shaped
//    set at n = 512 (126 instead of 113 TFLOP/s on the large products) and
//    34 % faster on the 135M-shaped set, whose small matrices then give
//    twice as many waves; the bits are the same.
//  - k is staged 64 at a time (8 chain steps) through two LDS buffers holding
//    the operands already widened to f32 (exactly, once per element and
//    block): widening inside the step loop would put 24 conversions between
//    every 16 MFMAs and keep the matrix core a quarter idle.
//  - Global loads run two stages ahead of their stash and three ahead of
//    their MFMAs: while stage st computes, stage st + 1's chunks (in one of
//    two register sets, one per stage parity) are widened and written to
//    the other buffer between the MFMAs, a few at a time, and each register
//    is refilled with its chunk of stage st + 3 (one stage of lead, with a
//    single register set, was 1-2 % slower on the large products and 20 %
//    on q/k/v, whose second round of blocks runs one block per CU).
//    Aligned operands use raw buffer loads whose resource covers only this
//    tile; an offset past its end reads zero, so rows past the matrix,
//    columns past n and chunks past k (k % 8 == 0: a chunk is all in or all
//    out) need no branch, and the loop waits on precise load counts.
//  - Zero chunks past k are harmless: the step C + 0 * 0 leaves every
//    accumulator unchanged because an accumulator starting at +0 never
//    becomes -0.  Rows past `rows` and columns past n are not stored.
//  - Blocks walk the output tiles in an XCD-aware order (block b runs on
//    XCD b % 8, each XCD takes a contiguous range of tiles, the column tiles
//    of one weight-row block are consecutive), so each weight row block is
//    read from HBM once and re-read from that XCD's L2.
//
// Launches with few 32 x 32 output tiles use tinyblas_lanes instead (below):
// one tile per block, its four instructions on four waves.
//
// Matrix-core bound: rows*n*k chain steps = 2*rows*n*k flops at the fp32
// MFMA rate.
#include "buffer_rsrc.h"
#include "f16_round.h"
#include "kernels.h"

#include <type_traits>

namespace f16wm {
namespace {

typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 64;                   // weight rows per block
constexpr int kBN = 64;                   // activation columns per block
constexpr int kKS = 64;                   // k per stage
constexpr int kSteps = kKS / 8;           // chain steps per stage
constexpr int kWG = kBM * 16 + 16;        // bytes of one (step, half) group, weights
constexpr int kXG = kBN * 16 + 16;        // bytes of one (step, half) group, activations
constexpr int kWBuf = 2 * kSteps * kWG;   // bytes of one weight buffer
constexpr int kXBuf = 2 * kSteps * kXG;   // bytes of one activation buffer
constexpr int kWPT = kBM * kSteps / 256;  // 16-byte weight chunks per thread
constexpr int kXPT = kBN * kSteps / 256;  // 16-byte activation chunks per thread
static_assert(kWPT * 256 == kBM * kSteps && kXPT * 256 == kBN * kSteps, "chunks must divide evenly");

template <bool kAligned>
__device__ __forceinline__ u32x4 load8(const uint16_t *p)
{
    if (kAligned) return *reinterpret_cast<const u32x4 *>(p);
    u32x4 v;
    v.x = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
    v.y = (uint32_t)p[2] | ((uint32_t)p[3] << 16);
    v.z = (uint32_t)p[4] | ((uint32_t)p[5] << 16);
    v.w = (uint32_t)p[6] | ((uint32_t)p[7] << 16);
    return v;
}

// Where a stage's chunks come from.  kBuf: 16-byte aligned operands and
// kBN * k * ESZ < 2^31 bytes, read with raw buffer loads whose resource covers
// just this tile's rows (or columns); an offset at or past the resource's
// end returns zero, so rows past the matrix, columns past n and chunks past
// k need no branch.  Otherwise plain loads guarded by the same conditions.
// kF32: the activation block holds f32 values (ESZ = 4 bytes), rounded to f16
// when a chunk is stashed; a chunk is then 32 bytes, kept raw as two
// 16-byte halves until the stash.  Otherwise f16 patterns (ESZ = 2), one
// 16-byte half.
template <bool kBuf, bool kF32>
struct Src {
    static constexpr int ESZ = kF32 ? 4 : 2;
    const uint16_t *w;
    const char *a;
    int64_t rows, n, k, row0, col0;
    __amdgpu_buffer_rsrc_t rw, rx;

    __device__ __forceinline__ Src(const uint16_t *w_, int64_t rows_, const void *a_, int64_t n_, int64_t k_,
                                   int64_t row0_, int64_t col0_)
        : w(w_), a(static_cast<const char *>(a_)), rows(rows_), n(n_), k(k_), row0(row0_), col0(col0_)
    {
        if constexpr (kBuf) {
            const int64_t wr = rows - row0 < kBM ? rows - row0 : kBM;
            const int64_t xr = n - col0 < kBN ? n - col0 : kBN;
            rw = buffer_rsrc(w + row0 * k, wr * k * 2);
            rx = buffer_rsrc(a + col0 * k * ESZ, xr * k * ESZ);
        }
    }

    // Byte offset of chunk (r, gk) in a tile resource of esz-byte elements; a
    // chunk past k gets bit 31 set, which puts it past the resource's end
    // (under 2^31 bytes).
    __device__ __forceinline__ uint32_t offset(int r, int64_t gk, int esz) const
    {
        return (uint32_t)((r * k + gk) * esz) | (gk < k ? 0u : 0x80000000u);
    }

    // chunk (r, elements gk .. gk + 7) of the weight tile
    __device__ __forceinline__ u32x4 wchunk(int r, int64_t gk) const
    {
        if constexpr (kBuf) {
            return __builtin_amdgcn_raw_buffer_load_b128(rw, (int)offset(r, gk, 2), 0, 0);
        } else {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row0 + r < rows && gk < k) v = load8<false>(w + (row0 + r) * k + gk);
            return v;
        }
    }
    // chunk (r, elements gk .. gk + 7) of the activation tile, raw
    __device__ __forceinline__ void xchunk(int r, int64_t gk, u32x4 (&x)[2]) const
    {
        if constexpr (kBuf) {
            const uint32_t off = offset(r, gk, ESZ);
            x[0] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
            if constexpr (kF32) x[1] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16), 0, 0);
        } else {
            const u32x4 z = {0u, 0u, 0u, 0u};
            x[0] = z;
            if constexpr (kF32) x[1] = z;
            if (col0 + r < n && gk < k) {
                if constexpr (kF32) {
                    const uint32_t *f = reinterpret_cast<const uint32_t *>(a) + (col0 + r) * k + gk;
                    x[0] = u32x4{f[0], f[1], f[2], f[3]};
                    x[1] = u32x4{f[4], f[5], f[6], f[7]};
                } else {
                    x[0] = load8<false>(reinterpret_cast<const uint16_t *>(a) + (col0 + r) * k + gk);
                }
            }
        }
    }
};

// Four activation values of a stashed chunk (elements 4 hf .. 4 hf + 3),
// widened to f32: the f16 patterns as they are, or f32 values rounded to f16
// first by the rounding every kernel shares (so the result equals
// f16wm_to_f16 followed by the f16 product).  Elements are copied out of the
// vectors before use: this clang miscompiles __builtin_bit_cast applied to a
// vector element in place.
__device__ __forceinline__ float widen_h(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

template <bool kF32>
__device__ __forceinline__ f32x4 act4(const u32x4 (&x)[2], int hf)
{
    if constexpr (kF32) {
        const u32x4 p = hf ? x[1] : x[0];
        const uint32_t e0 = p[0], e1 = p[1], e2 = p[2], e3 = p[3];
        return f32x4{widen_h(rne_f16(__uint_as_float(e0))), widen_h(rne_f16(__uint_as_float(e1))),
                     widen_h(rne_f16(__uint_as_float(e2))), widen_h(rne_f16(__uint_as_float(e3)))};
    } else {
        const half8 h = __builtin_bit_cast(half8, x[0]);
        return f32x4{(float)h[4 * hf], (float)h[4 * hf + 1], (float)h[4 * hf + 2], (float)h[4 * hf + 3]};
    }
}

// Global -> registers for the stage at k0.  Chunk c of a tile is row (or
// column) c / kSteps, elements 8 (c % kSteps) .. + 7 of the stage; zero past
// rows, n or k (k % 8 == 0: a chunk is all inside k or all outside).
template <bool kBuf, bool kF32>
__device__ __forceinline__ void fetch_stage(u32x4 (&wr)[kWPT], u32x4 (&xr)[kXPT][2], const Src<kBuf, kF32> &src,
                                            int64_t k0, int tid)
{
#pragma unroll
    for (int p = 0; p < kWPT; p++) {
        const int c = p * 256 + tid;
        wr[p] = src.wchunk(c / kSteps, k0 + 8 * (c % kSteps));
    }
#pragma unroll
    for (int p = 0; p < kXPT; p++) {
        const int c = p * 256 + tid;
        src.xchunk(c / kSteps, k0 + 8 * (c % kSteps), xr[p]);
    }
}

// Chunk j (weights first) of the stage at k0 into its register.
template <bool kBuf, bool kF32, int j>
__device__ __forceinline__ void fetch_chunk(u32x4 (&wr)[kWPT], u32x4 (&xr)[kXPT][2], const Src<kBuf, kF32> &src,
                                            int64_t k0, int tid)
{
    constexpr bool isw = j < kWPT;
    const int c = (isw ? j : j - kWPT) * 256 + tid;
    if constexpr (isw)
        wr[isw ? j : 0] = src.wchunk(c / kSteps, k0 + 8 * (c % kSteps));
    else
        src.xchunk(c / kSteps, k0 + 8 * (c % kSteps), xr[isw ? 0 : j - kWPT]);
}

// Registers -> LDS, widened exactly to f32 once here.  Entry (t, h, row) is
// 16 bytes: elements 8t + 4h .. + 3 of one row, the four values a thread
// feeds to the four instructions of step t; rows are contiguous, so a
// half-wave reads 512 contiguous bytes, and the 16-byte pad per group puts
// the eight steps of one row, written by eight neighbouring lanes, in eight
// different bank groups.  Half q (0 .. kHalves - 1) is one entry: chunk q / 2
// (weights first), elements 4 (q % 2) .. + 3.
constexpr int kHalves = 2 * (kWPT + kXPT);

template <bool kF32, int q>
__device__ __forceinline__ void stash_half(char *wl, char *xl, const u32x4 (&wr)[kWPT],
                                           const u32x4 (&xr)[kXPT][2], int tid)
{
    constexpr int cq = q / 2, hf = q % 2;
    constexpr bool isw = cq < kWPT;
    const int c = (isw ? cq : cq - kWPT) * 256 + tid;
    const int r = c / kSteps, t = c % kSteps;
    f32x4 v;
    if constexpr (isw) {
        const half8 x = __builtin_bit_cast(half8, wr[isw ? cq : 0]);
        v = f32x4{(float)x[4 * hf], (float)x[4 * hf + 1], (float)x[4 * hf + 2], (float)x[4 * hf + 3]};
    } else {
        v = act4<kF32>(xr[isw ? 0 : cq - kWPT], hf);
    }
    char *grp = isw ? wl : xl;
    const int gsize = isw ? kWG : kXG;
    *reinterpret_cast<f32x4 *>(grp + (2 * t + hf) * gsize + r * 16) = v;
}

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <bool kF32>
__device__ __forceinline__ void stash_stage(char *wl, char *xl, const u32x4 (&wr)[kWPT],
                                            const u32x4 (&xr)[kXPT][2], int tid)
{
    static_for<0, kHalves>([&](auto qc) { stash_half<kF32, decltype(qc)::value>(wl, xl, wr, xr, tid); });
}

// The stage's 4 * kSteps MFMA slots (step t, instruction p) share out the
// kHalves stash entries evenly: entry q goes after slot q * 4 kSteps / kHalves.
template <int t, int p>
struct Slot {
    static constexpr int kFlat = 4 * t + p;
    static constexpr int kQ = (kFlat * kHalves + 4 * kSteps - 1) / (4 * kSteps);
    static constexpr bool kUsed = kQ < kHalves && kQ * 4 * kSteps / kHalves == kFlat;
};
static_assert(kHalves <= 4 * kSteps, "more stash entries than MFMA slots");

// Step t's operands: lanes 4h .. 4h + 3 of the thread's weight row and of
// its activation column.
__device__ __forceinline__ void read_step(const char *wl, const char *xl, int t, int h, int wrow, int xcol,
                                          f32x4 &wa, f32x4 &x0)
{
    wa = *reinterpret_cast<const f32x4 *>(wl + (2 * t + h) * kWG + wrow * 16);
    x0 = *reinterpret_cast<const f32x4 *>(xl + (2 * t + h) * kXG + xcol * 16);
}

template <bool kBuf, bool kF32>
__global__ __launch_bounds__(256, 2) void tinyblas_mfma(GemmTable g, int64_t k, const void *__restrict__ a,
                                                        int64_t n, int nct)
{
    __shared__ __attribute__((aligned(16))) char lds[2 * (kWBuf + kXBuf)];

    int mi, rt, ct;
    gemm_tile(g, xcd_tile(blockIdx.x, g.tile0[g.count]), nct, mi, rt, ct);
    const int64_t rows = g.rows[mi];
    float *__restrict__ out = g.out[mi];
    const int64_t row0 = (int64_t)rt * kBM;
    const int64_t col0 = (int64_t)ct * kBN;
    const Src<kBuf, kF32> src(g.w[mi], rows, a, n, k, row0, col0);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int i = lane & 31;          // row (A) / column (B) within the 32 x 32 tile
    const int h = lane >> 5;          // 0: chain lanes 0..3, 1: chain lanes 4..7
    const int wrow = (wave >> 1) * 32 + i;  // the thread's weight row within the block
    const int xcol = (wave & 1) * 32 + i;   // its activation column within the block

    f32x32 acc[4];
#pragma unroll
    for (int p = 0; p < 4; p++)
#pragma unroll
        for (int v = 0; v < 32; v++) acc[p][v] = 0.f;

    // Pipeline: during stage st the MFMAs read LDS buffer st % 2, the chunks
    // of stage st + 1 (in registers) are stashed into buffer (st + 1) % 2
    // between them, and each register, once stashed, is reloaded with its
    // chunk of stage st + 3: two register sets, one per stage parity, so a
    // chunk has two whole stages to arrive.  Chunks past k are zero, so the
    // last stages need no special case.
    const int64_t nstages = (k + kKS - 1) / kKS;
    u32x4 wr0[kWPT], xr0[kXPT][2], wr1[kWPT], xr1[kXPT][2];
    fetch_stage<kBuf, kF32>(wr0, xr0, src, 0, tid);
    stash_stage<kF32>(lds, lds + kWBuf, wr0, xr0, tid);
    fetch_stage<kBuf, kF32>(wr1, xr1, src, kKS, tid);       // stage 1: set 1
    fetch_stage<kBuf, kF32>(wr0, xr0, src, 2 * kKS, tid);   // stage 2: set 0
    __syncthreads();
    // Stage st, whose next stage waits in (wreg, xreg): the set of parity
    // (st + 1) % 2.
    auto stage = [&](int64_t st, u32x4(&wreg)[kWPT], u32x4(&xreg)[kXPT][2]) {
        const char *wl = lds + (st & 1) * (kWBuf + kXBuf);
        const char *xl = wl + kWBuf;
        char *nwl = lds + ((st + 1) & 1) * (kWBuf + kXBuf);
        char *nxl = nwl + kWBuf;
        const int64_t kfetch = (st + 3) * kKS;
        // operands two steps ahead of the MFMAs that use them
        f32x4 wa, x0, wa1, x01;
        read_step(wl, xl, 0, h, wrow, xcol, wa, x0);
        read_step(wl, xl, 1, h, wrow, xcol, wa1, x01);
        static_for<0, kSteps>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            f32x4 nwa, nx0;
            if constexpr (t + 2 < kSteps) read_step(wl, xl, t + 2, h, wrow, xcol, nwa, nx0);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, 4>([&](auto pc) {
                constexpr int p = decltype(pc)::value;
                acc[p] = __builtin_amdgcn_mfma_f32_32x32x1f32(wa[p], x0[p], acc[p], 0, 0, 0);
                if constexpr (Slot<t, p>::kUsed) {
                    constexpr int q = Slot<t, p>::kUsed ? Slot<t, p>::kQ : 0;
                    __builtin_amdgcn_sched_barrier(0);
                    stash_half<kF32, q>(nwl, nxl, wreg, xreg, tid);
                    if constexpr (q % 2 == 1) fetch_chunk<kBuf, kF32, q / 2>(wreg, xreg, src, kfetch, tid);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            if constexpr (t + 1 < kSteps) {
                wa = wa1;
                x0 = x01;
            }
            if constexpr (t + 2 < kSteps) {
                wa1 = nwa;
                x01 = nx0;
            }
        });
        // buffer (st + 1) % 2 is complete, and every wave is done reading
        // buffer st % 2, which stage st + 1 overwrites
        __syncthreads();
    };
    int64_t st = 0;
    for (; st + 1 < nstages; st += 2) {
        stage(st, wr1, xr1);
        stage(st + 1, wr0, xr0);
    }
    if (st < nstages) stage(st, wr1, xr1);

    // hsum in the page's order, then out[c*rows + r] for 4 consecutive rows.
    // Register v (< 16) of instruction p holds chain lane p and v + 16 lane
    // p + 4 of the element at row (v / 4) * 8 + h * 4 + v % 4, column i.
    const bool o16 = ((uintptr_t)out & 15) == 0;
    {
        const int64_t c = col0 + xcol;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int64_t r = row0 + (wrow - i) + 8 * q + 4 * h;
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int v = 4 * q + e;
                o[e] = ((acc[0][v] + acc[0][v + 16]) + (acc[2][v] + acc[2][v + 16])) +
                       ((acc[1][v] + acc[1][v + 16]) + (acc[3][v] + acc[3][v + 16]));
            }
            // rows % 4 == 0 and r % 4 == 0: r < rows covers r .. r + 3
            if (r < rows && c < n) {
                float *dst = out + c * rows + r;
                if (o16) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                } else {
                    dst[0] = o[0];
                    dst[1] = o[1];
                    dst[2] = o[2];
                    dst[3] = o[3];
                }
            }
        }
    }
}

// Small grids: one 32 x 32 tile per block, its four instructions split over
// the block's four waves (wave p carries chain lanes p and p + 4 of all
// 1024 elements, one MFMA per step), so a product with few tiles runs four
// times as many waves.  Each chain is the same sequence of FMA steps as in
// tinyblas_mfma; the eight lanes of an element meet in LDS at the end and
// are added in the page's order.  Operands go to LDS as f16 (activations
// rounded first), each row or column's 64 halves of a stage plus one pad
// word: a thread's 16-byte chunk is four word writes, and the 33-word row
// stride puts the 32 rows a wave reads per step in 32 different banks.  A
// stage's eight steps are read and widened before its first MFMA, so the
// dependent MFMAs issue back to back, and chunks are fetched two stages
// before they are stashed (two register sets, by stage parity).  Measured
// against f32 operands in LDS read one step ahead with one stage of fetch
// lead: 6-8 % faster with f16 activation blocks, 2-5 % with f32, same bits.
// The dependent chain itself bounds these launches: with no staging at all a
// timing copy is only 14-23 % faster, since each 32x32x1 step of one chain
// waits for the previous one.
constexpr int kLT = 32;                         // rows = columns per tile
constexpr int kLG = kLT + 1;                    // words per padded 32-float group (sizes the buffers)
constexpr int kLBuf = kSteps * 8 * kLG * 4;     // bytes per operand buffer; the end-of-tile gather needs 2 * 2 * kLBuf >= 32 KB
// the f16 stage (32 rows of kKS / 2 + 1 words) fits an operand buffer, and
// the end-of-tile gather (4 waves x 32 registers x 64 lanes of f32) fits the
// block's LDS
static_assert(kLT * (kKS / 2 + 1) * 4 <= kLBuf && 4 * 32 * 64 * 4 <= 2 * 2 * kLBuf, "LDS layout");
// Launches of at most this many 32 x 32 tiles take tinyblas_lanes (measured
// on the 135M-shaped products at n = 512: q/k/v, o and down, 288-480 tiles,
// 22-29 % faster; gate/up, 1536 tiles, no faster; 2048 tiles 20 % slower).
constexpr int64_t kLanesMaxTiles = 1024;

template <bool kF32>
__global__ __launch_bounds__(256) void tinyblas_lanes(GemmTable g, int64_t k, const void *__restrict__ a,
                                                      int64_t n, int nct)
{
    __shared__ __attribute__((aligned(16))) char lds[2 * 2 * kLBuf];

    int mi, rt, ct;
    gemm_tile(g, xcd_tile(blockIdx.x, g.tile0[g.count]), nct, mi, rt, ct);
    const int64_t rows = g.rows[mi];
    float *__restrict__ out = g.out[mi];
    const int64_t row0 = (int64_t)rt * kLT;
    const int64_t col0 = (int64_t)ct * kLT;
    const uint16_t *w = g.w[mi];
    const int64_t wr = rows - row0 < kLT ? rows - row0 : kLT;
    const int64_t xr = n - col0 < kLT ? n - col0 : kLT;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(w + row0 * k, wr * k * 2);
    constexpr int ESZ = kF32 ? 4 : 2;             // activation element bytes
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(static_cast<const char *>(a) + col0 * k * ESZ, xr * k * ESZ);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int p = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's instruction
    const int i = lane & 31, h = lane >> 5;
    const int q = p + 4 * h;                                  // this lane's chain lane
    // the thread's chunk of a stage: row (column) lr, step lt
    const int lr = tid >> 3, lt = tid & 7;
    const uint32_t coff = (uint32_t)((lr * k + 8 * lt) * 2);       // weights
    const uint32_t cxoff = (uint32_t)((lr * k + 8 * lt) * ESZ);    // activations

    f32x32 acc;
#pragma unroll
    for (int v = 0; v < 32; v++) acc[v] = 0.f;

    // chunk (lr, lt) of the stage at k0 (activations raw: one or two 16-byte
    // halves); past k: offset past the resource
    auto fetch = [&](int64_t k0, u32x4 &cw, u32x4 (&cx)[2]) {
        const bool in = k0 + 8 * lt < k;
        const int off = in ? (int)(coff + (uint32_t)(k0 * 2)) : 0x7ffffff0;
        const int xoff = in ? (int)(cxoff + (uint32_t)(k0 * ESZ)) : 0x7ffffff0;
        cw = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
        cx[0] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, 0, 0);
        if constexpr (kF32) cx[1] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xoff + 16 : xoff, 0, 0);
    };
    // f16 operands as stored (activations rounded first): row (column) lr,
    // halves 8 lt .. 8 lt + 7 of the stage at word offset lr * kHW + 4 lt
    constexpr int kHW = kKS / 2 + 1;              // words per row: 64 halves + one pad word
    auto stash = [&](char *buf, const u32x4 &cw, const u32x4 (&cx)[2]) {
        uint32_t *ww = reinterpret_cast<uint32_t *>(buf), *wx = reinterpret_cast<uint32_t *>(buf + kLBuf);
        u32x4 xh;
        if constexpr (kF32) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const u32x4 hp = e < 2 ? cx[0] : cx[1];
                const int b = 2 * (e & 1);
                xh[e] = (uint32_t)rne_f16(__uint_as_float(hp[b])) | ((uint32_t)rne_f16(__uint_as_float(hp[b + 1])) << 16);
            }
        } else {
            xh = cx[0];
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            ww[lr * kHW + 4 * lt + e] = cw[e];
            wx[lr * kHW + 4 * lt + e] = xh[e];
        }
    };

    const int64_t nstages = (k + kKS - 1) / kKS;
    // Two register sets: set A carries the odd stages, set B the even ones
    // (stage 0 goes straight to LDS), each fetched two stages before it is
    // stashed.
    u32x4 cwA, cxA[2], cwB, cxB[2];
    fetch(0, cwA, cxA);
    stash(lds, cwA, cxA);
    fetch(kKS, cwA, cxA);
    fetch(2 * kKS, cwB, cxB);
    __syncthreads();
    auto body = [&](int64_t st, u32x4 &cw, u32x4 (&cx)[2]) {
        const uint16_t *hw = reinterpret_cast<const uint16_t *>(lds + (st & 1) * 2 * kLBuf);
        const uint16_t *hx = hw + kLBuf / 2;
        char *nbuf = lds + ((st + 1) & 1) * 2 * kLBuf;
        float wv[kSteps], xv[kSteps];
#pragma unroll
        for (int t = 0; t < kSteps; t++) {
            wv[t] = widen_h(hw[i * 2 * kHW + 8 * t + q]);
            xv[t] = widen_h(hx[i * 2 * kHW + 8 * t + q]);
        }
#pragma unroll
        for (int t = 0; t < kSteps; t++) {
            acc = __builtin_amdgcn_mfma_f32_32x32x1f32(wv[t], xv[t], acc, 0, 0, 0);
            if (t == 3) {
                // stage st + 1 into the other buffer, then refill the set with st + 3
                stash(nbuf, cw, cx);
                fetch((st + 3) * kKS, cw, cx);
            }
        }
        __syncthreads();
    };
    for (int64_t st = 0; st < nstages; st += 2) {
        body(st, cwA, cxA);
        if (st + 1 < nstages) body(st + 1, cwB, cxB);
    }

    // Gather: wave p's registers v and v + 16 are chain lanes p and p + 4.
    // Thread (wave p', lane) then sums registers v = 4p' .. 4p' + 3 of its
    // lane, i.e. rows 8p' + 4h .. + 3 of column i, from all four waves.
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int v = 0; v < 32; v++) red[(p * 32 + v) * 64 + lane] = acc[v];
    __syncthreads();
    const int64_t c = col0 + i;
    const int64_t r = row0 + 8 * p + 4 * h;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const int v = 4 * p + e;
        float l[8];
#pragma unroll
        for (int w4 = 0; w4 < 4; w4++) {
            l[w4] = red[(w4 * 32 + v) * 64 + lane];
            l[w4 + 4] = red[(w4 * 32 + v + 16) * 64 + lane];
        }
        o[e] = ((l[0] + l[4]) + (l[2] + l[6])) + ((l[1] + l[5]) + (l[3] + l[7]));
    }
    // rows % 4 == 0 and r % 4 == 0: r < rows covers r .. r + 3
    if (r < rows && c < n) {
        float *dst = out + c * rows + r;
        if ((((uintptr_t)dst) & 15) == 0) {
            *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
            dst[0] = o[0];
            dst[1] = o[1];
            dst[2] = o[2];
            dst[3] = o[3];
        }
    }
}

}  // namespace

hipError_t launch_sgemm(GemmTable g, int64_t k, const void *a, int64_t n, bool aligned16, bool f32act,
                        hipStream_t stream)
{
    const int64_t esz = f32act ? 4 : 2;   // activation element bytes
    // few tiles: one block per 32 x 32 tile, its four instructions on four
    // waves (aligned operands, 32-row tile resources under 2^31 bytes)
    if (aligned16 && (int64_t)kLT * k * esz < ((int64_t)1 << 31)) {
        const int64_t nct32 = (n + kLT - 1) / kLT;
        int64_t t32 = 0;
        for (int m = 0; m < g.count; m++) t32 += (g.rows[m] + kLT - 1) / kLT * nct32;
        if (t32 <= kLanesMaxTiles) {
            int64_t acc = 0;
            for (int m = 0; m < g.count; m++) {
                g.tile0[m] = (int32_t)acc;
                acc += (g.rows[m] + kLT - 1) / kLT * nct32;
            }
            g.tile0[g.count] = (int32_t)acc;
            const dim3 grid((uint32_t)acc);
            if (f32act)
                tinyblas_lanes<true><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct32);
            else
                tinyblas_lanes<false><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct32);
            return hipGetLastError();
        }
    }
    const int64_t nct = (n + kBN - 1) / kBN;
    int64_t tiles = 0;
    for (int m = 0; m < g.count; m++) {
        g.tile0[m] = (int32_t)tiles;
        tiles += (g.rows[m] + kBM - 1) / kBM * nct;
        if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    }
    g.tile0[g.count] = (int32_t)tiles;
    const dim3 grid((uint32_t)tiles);
    // buffer offsets are 32-bit with bit 31 marking chunks past k: a tile of
    // kBN columns must stay under 2^31 bytes
    const bool buf = aligned16 && (int64_t)kBN * k * esz < ((int64_t)1 << 31);
    if (f32act) {
        if (buf)
            tinyblas_mfma<true, true><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
        else
            tinyblas_mfma<false, true><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    } else {
        if (buf)
            tinyblas_mfma<true, false><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
        else
            tinyblas_mfma<false, false><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    }
    return hipGetLastError();
}

}  // namespace f16wm
