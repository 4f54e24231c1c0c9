// The f16 attention helpers over an f16 KV cache: vec_dot_u16 scores against
// the K cache, and the V-accumulator updates mad and scale.
//
// bankML f16 page, Summary and Technical usage: the attention code uses
// vec_dot_u16 (the vec_dot order with the first operand given as f16 values)
// for K-cache rows, and mad (ggml_vec_mad_f16) and scale (ggml_vec_scale_f16)
// for the f16 V accumulator.
//
// kq: out[h][p] = vec_dot(K[p][h / G], q[h]) with the cache laid out
// position-major, K[p][j][0..d), and G = n_head / n_kv_head query heads per
// KV head.  For d of 64 or 128 with 16-byte aligned arrays (kq_dma) tiles of
// consecutive positions -- all KV heads, one contiguous stretch of the cache --
// stream into LDS by direct loads, and one lane per (position, query head)
// holds all 32 chains with its query in registers; otherwise (kq_generic) 32
// lanes per pair each own one chain and read global memory.  The reduction is
// the vec_dot tree (vec_dot_order.h); a d % 32 tail is added in binary64.
// The cache is read once: 2 * n_kv * n_kv_head * d bytes.
//
// mad / scale: element-wise over nvec vectors of n f16 values with one f32
// weight (factor) per vector: acc = f16(fma(f32(v), w, f32(acc))) and
// acc = f16(f32(acc) * s), the f16 rounding being the activation rounding
// (f16_round.h) applied to the finished f32 result (rne_f16_of_result keeps
// the compiler from fusing the two roundings into one mixed-precision
// instruction).  HBM-bound: 6 (mad) or 4 (scale) bytes per element.
#include <atomic>
#include <mutex>
#include <set>
#include <utility>

#include "buffer_rsrc.h"
#include "f16_round.h"
#include "kernels.h"
#include "vec_dot_order.h"

namespace f16wm {
namespace {

// Any d, any alignment: 32 lanes per (position, query head) pair, lane c
// owning chain c; one position per pair.
__global__ __launch_bounds__(256) void kq_generic(const uint16_t *__restrict__ kc, int64_t n_kv, int64_t n_kv_head,
                                                  int64_t d, const uint16_t *__restrict__ q, int64_t G, int P, int GB,
                                                  float *__restrict__ out)
{
    const int tid = threadIdx.x;
    const int pair = tid / 32;
    const int c = tid % 32;
    const int gl = pair / P;
    const int pp = pair % P;
    const int64_t j = blockIdx.y;
    const int64_t g = (int64_t)blockIdx.z * GB + gl;
    const int64_t p = (int64_t)blockIdx.x * P + pp;
    const bool valid = gl < GB && g < G && p < n_kv;
    const int64_t h = j * G + (valid ? g : 0);
    const uint16_t *krow = kc + ((valid ? p : 0) * n_kv_head + j) * d;
    const uint16_t *qrow = q + h * d;
    const int64_t nsteps = d >> 5;
    float acc[1] = {0.f};
    if (valid)
        for (int64_t t = 0; t < nsteps; t++) acc[0] = __builtin_fmaf(widen(krow[32 * t + c]), widen(qrow[32 * t + c]), acc[0]);
    float v = vec_dot_tree<1>(acc);
    if (valid && c == 0) {
        if (d & 31) {
            double s = (double)v;
            for (int64_t i = nsteps * 32; i < d; i++) s = s + (double)(widen(krow[i]) * widen(qrow[i]));
            v = (float)s;
        }
        out[h * n_kv + p] = v;
    }
}

// d in {64, 128}, 16-byte aligned cache and queries, n_head <= kKqThreads:
// one lane per (position, query head) holds all 32 chains of that score, so
// the whole vec_dot tree is in-lane adds; its query sits in registers as f32
// (a lane's query head never changes).  Blocks are persistent: block b takes
// tiles b, b + grid, ...; a tile is PB consecutive positions with all their
// KV heads (one contiguous stretch of the cache; the 32 KB loaded per tile
// may run into the next tile's first row, which goes unused).  Tiles go
// global -> LDS with buffer_load_dwordx4 ... lds (no registers, no ds_write;
// lane l of a load lands at M0 + 16 l), kKqBuf - 1 tiles ahead, marked
// nontemporal so the streamed cache does not push the partly written score
// lines out of L2 (their halves merge there before going to HBM).
// The S lanes of an aligned group (S = 4, 2 or 1, dividing G) hold S query
// heads of one KV head at one position, so they need the same K row: each
// reads and widens 1/S of it (chunk 4t + S u + k for lane k of the group),
// and every FMA takes its K value from the owning lane by a DPP permute
// inside the quad, folded into v_fmac_f32 (the mixed-precision FMA that
// widens on the fly issues at about 0.6 of v_fmac_f32's rate here).
// Rows (one position, one KV head: CH = d / 8 chunks of 16 bytes) keep chunk
// m in slot m ^ f(row), f spreading the rows one read instruction touches
// over the banks.  Rows past the cache read zero (buffer range check).
constexpr int kKqThreads = 512;               // threads per kq_dma block
constexpr int kKqBuf = 3;                     // LDS tile buffers
constexpr int kKqTile = 32768;                // bytes per tile
constexpr int kKqNW = kKqTile / 1024 / (kKqThreads / 64);   // loads per wave per tile
constexpr int kKqPastEnd = 0x7fff0000;        // a tile offset past every cache kq_dma takes

// LDS slot of chunk m of tile row r (an involution in m for each r).
template <int D>
__device__ __forceinline__ int kq_slot(int m, int r)
{
    if constexpr (D == 128)
        return m ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else
        return m ^ (((r >> 1) & 3) << 1);
}

// acc = fma(k of lane O of this lane's aligned group of S lanes, q, acc):
// one v_fmac_f32 whose first operand goes through a DPP quad permute.  The
// caller keeps the DPP read hazards clear: no VALU write of k in the two
// instructions before, no VALU write of EXEC in the five before.  Volatile,
// so these and widen8_ordered keep their program order.
#define F16WM_FMAC_DPP(PERM)                                                                        \
    asm volatile("v_fmac_f32_dpp %0, %1, %2 quad_perm:" PERM " row_mask:0xf bank_mask:0xf" : "+v"(acc) \
                 : "v"(k), "v"(q))
template <int S, int O>
__device__ __forceinline__ void fmac_group_lane(float &acc, float k, float q)
{
    if constexpr (S == 4) {
        if constexpr (O == 0) F16WM_FMAC_DPP("[0,0,0,0]");
        else if constexpr (O == 1) F16WM_FMAC_DPP("[1,1,1,1]");
        else if constexpr (O == 2) F16WM_FMAC_DPP("[2,2,2,2]");
        else F16WM_FMAC_DPP("[3,3,3,3]");
    } else {
        if constexpr (O == 0) F16WM_FMAC_DPP("[0,0,2,2]");
        else F16WM_FMAC_DPP("[1,1,3,3]");
    }
}
#undef F16WM_FMAC_DPP

// The eight f16 values of v widened to f32 (exact), element r in f[r], by
// conversions issued in that order.
__device__ __forceinline__ void widen8_ordered(float (&f)[8], u32x4 v)
{
#pragma unroll
    for (int w = 0; w < 4; w++) {
        asm volatile("v_cvt_f32_f16_e32 %0, %1" : "=v"(f[2 * w]) : "v"(v[w]));
        asm volatile("v_cvt_f32_f16_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1"
                     : "=v"(f[2 * w + 1])
                     : "v"(v[w]));
    }
}

template <int D, int S>
__global__ __launch_bounds__(kKqThreads) void kq_dma(const uint16_t *__restrict__ kc, int64_t n_kv, int64_t n_kv_head,
                                                     const uint16_t *__restrict__ q, int64_t n_head,
                                                     float *__restrict__ out)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    constexpr int CH = D / 8;                      // 16-byte chunks per row
    constexpr int NS = D / 32;                     // vec_dot steps
    constexpr int CPS = 4 / S;                     // chunks per step this lane reads
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rowbytes = (int)n_kv_head * D * 2;   // one position, all KV heads
    const int PB = kKqTile / rowbytes;             // positions per tile
    const int64_t ntiles = (n_kv + PB - 1) / PB;
    const int nh = (int)n_head;
    const int G = (int)(n_head / n_kv_head);
    const int slots = kKqThreads / nh;             // positions per pass
    const int h = tid % nh, slot = tid / nh;
    const bool active = slot < slots;
    const int j = h / G;                           // this lane's KV head
    const int gk = lane & (S - 1);                 // this lane's place in its group

    // Loads of one tile: load i of wave w fills LDS chunks (w NW + i) 64 + lane.
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kc, n_kv * rowbytes);
    int goff[kKqNW];
#pragma unroll
    for (int i = 0; i < kKqNW; i++) {
        const int c = (wave * kKqNW + i) * 64 + lane;
        const int row = c / CH;
        goff[i] = (row * CH + kq_slot<D>(c % CH, row)) * 16;
    }
    // Block b's k-th tile is b + k * grid, held in buffer k % kKqBuf.  Past
    // the block's last tile the same loads read zero (offset past the
    // cache), so every wave issues kKqNW loads per tile and the waits count
    // them (score stores share the counter: they only lengthen a wait).
    const int64_t G0 = blockIdx.x, GS = gridDim.x;
    const int64_t mine = G0 < ntiles ? (ntiles - 1 - G0) / GS + 1 : 0;
    auto issue = [&](int64_t k) {
        unsigned char *buf = lds + (int)(k % kKqBuf) * kKqTile;
        const int base = k < mine ? (int)((G0 + k * GS) * PB * rowbytes) : kKqPastEnd;
#pragma unroll
        for (int i = 0; i < kKqNW; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                kr, (__attribute__((address_space(3))) void *)(buf + (wave * kKqNW + i) * 1024), 16,
                base + goff[i], 0, 0, 2);
    };

    // this lane's query, widened
    float qf[D];
#pragma unroll
    for (int c = 0; c < CH; c++) {
        const half8 v = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4 *>(q + (int64_t)h * D + 8 * c));
#pragma unroll
        for (int r = 0; r < 8; r++) qf[8 * c + r] = (float)v[r];
    }

#pragma unroll
    for (int k = 0; k < kKqBuf - 1; k++) issue(k);
    for (int64_t k = 0; k < mine; k++) {
        // this wave's loads of tile k are in LDS, every wave's after the
        // barrier, and every wave is done with buffer (k - 1) % kKqBuf
        constexpr int YOUNG = (kKqBuf - 2) * kKqNW;
        __builtin_amdgcn_s_waitcnt((YOUNG & 15) | 0x0F70 | ((YOUNG >> 4) << 14));
        asm volatile("s_barrier" ::: "memory");
        issue(k + kKqBuf - 1);

        const unsigned char *tl = lds + (int)(k % kKqBuf) * kKqTile;
        const int64_t p0 = (G0 + k * GS) * PB;
        for (int pp = slot; pp < PB; pp += slots) {
            const int64_t p = p0 + pp;
            if (!active || p >= n_kv) continue;    // a whole group of S lanes at once
            const int row = pp * (int)n_kv_head + j;
            const unsigned char *kl = tl + row * CH * 16;
            float acc[32];
#pragma unroll
            for (int c = 0; c < 32; c++) acc[c] = 0.f;
            if constexpr (S > 1) asm volatile("s_nop 4");   // an EXEC write before the first DPP read
#pragma unroll
            for (int t = 0; t < NS; t++) {
                // this lane's chunks of step t, widened: chunk 4t + S u + gk
                float kf[CPS][8];
#pragma unroll
                for (int u = 0; u < CPS; u++) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(kl + 16 * kq_slot<D>(4 * t + S * u + gk, row));
                    if constexpr (S == 1) {
                        const half8 hv = __builtin_bit_cast(half8, v);
#pragma unroll
                        for (int r = 0; r < 8; r++) kf[u][r] = (float)hv[r];
                    } else {
                        widen8_ordered(kf[u], v);
                    }
                }
                // quarter i of step t is chunk 4t + i: lane i % S of the
                // group holds it as its chunk u = i / S; chain 8 i + r.  In
                // this order FMA number 8 u' + r reads kf[u][r], widened at
                // least seven instructions earlier.
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int r = 0; r < 8; r++) {
                        float &a = acc[8 * i + r];
                        const float kv = kf[i / S][r], qv = qf[32 * t + 8 * i + r];
                        if constexpr (S == 1)
                            a = __builtin_fmaf(kv, qv, a);
                        else if (i % S == 0)
                            fmac_group_lane<S, 0>(a, kv, qv);
                        else if (i % S == 1)
                            fmac_group_lane<S, 1>(a, kv, qv);
                        else if (i % S == 2)
                            fmac_group_lane<S, 2>(a, kv, qv);
                        else
                            fmac_group_lane<S, 3>(a, kv, qv);
                    }
            }
            out[(int64_t)h * n_kv + p] = vec_dot_tree<32>(acc);   // all in-lane
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);            // the zero loads past the end have landed
}

// Eight elements per thread (n % 8 == 0, 16-byte aligned arrays) or one.
// The 16-byte accesses are nontemporal: with every array cold (rotating
// copies) mad is 7 % and scale 16 % faster, and with one accumulator updated
// launch after launch (hot in the cache) neither changes.
template <bool kVec8>
__global__ __launch_bounds__(256) void mad_kernel(uint16_t *__restrict__ acc, const uint16_t *__restrict__ v,
                                                  const float *__restrict__ w, int64_t nvec, int64_t n)
{
    const int64_t total = nvec * n;
    const int64_t per = kVec8 ? 8 : 1;
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * per; e < total;
         e += (int64_t)gridDim.x * 256 * per) {
        const float wb = w[e / n];
        if (kVec8) {
            const half8 a = __builtin_bit_cast(half8, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(acc + e)));
            const half8 x = __builtin_bit_cast(half8, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(v + e)));
            uint16_t r[8];
#pragma unroll
            for (int i = 0; i < 8; i++) r[i] = rne_f16_of_result(__builtin_fmaf((float)x[i], wb, (float)a[i]));
            u32x4 o;
            o[0] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
            o[1] = (uint32_t)r[2] | ((uint32_t)r[3] << 16);
            o[2] = (uint32_t)r[4] | ((uint32_t)r[5] << 16);
            o[3] = (uint32_t)r[6] | ((uint32_t)r[7] << 16);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(acc + e));
        } else {
            acc[e] = rne_f16_of_result(__builtin_fmaf(widen(v[e]), wb, widen(acc[e])));
        }
    }
}

template <bool kVec8>
__global__ __launch_bounds__(256) void scale_kernel(uint16_t *__restrict__ acc, const float *__restrict__ s,
                                                    int64_t nvec, int64_t n)
{
    const int64_t total = nvec * n;
    const int64_t per = kVec8 ? 8 : 1;
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * per; e < total;
         e += (int64_t)gridDim.x * 256 * per) {
        const float sb = s[e / n];
        if (kVec8) {
            const half8 a = __builtin_bit_cast(half8, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(acc + e)));
            uint16_t r[8];
#pragma unroll
            for (int i = 0; i < 8; i++) r[i] = rne_f16_of_result((float)a[i] * sb);
            u32x4 o;
            o[0] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
            o[1] = (uint32_t)r[2] | ((uint32_t)r[3] << 16);
            o[2] = (uint32_t)r[4] | ((uint32_t)r[5] << 16);
            o[3] = (uint32_t)r[6] | ((uint32_t)r[7] << 16);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(acc + e));
        } else {
            acc[e] = rne_f16_of_result(widen(acc[e]) * sb);
        }
    }
}

// Enough blocks to fill the GPU several times over; the kernels stride.
uint32_t elementwise_grid(int64_t items)
{
    const int64_t blocks = (items + 255) / 256;
    return (uint32_t)(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192);
}

}  // namespace

int64_t device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

void allow_dynamic_lds(const void *fn, int bytes)
{
    static std::mutex mu;
    static std::set<std::pair<int, const void *>> done;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lock(mu);
    if (done.insert({dev, fn}).second)
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_kq(const uint16_t *kc, int64_t n_kv, int64_t n_kv_head, int64_t d, const uint16_t *q,
                     int64_t n_head, bool vec8, float *out, hipStream_t stream)
{
    // LDS kernel: d of 64 or 128, a position row of at most one 32 KB tile,
    // a cache of at most kKqPastEnd bytes, at most 512 query heads.
    const int64_t rowbytes = n_kv_head * d * 2;
    if (vec8 && (d == 64 || d == 128) && n_head <= kKqThreads && rowbytes <= kKqTile &&
        n_kv * rowbytes <= kKqPastEnd) {
        typedef void (*KqFn)(const uint16_t *, int64_t, int64_t, const uint16_t *, int64_t, float *);
        static const KqFn fns[2][3] = {{kq_dma<64, 1>, kq_dma<64, 2>, kq_dma<64, 4>},
                                       {kq_dma<128, 1>, kq_dma<128, 2>, kq_dma<128, 4>}};
        const int64_t G = n_head / n_kv_head;
        const int si = G % 4 == 0 ? 2 : G % 2 == 0 ? 1 : 0;   // S = 4, 2, 1 query heads share a K row read
        allow_dynamic_lds(reinterpret_cast<const void *>(fns[d == 128][si]), kKqBuf * kKqTile);
        const int64_t PB = kKqTile / rowbytes;
        const int64_t ntiles = (n_kv + PB - 1) / PB;
        // one resident block per CU (the LDS buffers and registers allow one):
        // every block streams ntiles / CUs tiles through its pipeline
        const int64_t cus = device_cus();
        const int64_t gx = ntiles < cus ? ntiles : cus;
        hipLaunchKernelGGL(fns[d == 128][si], dim3((uint32_t)gx), dim3(kKqThreads), kKqBuf * kKqTile, stream, kc, n_kv,
                           n_kv_head, q, n_head, out);
        return hipGetLastError();
    }
    const int pairs = 8;                           // 32 lanes per pair
    const int64_t G = n_head / n_kv_head;
    const int GB = (int)(G < pairs ? G : pairs);   // query heads per block
    const int P = pairs / GB;                      // positions per block
    const int64_t gx = (n_kv + P - 1) / P, gz = (G + GB - 1) / GB;
    if (gx > 0x7fffffff || n_kv_head > 65535 || gz > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)gx, (uint32_t)n_kv_head, (uint32_t)gz);
    kq_generic<<<grid, dim3(256), 0, stream>>>(kc, n_kv, n_kv_head, d, q, G, P, GB, out);
    return hipGetLastError();
}

hipError_t launch_mad(uint16_t *acc, const uint16_t *v, const float *w, int64_t nvec, int64_t n, bool vec8,
                      hipStream_t stream)
{
    const int64_t items = vec8 ? nvec * n / 8 : nvec * n;
    const dim3 grid(elementwise_grid(items));
    if (vec8)
        mad_kernel<true><<<grid, dim3(256), 0, stream>>>(acc, v, w, nvec, n);
    else
        mad_kernel<false><<<grid, dim3(256), 0, stream>>>(acc, v, w, nvec, n);
    return hipGetLastError();
}

hipError_t launch_scale(uint16_t *acc, const float *s, int64_t nvec, int64_t n, bool vec8, hipStream_t stream)
{
    const int64_t items = vec8 ? nvec * n / 8 : nvec * n;
    const dim3 grid(elementwise_grid(items));
    if (vec8)
        scale_kernel<true><<<grid, dim3(256), 0, stream>>>(acc, s, nvec, n);
    else
        scale_kernel<false><<<grid, dim3(256), 0, stream>>>(acc, s, nvec, n);
    return hipGetLastError();
}

}  // namespace f16wm
