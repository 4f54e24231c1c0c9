// The vec_dot reduction as GPU lane code, shared by the kernels that run the
// vec_dot order (the GEMV family and the K-cache scores).  Not part of the ABI.
//
// bankML f16 page, Design notes ("vec_dot"): every element is 32 sequential
// f32 FMA chains (chain c takes elements 32t + c, ascending t), reduced
// (a0+a2)+(a1+a3), low half + high half, then two horizontal adds of adjacent
// pairs.  Here one chain always lives in one lane; the reduction is a fixed
// sequence of adds, across lanes by shuffles or inside a lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace f16wm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Exact f16 -> f32 (subnormals kept).
static __device__ __forceinline__ float widen(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// The 32 chains of one element, spread over LPR lanes (CPL = 32 / LPR chains
// per lane: global chain c = CPL*j + i for lane j, register i), reduced in the
// vec_dot tree: c with c^16 and c^8 ((a0+a2)+(a1+a3)), c^4 (low + high half),
// c^1 then c^2 (the two horizontal adds).  A pairing across lanes is a shuffle
// by (bit / CPL); a pairing inside a lane adds two registers.  The result is
// in register 0 of every lane of the row.
// x of the lane whose index is this lane's xor M, for M = 1, 2: within a
// quad, by a DPP quad_perm move (no LDS traffic); other distances use
// __shfl_xor.
template <int M>
__device__ __forceinline__ float lane_xor(float x)
{
    if constexpr (M == 1 || M == 2) {
        constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false));
    } else {
        return __shfl_xor(x, M);
    }
}

template <int CPL>
__device__ __forceinline__ float vec_dot_tree(float (&v)[CPL])
{
    constexpr int kBits[5] = {16, 8, 4, 1, 2};
#pragma unroll
    for (int L = 0; L < 5; L++) {
        const int b = kBits[L];
        if (b >= CPL) {
            const int m = b / CPL;                 // lane distance, constant once unrolled
#pragma unroll
            for (int i = 0; i < CPL; i++) {
                const float o = m == 1 ? lane_xor<1>(v[i]) : m == 2 ? lane_xor<2>(v[i]) : __shfl_xor(v[i], m);
                v[i] = v[i] + o;
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPL; i++)
                if ((i & b) == 0) v[i] = v[i] + v[i | b];
        }
    }
    return v[0];
}

template <int N>
struct Halves;
template <>
struct Halves<8> { typedef u32x4 T; };
template <>
struct Halves<4> { typedef uint2 T; };
template <>
struct Halves<2> { typedef uint32_t T; };
template <>
struct Halves<1> { typedef uint16_t T; };

// acc[i] = fma(w_i, a_i, acc[i]) for the CPL f16 pairs packed in w and a.
template <int CPL>
__device__ __forceinline__ void fma_halves(float (&acc)[CPL], typename Halves<CPL>::T w,
                                           typename Halves<CPL>::T a)
{
    typedef _Float16 hv __attribute__((ext_vector_type(CPL == 1 ? 2 : CPL)));
    if constexpr (CPL == 1) {
        acc[0] = __builtin_fmaf(widen(w), widen(a), acc[0]);
    } else {
        const hv wh = __builtin_bit_cast(hv, w);
        const hv ah = __builtin_bit_cast(hv, a);
#pragma unroll
        for (int i = 0; i < CPL; i++) acc[i] = __builtin_fmaf((float)wh[i], (float)ah[i], acc[i]);
    }
}

}  // namespace f16wm
