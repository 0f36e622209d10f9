// Cross-lane reductions for 64-wide wavefronts on gfx950.
//
// Inside a row of 16 lanes the max goes through DPP (quad permutes, then the
// half-row and row mirrors, which pair every lane with one from the other
// half); across rows it goes through ds_bpermute shuffles.  All lanes of the
// wave must be active when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// DPP control codes (GCN/CDNA encoding)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within each 8
constexpr int kDppRowMirror = 0x140;    // lane i <-> 15 - i within each 16
constexpr int kDppWaveShl1 = 0x130;     // lane i reads lane i + 1 (whole wave)

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// the value of lane + 1 of the wave (VALU data movement, no LDS); lane 63
// receives 0
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v) { return dpp<kDppWaveShl1>(v); }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// packed max of two pairs of u16
__device__ __forceinline__ uint32_t pkmax(uint32_t a, uint32_t b)
{
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}

// max over aligned groups of N lanes (N in 1, 2, 4, 8, 16); every lane of the
// group receives the result
template <int N>
__device__ __forceinline__ uint32_t group_max(uint32_t v)
{
    if constexpr (N >= 2) v = umax(v, dpp<kDppQuadXor1>(v));
    if constexpr (N >= 4) v = umax(v, dpp<kDppQuadXor2>(v));
    if constexpr (N >= 8) v = umax(v, dpp<kDppHalfMirror>(v));
    if constexpr (N >= 16) v = umax(v, dpp<kDppRowMirror>(v));
    return v;
}

// max over the whole wave, returned wave-uniform
__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    v = group_max<16>(v);
    uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return umax(umax(a, b), umax(c, d));
}

// max over lanes that differ only in lane bits >= log2(FIRST) (FIRST a power
// of two), i.e. across all lanes sharing lane % FIRST; every lane receives it
template <int FIRST>
__device__ __forceinline__ uint32_t strided_pkmax(uint32_t v)
{
#pragma unroll
    for (int m = FIRST; m < 64; m <<= 1)
        v = pkmax(v, (uint32_t)__shfl_xor((int)v, m, 64));
    return v;
}

}  // namespace mxq
