// Device-side building blocks shared by the gfx950 quantization kernels.
//
// Every element goes through the same four steps:
//   1. bf16 -> fp32 by a shift (exact; a subnormal stays subnormal),
//   2. amax on the bf16 bit patterns: for finite values |a| <= |b| iff
//      (a & 0x7FFF) <= (b & 0x7FFF) as unsigned, so two elements per
//      v_pk_max_u16,
//   3. one fp32 multiply by the scale (kernels are built with IEEE fp32
//      denormals, so a subnormal input times 2^127 is exact),
//   4. v_med3_f32 clamp to +-448, then v_cvt_pk_fp8_f32 (OCP E4M3FN, round to
//      nearest even) packing two results per instruction.
// The scale is either the fp32 multiplier 448 / max(amax, 1e-12) computed by
// the compiler's correctly rounded division, or an e8m0 code whose multiplier
// 2^(127 - code) is built directly from its exponent bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxEps = 1e-12f;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// packed running max of |bf16| over the two halves of a dword
__device__ __forceinline__ uint32_t absmax2(uint32_t m, uint32_t v)
{
    u16x2 a = __builtin_bit_cast(u16x2, m);
    u16x2 b = __builtin_bit_cast(u16x2, v & 0x7fff7fffu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// max of the two 16-bit halves
__device__ __forceinline__ uint32_t fold2(uint32_t m)
{
    uint32_t lo = m & 0xffffu, hi = m >> 16;
    return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t absmax_u4(const uint4 &v)
{
    uint32_t m = absmax2(absmax2(v.x & 0x7fff7fffu, v.y), absmax2(v.z & 0x7fff7fffu, v.w));
    return m;
}

// fp32 quantize multiplier from the |bf16| bit pattern of amax
__device__ __forceinline__ float fp32_scale(uint32_t amax16)
{
    float a = __uint_as_float(amax16 << 16);
    return kE4M3Max / fmaxf(a, kAmaxEps);
}

// e8m0 "floor" code from the |bf16| bit pattern of amax:
// floor(log2 amax) = exponent field - 127 for normal amax, and anything
// below 2^-118 clamps to code 0, so code = max(field - 8, 0).
__device__ __forceinline__ uint32_t e8m0_floor_code(uint32_t amax16)
{
    int f = (int)((amax16 >> 7) & 0xffu);
    return f > 8 ? (uint32_t)(f - 8) : 0u;
}

// e8m0 "rceil" code: the smallest se with amax <= 448 * 2^se (the scale
// amax / 448 rounded up to a power of two, so nothing saturates).  With
// amax = (1 + m/128) * 2^(field - 127), 448 = 1.75 * 2^8 and 1.75 = 1 + 96/128:
// se = field - 135 when m <= 96, else field - 134; clamped at code 0.
__device__ __forceinline__ uint32_t e8m0_rceil_code(uint32_t amax16)
{
    int f = (int)((amax16 >> 7) & 0xffu) - 8 + ((amax16 & 0x7fu) > 96u ? 1 : 0);
    return f > 0 ? (uint32_t)f : 0u;
}

__device__ __forceinline__ uint32_t e8m0_code(uint32_t amax16, bool rceil)
{
    return rceil ? e8m0_rceil_code(amax16) : e8m0_floor_code(amax16);
}

// element multiplier 2^(127 - code) for code in [0, 246] (always normal)
__device__ __forceinline__ float e8m0_multiplier(uint32_t code)
{
    return __uint_as_float((254u - code) << 23);
}

__device__ __forceinline__ float sat(float y) { return __builtin_amdgcn_fmed3f(y, -kE4M3Max, kE4M3Max); }

// four fp32 values -> four e4m3 bytes, a in the lowest byte
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d)
{
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), r, true);
    return (uint32_t)r;
}

// one element -> one byte
__device__ __forceinline__ uint32_t cvt1(float a)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(a), 0.0f, 0, false) & 0xffu;
}

// Unclamped form for the fp32-multiplier paths.  With s = RN32(448 / m),
// m = max(amax, eps) >= |x|, every product obeys
// |RN32(x * s)| <= RN32(448 * (1 + 2^-24)) <= 448 + 2^-15 < 464, and
// v_cvt_pk_fp8_f32 rounds to nearest even exactly below the 448/480 midpoint
// 464 (checked on gfx950 over every fp32 pattern in [2^-13, 1024] and a
// sample of the rest), so a clamp would never change a result there.  The
// conversion writes only the selected half of its destination; `a` is dead
// after the call, so its register serves as the destination without a move.
__device__ __forceinline__ uint32_t cvt4_nosat(float a, float b, float c, float d)
{
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)__float_as_uint(a), false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// SAT: e8m0 paths (scaled values reach 512 and need the clamp); !SAT: fp32
// multiplier paths
template <bool SAT>
__device__ __forceinline__ uint32_t cvt4_sel(float a, float b, float c, float d)
{
    if constexpr (SAT)
        return cvt4(a, b, c, d);
    else
        return cvt4_nosat(a, b, c, d);
}

// eight bf16 (one 16-byte load) times one multiplier -> eight bytes
__device__ __forceinline__ uint2 quant8(const uint4 &v, float s)
{
    uint2 r;
    r.x = cvt4(bf16_lo(v.x) * s, bf16_hi(v.x) * s, bf16_lo(v.y) * s, bf16_hi(v.y) * s);
    r.y = cvt4(bf16_lo(v.z) * s, bf16_hi(v.z) * s, bf16_lo(v.w) * s, bf16_hi(v.w) * s);
    return r;
}

// the same for an fp32 multiplier s = 448 / max(amax, eps) of a group or
// block containing every element of v (no clamp needed, see cvt4_nosat)
__device__ __forceinline__ uint2 quant8_fp32scale(const uint4 &v, float s)
{
    uint2 r;
    r.x = cvt4_nosat(bf16_lo(v.x) * s, bf16_hi(v.x) * s, bf16_lo(v.y) * s, bf16_hi(v.y) * s);
    r.y = cvt4_nosat(bf16_lo(v.z) * s, bf16_hi(v.z) * s, bf16_lo(v.w) * s, bf16_hi(v.w) * s);
    return r;
}

// bf16 element j (0..7) of a 16-byte load, as fp32
__device__ __forceinline__ float elem8(const uint4 &v, int j)
{
    uint32_t d = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return (j & 1) ? bf16_hi(d) : bf16_lo(d);
}

__device__ __forceinline__ uint32_t elem8_bits(const uint4 &v, int j)
{
    uint32_t d = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return (j & 1) ? (d >> 16) : (d & 0xffffu);
}

// global memory access helpers: 16-byte loads, 16/8-byte stores.  The
// streaming ("nt") forms carry the nontemporal hint: data read or written
// once should not displace lines that are still wanted in L2 / the MALL.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint4 ld16_nt(const uint16_t *p)
{
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(uint8_t *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }
__device__ __forceinline__ void st16_nt(uint8_t *p, uint4 v)
{
    u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
}
__device__ __forceinline__ void st8(uint8_t *p, uint2 v) { *reinterpret_cast<uint2 *>(p) = v; }
__device__ __forceinline__ void st8_nt(uint8_t *p, uint2 v)
{
    u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t *>(p));
}

// Raw buffer access (CDNA buffer descriptor: base, no stride, a byte range).
// A load whose bytes lie at or past `bytes` returns zeros and reads no
// memory, so loads past the end of a row, or of every row, need no branch.
// Branch-free loads matter for latency hiding: after loads issued under a
// condition the compiler can no longer count how many are outstanding and
// waits for all of them at the first use of any.  Word 3 is the gfx9-family
// raw-buffer format; aux 2 is the nontemporal hint.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte store through a buffer descriptor, nontemporal at device scope
// (aux 18: nt sc1), so the line is written through the XCD's L2 rather than
// left dirty in it: the 3D kernel's column runs measured 1% faster so.
__device__ __forceinline__ void stbuf16_nt_device(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint4 v)
{
    u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)byte_off, 0, 18);
}
__device__ __forceinline__ uint4 ldbuf16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ldbuf16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace mxq
