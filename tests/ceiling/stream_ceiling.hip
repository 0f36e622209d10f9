// Streaming probes for the practical HBM ceiling of the quantization
// kernels' traffic (bench infrastructure, not part of libmxq).
//
// Every probe walks n bf16 elements of a contiguous buffer with 16-byte
// nontemporal loads and / or 8-byte nontemporal stores of one byte per
// element, the access sizes and hints the quantizers use, and does no
// arithmetic worth the name:
//   mode 0  2 bytes read + 1 byte written per element (the quantizers' mix);
//   mode 1  2 bytes read per element (a word is stored only if the XOR of
//           everything read equals a value that never occurs, which keeps
//           the loads alive);
//   mode 2  1 byte written per element;
//   mode 3  as mode 0, the stores nontemporal at device scope (written
//           through the XCD's L2; the MX 3D kernel's store form), through a
//           buffer descriptor over the output;
//   mode 4  2 bytes read + 2 bytes written per element, 16-byte nontemporal
//           stores (the 1:1 mix of the scale re-layout).
// A workgroup of 256 threads handles 4 x 2048 consecutive elements, each
// thread issuing its four loads before its first store.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kPerBlock = (int64_t)kThreads * 8 * kUnroll;

// high byte of each of the eight bf16 values of a 16-byte load
__device__ __forceinline__ u32x2 pack_high_bytes(u32x4 v)
{
    u32x2 r;
    r.x = ((v.x >> 8) & 0xffu) | ((v.x >> 16) & 0xff00u) | (((v.y >> 8) & 0xffu) << 16) |
          ((v.y & 0xff000000u));
    r.y = ((v.z >> 8) & 0xffu) | ((v.z >> 16) & 0xff00u) | (((v.w >> 8) & 0xffu) << 16) |
          ((v.w & 0xff000000u));
    return r;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void stream_kernel(const uint16_t *__restrict__ in,
                                                          uint8_t *__restrict__ out, int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * kPerBlock + 8 * threadIdx.x;
    u32x4 v[kUnroll];
    if constexpr (MODE != 2) {   // modes 0, 1, 3, 4 read
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kThreads * 8;
            v[u] = e < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(in + e))
                         : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if constexpr (MODE == 0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kThreads * 8;
            if (e < n)
                __builtin_nontemporal_store(pack_high_bytes(v[u]), reinterpret_cast<u32x2 *>(out + e));
        }
    } else if constexpr (MODE == 3) {
        // out is at most 2^32 - 1 bytes (checked on the host)
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(out, (short)0, (int)0xFFFFFFFFu, 0x00020000);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kThreads * 8;
            if (e < n) {
                const u32x2 w = pack_high_bytes(v[u]);
                __builtin_amdgcn_raw_buffer_store_b64(w, rs, (int)(uint32_t)e, 0, 18);
            }
        }
    } else if constexpr (MODE == 4) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kThreads * 8;
            if (e < n)
                __builtin_nontemporal_store(v[u] ^ u32x4{1u, 1u, 1u, 1u},
                                            reinterpret_cast<u32x4 *>(out + 2 * e));
        }
    } else if constexpr (MODE == 1) {
        uint32_t acc = 0u;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        if (acc == 0x9E3779B9u && base < n)
            out[(blockIdx.x * kThreads + threadIdx.x) & 1023] = (uint8_t)acc;
    } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kThreads * 8;
            if (e < n) {
                const uint32_t w = (uint32_t)e;
                __builtin_nontemporal_store(u32x2{w, w ^ 0x5a5a5a5au}, reinterpret_cast<u32x2 *>(out + e));
            }
        }
    }
}

}  // namespace

// n: elements, a multiple of 8 (below 2^32 for mode 3); in: 2n bytes (modes
// 0, 1, 3, 4), out: n bytes (modes 0, 2, 3), 2n bytes (mode 4) or 1024
// bytes (mode 1); both 16-byte aligned.  Returns 0, or
// -1 for bad arguments, or the HIP error of the launch.
extern "C" int ceiling_stream(const void *in, void *out, int64_t n, int mode, void *stream)
{
    if (n <= 0 || n % 8 != 0 || mode < 0 || mode > 4 || !out || (mode != 2 && !in))
        return -1;
    if (mode == 3 && n > (int64_t)UINT32_MAX)
        return -1;
    const int64_t blocks = (n + kPerBlock - 1) / kPerBlock;
    if (blocks > INT32_MAX)
        return -1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const uint16_t *x = reinterpret_cast<const uint16_t *>(in);
    uint8_t *y = reinterpret_cast<uint8_t *>(out);
    if (mode == 0)
        stream_kernel<0><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(x, y, n);
    else if (mode == 1)
        stream_kernel<1><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(x, y, n);
    else if (mode == 3)
        stream_kernel<3><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(x, y, n);
    else if (mode == 4)
        stream_kernel<4><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(x, y, n);
    else
        stream_kernel<2><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(x, y, n);
    return (int)hipGetLastError();
}
