// dfc_probe.hip - a streaming ceiling for the benchmark (libdfc_probe.so; not
// part of the codec and not linked into libdfc).
//
// The decoder reads about 1.34 bytes and writes 2 bytes per weight.  This
// kernel moves 1 byte in and 2 bytes out per value with nothing else to do:
// a grid-stride loop over octets (8 bytes read, 16 bytes written per lane
// and step, 1 KB contiguous per wavefront store), the simplest kernel with
// the decoder's read/write mix.  Its rate is what a streaming kernel of that
// mix reaches on the chip, next to the 8 TB/s peak the roofline is priced
// against.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

using u32x2 = __attribute__((ext_vector_type(2))) uint32_t;
using u32x4 = __attribute__((ext_vector_type(4))) uint32_t;

// UNROLL octets per lane in flight per step.
template <int UNROLL>
__global__ __launch_bounds__(256) void expand_kernel(const uint8_t *src, uint16_t *dst, uint64_t octets) {
    const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
    uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < octets; i += UNROLL * stride) {
        u32x2 r[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) r[u] = *reinterpret_cast<const u32x2 *>(src + 8 * (i + u * stride));
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            // byte b -> 16-bit value b << 8 | b (any expansion; the work is the bytes)
            const uint32_t a = r[u].x, b = r[u].y;
            const u32x4 o = {__builtin_amdgcn_perm(0u, a, 0x01010000u), __builtin_amdgcn_perm(0u, a, 0x03030202u),
                             __builtin_amdgcn_perm(0u, b, 0x01010000u), __builtin_amdgcn_perm(0u, b, 0x03030202u)};
            *reinterpret_cast<u32x4 *>(dst + 8 * (i + u * stride)) = o;
        }
    }
    for (; i < octets; i += stride) {
        const u32x2 r = *reinterpret_cast<const u32x2 *>(src + 8 * i);
        const u32x4 o = {__builtin_amdgcn_perm(0u, r.x, 0x01010000u), __builtin_amdgcn_perm(0u, r.x, 0x03030202u),
                         __builtin_amdgcn_perm(0u, r.y, 0x01010000u), __builtin_amdgcn_perm(0u, r.y, 0x03030202u)};
        *reinterpret_cast<u32x4 *>(dst + 8 * i) = o;
    }
}

}  // namespace

extern "C" {

// dst[j] = src[j] * 0x0101 for j < 8 * octets.  src 8-byte and dst 16-byte
// aligned; grid workgroups of 256 threads; unroll 1, 2 or 4.  Returns 0, or
// -1 on bad arguments, -5 on a launch failure.
int dfc_probe_expand(const void *src, void *dst, uint64_t octets, uint32_t grid, uint32_t unroll, void *stream) {
    if (!src || !dst || !grid || (reinterpret_cast<uintptr_t>(src) & 7u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
        return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint8_t *s = static_cast<const uint8_t *>(src);
    uint16_t *d = static_cast<uint16_t *>(dst);
    switch (unroll) {
        case 1: expand_kernel<1><<<dim3(grid), dim3(256), 0, st>>>(s, d, octets); break;
        case 2: expand_kernel<2><<<dim3(grid), dim3(256), 0, st>>>(s, d, octets); break;
        case 4: expand_kernel<4><<<dim3(grid), dim3(256), 0, st>>>(s, d, octets); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
