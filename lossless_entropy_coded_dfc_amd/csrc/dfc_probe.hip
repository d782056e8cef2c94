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

// The decoder's schedule without its decoding: "blocks" of kBlockRounds
// rounds of 512 values (8 bytes read and 16 written per lane and round, as
// the decoder's raw bytes and output) plus 1 KB of stream words read per
// block, a wavefront decoding block after block with the next block's loads
// in flight while it stores the current one.  run = 0: each wavefront takes
// one contiguous share of the blocks; run > 0: runs of `run` blocks dealt to
// the wavefronts in turn (first wavefront of every workgroup first), as the
// decoder deals them.
constexpr int kBlockRounds = 6;

__global__ __launch_bounds__(512) void schedule_kernel(const uint8_t *src, const uint32_t *words, uint16_t *dst,
                                                       uint32_t nblocks, uint32_t run) {
    const uint32_t lane = threadIdx.x % 64u;
    const uint32_t waves = blockDim.x / 64u;
    const uint32_t V = gridDim.x * waves;
    const uint32_t v = (threadIdx.x / 64u) * gridDim.x + blockIdx.x;
    uint32_t b, b_end, step_runs, len;
    if (run == 0) {
        len = (nblocks + V - 1u) / V;
        b = min(v * len, nblocks);
        step_runs = 0;
    } else {
        len = run;
        b = min(v, (nblocks + run - 1u) / run) * run;
        step_runs = V * run;
    }
    b_end = min(b + len, nblocks);
    if (b >= b_end) return;
    auto raw_at = [&](uint32_t blk, int j) { return uint64_t(blk) * (kBlockRounds * 512) + 512u * j + 8u * lane; };
    struct Raw {
        u32x2 v[kBlockRounds];
    } r, rn;
    u32x4 w;
#pragma unroll
    for (int j = 0; j < kBlockRounds; ++j) r.v[j] = *reinterpret_cast<const u32x2 *>(src + raw_at(b, j));
    w = *reinterpret_cast<const u32x4 *>(words + uint64_t(b) * 256u + 4u * lane);
    for (;;) {
        // the next block: this run's next, or the first of the next run
        uint32_t bn = b + 1u, bn_end = b_end;
        if (bn >= b_end) {
            bn = step_runs ? b_end - len + step_runs : nblocks;
            bn_end = min(bn + len, nblocks);
        }
        const bool more = bn < bn_end;
        u32x4 wn = {0u, 0u, 0u, 0u};
        if (more) {
#pragma unroll
            for (int j = 0; j < kBlockRounds; ++j) rn.v[j] = *reinterpret_cast<const u32x2 *>(src + raw_at(bn, j));
            wn = *reinterpret_cast<const u32x4 *>(words + uint64_t(bn) * 256u + 4u * lane);
        }
        // the stream words are zeros: folding them in keeps their loads
        const uint32_t k = w.x ^ w.y ^ w.z ^ w.w;
#pragma unroll
        for (int j = 0; j < kBlockRounds; ++j) {
            const uint32_t a = r.v[j].x, c = r.v[j].y;
            const u32x4 o = {k ^ __builtin_amdgcn_perm(0u, a, 0x01010000u), __builtin_amdgcn_perm(0u, a, 0x03030202u),
                             __builtin_amdgcn_perm(0u, c, 0x01010000u), __builtin_amdgcn_perm(0u, c, 0x03030202u)};
            *reinterpret_cast<u32x4 *>(dst + raw_at(b, j)) = o;
        }
        if (!more) break;
        r = rn;
        w = wn;
        b = bn;
        b_end = bn_end;
    }
}

}  // namespace

extern "C" {

// The schedule probe over nblocks blocks of 3,072 values: src holds 3,072
// bytes and words 1,024 bytes (zeros) per block, dst 6,144; grid workgroups
// of `threads` (a multiple of 64, at most 512) threads; run as above (at
// most 64).  Returns 0, or -1 on bad arguments, -5 on a launch failure.
int dfc_probe_schedule(const void *src, const void *words, void *dst, uint32_t nblocks, uint32_t grid,
                       uint32_t threads, uint32_t run, void *stream) {
    if (!src || !words || !dst || !grid || !threads || threads % 64u || threads > 512u || run > 64u ||
        (reinterpret_cast<uintptr_t>(src) & 7u) || (reinterpret_cast<uintptr_t>(words) & 15u) ||
        (reinterpret_cast<uintptr_t>(dst) & 15u))
        return -1;
    schedule_kernel<<<dim3(grid), dim3(threads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint8_t *>(src), static_cast<const uint32_t *>(words), static_cast<uint16_t *>(dst), nblocks,
        run);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}


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
