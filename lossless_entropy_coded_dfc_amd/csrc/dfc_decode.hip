// dfc_decode.hip - gfx950 decoder for DFC1 containers and its C-ABI launchers.
//
// DFloat11 blog ("70% Size, 100% Accuracy ... (DFloat11)"), section 03:
//   item 1: compact hierarchical lookup tables in on-chip memory find code
//           boundaries fast -> the first-level k-bit table and the per-length
//           canonical tables are copied into LDS by every workgroup;
//   item 2: a two-phase kernel; in phase one threads agree on read and write
//           positions through small auxiliary variables, phase two rebuilds
//           the weights -> per-chunk start offsets and per-block output
//           offsets come from the container, each lane counts the codes of
//           its chunk, a wavefront prefix scan turns counts into write
//           positions, and the exponents are written to LDS and merged with
//           the raw bytes into bf16 with coalesced 16-byte stores.
//
// Work decomposition: one lane per chunk (C bytes of code stream), one
// wavefront (64 lanes) per block of 64 chunks, several wavefronts per
// workgroup sharing one LDS copy of the decode tables.  All decoding is
// integer work on bit patterns.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "dfc.h"
#include "dfc_format.h"

namespace {

constexpr int kWave = 64;

struct ItemArgs {
    const uint32_t *words;     // code stream
    const uint32_t *offw;      // packed 5-bit chunk offsets
    const uint32_t *blockout;  // u32 out[n_blocks + 1]
    const uint8_t *raw;        // raw bytes (sign << 7 | mantissa), padded to 16
    const uint8_t *tables;     // derived decode tables
    uint16_t *dst;             // bf16 output
    uint64_t total_bits;
    uint32_t n_blocks;
    uint32_t wg_begin;         // first workgroup of this item in the grid
    uint32_t tables_bytes;     // multiple of 16
    uint32_t lut_bits;
};

struct BatchArgs {
    ItemArgs item[DFC_MAX_BATCH];
    uint32_t count;
    uint32_t blocks_per_wave;
    uint32_t stage_bytes;  // LDS exponent staging per wavefront
    uint32_t pad;
    uint32_t *status;
};

// LDS views of the per-length canonical tables (index = code length).
struct Tabs {
    const uint32_t *limit, *first, *base;
    const uint8_t *order;
};

// Codes longer than the first-level table: the smallest length l with
// window < limit[l] (left-justified 24-bit comparison), then the symbol by
// canonical rank.
__device__ __forceinline__ uint32_t long_code(uint32_t w24, int kb, const Tabs &t, uint32_t &sym) {
    uint32_t l = uint32_t(kb) + 1;
    while (l < 24u && w24 >= t.limit[l]) ++l;
    sym = t.order[t.base[l] + (w24 >> (24u - l)) - t.first[l]];
    return l;
}

// 5-bit chunk start offset i (little-endian bit array of u32 words).
__device__ __forceinline__ uint32_t off_field(const uint32_t *ow, uint64_t i) {
    const uint64_t g = 5ull * i;
    const uint32_t *p = ow + (g >> 5);
    return __builtin_amdgcn_alignbit(p[1], p[0], uint32_t(g & 31)) & 31u;
}

template <int C>
struct Chunk {
    static constexpr int NW = C / 4;
    uint32_t w[NW + 1];  // the chunk's words plus one lookahead word
};

template <int C>
__device__ __forceinline__ void load_chunk(const uint32_t *words, uint64_t chunk, Chunk<C> &ck) {
    const uint32_t *p = words + chunk * (C / 4);
    if constexpr (C == 4) {
        ck.w[0] = p[0];
    } else if constexpr (C == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        ck.w[0] = v.x;
        ck.w[1] = v.y;
    } else {
#pragma unroll
        for (int q = 0; q < C / 16; ++q) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p + 4 * q);
            ck.w[4 * q + 0] = v.x;
            ck.w[4 * q + 1] = v.y;
            ck.w[4 * q + 2] = v.z;
            ck.w[4 * q + 3] = v.w;
        }
    }
    ck.w[C / 4] = p[C / 4];
}

// Phase one: number of codes that start in [start, end) of this chunk (bit
// positions relative to the chunk's first bit).  The k-loop walks the chunk
// one 32-bit word at a time so that every window is a funnel shift of two
// registers: a code starting at pos in (32k, 32k + 32] lies inside words
// k and k + 1.  Each lookup counts every code that fits in the k-bit window
// (popcount of the boundary mask); the last lookup may count codes that
// start at or after `end`, which are subtracted at the end.
template <int C>
__device__ __forceinline__ int count_codes(const Chunk<C> &ck, int start, int end, const uint2 *lut, int kb,
                                           const Tabs &t) {
    int pos = start, cnt = 0, last_pos = 0;
    uint32_t last_mask = 0;
    const uint32_t kshift = 32u - uint32_t(kb);
#pragma unroll
    for (int k = -1; k < C / 4; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        const int top = 32 * (k + 1);
        const int lim = min(end, top + 1);
        while (pos < lim) {
            const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, uint32_t(top - pos));
            const uint32_t eh = lut[win >> kshift].y;
            const uint32_t mask = (eh >> 8) & 0xFFFu;
            if (mask == 0u) {
                uint32_t sym;
                pos += int(long_code(win >> 8, kb, t, sym));
                cnt += 1;
                last_mask = 0;
            } else {
                cnt += __popc(mask);
                last_pos = pos;
                last_mask = mask;
                pos += int((eh >> 20) & 0xFu);
            }
        }
    }
    if (pos > end && last_mask) cnt -= __popc(last_mask >> uint32_t(end - last_pos));
    return cnt;
}

// Phase two: decode the chunk again and write its `cnt` exponents to LDS.
// While four or more codes remain, all four symbol bytes of a lookup are
// stored: bytes past the lookup's own symbols land on positions this lane
// writes again in its next lookup.
template <int C>
__device__ __forceinline__ void write_codes(const Chunk<C> &ck, int start, int cnt, uint8_t *out,
                                            const uint2 *lut, int kb, const Tabs &t) {
    int pos = start, done = 0;
    const uint32_t kshift = 32u - uint32_t(kb);
#pragma unroll
    for (int k = -1; k < C / 4; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        const int top = 32 * (k + 1);
        while (done < cnt && pos <= top) {
            const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, uint32_t(top - pos));
            const uint2 e = lut[win >> kshift];
            const int ns = int(e.y & 0xFu);
            if (ns == 0) {
                uint32_t sym;
                pos += int(long_code(win >> 8, kb, t, sym));
                out[done] = uint8_t(sym);
                done += 1;
            } else if (cnt - done >= 4) {
                out[done + 0] = uint8_t(e.x);
                out[done + 1] = uint8_t(e.x >> 8);
                out[done + 2] = uint8_t(e.x >> 16);
                out[done + 3] = uint8_t(e.x >> 24);
                done += ns;
                pos += int((e.y >> 4) & 0xFu);
            } else {
                const int take = min(ns, cnt - done);
                out[done] = uint8_t(e.x);
                if (take > 1) out[done + 1] = uint8_t(e.x >> 8);
                if (take > 2) out[done + 2] = uint8_t(e.x >> 16);
                done += take;
                pos += int((e.y >> 4) & 0xFu);
            }
        }
    }
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

// Two bf16 values from the pair x = [raw_a, exp_a, raw_b, exp_b] (bytes, low
// to high): sign from raw bit 7, exponent, mantissa from raw bits 6..0.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t x) {
    return ((x >> 1) & 0x7F807F80u) | (x & 0x007F007Fu) | ((x << 8) & 0x80008000u);
}

__device__ __forceinline__ void assemble16(const uint4 &E, const uint4 &R, uint32_t o[8]) {
    const uint32_t e[4] = {E.x, E.y, E.z, E.w};
    const uint32_t r[4] = {R.x, R.y, R.z, R.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (r[q] & 0xFFu) | ((e[q] & 0xFFu) << 8) | ((r[q] & 0xFF00u) << 8) | ((e[q] & 0xFF00u) << 16);
        const uint32_t hi = ((r[q] >> 16) & 0xFFu) | ((e[q] >> 8) & 0xFF00u) | ((r[q] >> 8) & 0xFF0000u) |
                            (e[q] & 0xFF000000u);
        o[2 * q] = bf16_pair(lo);
        o[2 * q + 1] = bf16_pair(hi);
    }
}

template <int C>
__device__ __forceinline__ void decode_block(const ItemArgs &a, uint32_t b, int lane, uint8_t *stage,
                                             const uint2 *lut, const Tabs &t, uint32_t *status) {
    const uint64_t chunk = uint64_t(b) * kWave + uint32_t(lane);
    Chunk<C> ck;
    load_chunk<C>(a.words, chunk, ck);
    const int start = int(off_field(a.offw, chunk));
    const int next_off = int(off_field(a.offw, chunk + 1));
    const uint32_t s_out = __builtin_amdgcn_readfirstlane(a.blockout[b]);
    const uint32_t e_out = __builtin_amdgcn_readfirstlane(a.blockout[b + 1]);
    const int64_t rem = int64_t(a.total_bits) - int64_t(chunk * (8ull * C));
    const int end = int(min(int64_t(8 * C + next_off), max(rem, int64_t(-1))));
    const int kb = int(a.lut_bits);

    const int cnt = start < end ? count_codes<C>(ck, start, end, lut, kb, t) : 0;
    const int incl = wave_inclusive_scan(cnt, lane);
    const int total = __shfl(incl, kWave - 1, kWave);
    if (uint32_t(total) != e_out - s_out) {
        if (lane == 0 && status) atomicOr(status, 1u);
        return;
    }
    const uint32_t lead = s_out & 15u;
    if (cnt) write_codes<C>(ck, start, cnt, stage + lead + uint32_t(incl - cnt), lut, kb, t);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const uint32_t g0 = s_out >> 4, g1 = (e_out + 15u) >> 4;
    for (uint32_t g = g0 + uint32_t(lane); g < g1; g += kWave) {
        const uint4 E = *reinterpret_cast<const uint4 *>(stage + 16u * (g - g0));
        const uint4 R = *reinterpret_cast<const uint4 *>(a.raw + 16ull * g);
        uint32_t o[8];
        assemble16(E, R, o);
        const uint32_t j0 = 16u * g;
        uint16_t *d = a.dst + j0;
        if (j0 >= s_out && j0 + 16u <= e_out) {
            reinterpret_cast<uint4 *>(d)[0] = make_uint4(o[0], o[1], o[2], o[3]);
            reinterpret_cast<uint4 *>(d)[1] = make_uint4(o[4], o[5], o[6], o[7]);
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint32_t j = j0 + uint32_t(q);
                if (j >= s_out && j < e_out) d[q] = uint16_t(o[q >> 1] >> (16 * (q & 1)));
            }
        }
    }
    // The next block reuses this wavefront's staging area.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int C>
__global__ __launch_bounds__(1024) void dfc_decode_kernel(const BatchArgs args) {
    extern __shared__ __align__(16) uint8_t lds[];
    const uint32_t wg = blockIdx.x;
    uint32_t it = 0;
    for (uint32_t k = 1; k < args.count; ++k)
        if (wg >= args.item[k].wg_begin) it = k;
    const ItemArgs &a = args.item[it];

    // Stage the decode tables in LDS (16 bytes per thread per step).
    for (uint32_t o = threadIdx.x * 16u; o < a.tables_bytes; o += blockDim.x * 16u)
        *reinterpret_cast<uint4 *>(lds + o) = *reinterpret_cast<const uint4 *>(a.tables + o);
    __syncthreads();

    const int kb = int(a.lut_bits);
    const uint2 *lut = reinterpret_cast<const uint2 *>(lds);
    Tabs t;
    t.limit = reinterpret_cast<const uint32_t *>(lds + (8u << kb));
    t.first = t.limit + 32;
    t.base = t.limit + 64;
    t.order = lds + (8u << kb) + 384;

    const uint32_t waves = blockDim.x / kWave;
    const uint32_t wave = threadIdx.x / kWave;
    const int lane = int(threadIdx.x % kWave);
    uint8_t *stage = lds + a.tables_bytes + wave * args.stage_bytes;
    const uint32_t per_wg = waves * args.blocks_per_wave;
    const uint32_t first = (wg - a.wg_begin) * per_wg;
    for (uint32_t r = 0; r < args.blocks_per_wave; ++r) {
        const uint32_t b = first + r * waves + wave;
        if (b >= a.n_blocks) break;
        decode_block<C>(a, b, lane, stage, lut, t, args.status);
    }
}

// ------------------------------------------------------------------ launch

struct LaunchCfg {
    uint32_t waves = 0, blocks_per_wave = 0;
} g_launch;

int device_cu_count() {
    static int cus = 0;
    static std::once_flag once;
    std::call_once(once, [] {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    });
    return cus;
}

template <int C>
dfc_status launch_group(const dfc_batch_item *items, const uint32_t *idx, uint32_t count, uint32_t *status,
                        hipStream_t stream) {
    BatchArgs args;
    std::memset(&args, 0, sizeof(args));
    uint32_t min_len = 24, max_tables = 0;
    uint64_t total_blocks = 0;
    for (uint32_t k = 0; k < count; ++k) {
        const dfc_info &in = *items[idx[k]].info;
        min_len = std::min(min_len, std::max(1u, in.min_len));
        max_tables = std::max<uint32_t>(max_tables, uint32_t(in.tables_bytes));
        total_blocks += in.n_blocks;
    }
    const uint32_t stage = uint32_t((16 + kWave * dfc::ceil_div(8ull * C, min_len) + 16 + 15) & ~15ull);
    const uint32_t tbytes = (max_tables + 15u) & ~15u;
    uint32_t waves = g_launch.waves ? g_launch.waves : 8;
    while (waves > 1 && tbytes + waves * stage > 160u * 1024u) waves /= 2;
    if (tbytes + waves * stage > 160u * 1024u) return DFC_EUNSUPPORTED;
    uint32_t bpw = g_launch.blocks_per_wave;
    if (!bpw) {
        const uint64_t target_wgs = uint64_t(device_cu_count()) * 2;
        bpw = uint32_t(std::min<uint64_t>(16, std::max<uint64_t>(1, total_blocks / (target_wgs * waves))));
    }
    const uint32_t per_wg = waves * bpw;
    uint32_t wg = 0, used = 0;
    for (uint32_t k = 0; k < count; ++k) {
        const dfc_batch_item &bi = items[idx[k]];
        const dfc_info &in = *bi.info;
        if (in.n_blocks == 0) continue;
        const uint8_t *base = static_cast<const uint8_t *>(bi.blob_dev);
        ItemArgs &a = args.item[used++];
        a.words = reinterpret_cast<const uint32_t *>(base + in.off_words);
        a.offw = reinterpret_cast<const uint32_t *>(base + in.off_offsets);
        a.blockout = reinterpret_cast<const uint32_t *>(base + in.off_blockout);
        a.raw = base + in.off_raw;
        a.tables = base + in.off_tables;
        a.dst = bi.dst_dev;
        a.total_bits = in.total_bits;
        a.n_blocks = uint32_t(in.n_blocks);
        a.wg_begin = wg;
        a.tables_bytes = uint32_t((in.tables_bytes + 15) & ~15ull);
        a.lut_bits = in.lut_bits;
        wg += uint32_t(dfc::ceil_div(in.n_blocks, per_wg));
    }
    if (used == 0) return DFC_OK;
    args.count = used;
    args.blocks_per_wave = bpw;
    args.stage_bytes = stage;
    args.status = status;
    const uint32_t lds = tbytes + waves * stage;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(&dfc_decode_kernel<C>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
            return DFC_EHIP;
        attr_set = true;
    }
    hipLaunchKernelGGL(dfc_decode_kernel<C>, dim3(wg), dim3(waves * kWave), lds, stream, args);
    return hipGetLastError() == hipSuccess ? DFC_OK : DFC_EHIP;
}

dfc_status check_item(const dfc_batch_item &it) {
    if (!it.info) return DFC_EINVAL;
    const dfc_info &in = *it.info;
    if (it.n != in.n) return DFC_ESIZE;
    if (in.n == 0) return DFC_OK;
    if (!it.blob_dev || !it.dst_dev) return DFC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(it.blob_dev) & 255u) || (reinterpret_cast<uintptr_t>(it.dst_dev) & 15u))
        return DFC_EINVAL;
    if (in.layout != DFC_LAYOUT_FLAT) return DFC_EUNSUPPORTED;
    if (in.lanes_per_block != 64) return DFC_EUNSUPPORTED;
    const uint32_t C = in.chunk_bytes;
    if (C != 4 && C != 8 && C != 16 && C != 32) return DFC_EINVAL;
    if (in.lut_bits < 8 || in.lut_bits > 12 || in.min_len < 1) return DFC_EINVAL;
    return DFC_OK;
}

}  // namespace

extern "C" {

dfc_status dfc_set_launch(uint32_t waves_per_group, uint32_t blocks_per_wave) {
    if (waves_per_group && waves_per_group != 4 && waves_per_group != 8 && waves_per_group != 16) return DFC_EINVAL;
    if (blocks_per_wave > 64) return DFC_EINVAL;
    g_launch.waves = waves_per_group;
    g_launch.blocks_per_wave = blocks_per_wave;
    return DFC_OK;
}

dfc_status dfc_decode_batch(const dfc_batch_item *items, uint32_t count, uint32_t *status_dev, void *stream) {
    if (count == 0) return DFC_OK;
    if (!items || count > DFC_MAX_BATCH) return DFC_EINVAL;
    for (uint32_t k = 0; k < count; ++k) {
        dfc_status s = check_item(items[k]);
        if (s != DFC_OK) return s;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    static const int sizes[4] = {4, 8, 16, 32};
    for (int c : sizes) {
        uint32_t idx[DFC_MAX_BATCH], m = 0;
        for (uint32_t k = 0; k < count; ++k)
            if (items[k].info->n && items[k].info->chunk_bytes == uint32_t(c)) idx[m++] = k;
        if (!m) continue;
        dfc_status s = DFC_OK;
        switch (c) {
            case 4: s = launch_group<4>(items, idx, m, status_dev, st); break;
            case 8: s = launch_group<8>(items, idx, m, status_dev, st); break;
            case 16: s = launch_group<16>(items, idx, m, status_dev, st); break;
            default: s = launch_group<32>(items, idx, m, status_dev, st); break;
        }
        if (s != DFC_OK) return s;
    }
    return DFC_OK;
}

dfc_status dfc_decode(const void *blob_dev, const dfc_info *info, uint16_t *dst_dev, uint64_t n,
                      uint32_t *status_dev, void *stream) {
    dfc_batch_item it;
    it.blob_dev = blob_dev;
    it.info = info;
    it.dst_dev = dst_dev;
    it.n = n;
    return dfc_decode_batch(&it, 1, status_dev, stream);
}

}  // extern "C"
