// dfc_decode.hip - gfx950 decoder for DFC1 containers and its C-ABI launchers.
//
// DFloat11 blog ("70% Size, 100% Accuracy ... (DFloat11)"), section 03:
//   item 1: compact hierarchical lookup tables in on-chip memory find code
//           boundaries fast -> the first-level k-bit tables (step, symbols,
//           boundary mask) and the per-length canonical tables for longer
//           codes are copied into LDS once per workgroup;
//   item 2: a two-phase kernel; in phase one threads agree on read and write
//           positions through small auxiliary variables, phase two rebuilds
//           the weights -> per-chunk start offsets and per-block output
//           offsets come from the container, each lane counts the codes of
//           its chunk, a wavefront prefix scan turns counts into write
//           positions, the exponents go to LDS and are merged with the raw
//           bytes into bf16 with coalesced 16-byte stores.  Containers in the
//           padded layout have no chunk offsets: there every chunk starts
//           with a code and ends with its last whole code.
//
// Work decomposition: one lane per chunk (C bytes of code stream), one
// wavefront (64 lanes) per block of 64 chunks.  Workgroups are persistent:
// the grid is sized to the resident capacity of the GPU, each workgroup owns
// a contiguous run of blocks of one matrix, and its wavefronts take those
// blocks in turn while prefetching the next block's stream words, offsets
// and raw bytes.  All decoding is integer work on bit patterns.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <vector>

#include "dfc.h"
#include "dfc_ans_launch.h"
#include "dfc_decode_core.h"
#include "dfc_format.h"

namespace {

struct ItemArgs {
    const uint32_t *words;     // code stream (with its guard words)
    const uint32_t *offw;      // packed 5-bit chunk offsets
    const uint32_t *blockout;  // u32 out[n_blocks + 1]
    const uint8_t *raw;        // raw bytes (sign << 7 | mantissa), padded to 16
    const uint8_t *tables;     // derived decode tables
    uint16_t *dst;             // bf16 output
    uint64_t total_bits;
    uint32_t words_bytes, offw_bytes, raw_bytes, dst_bytes;  // buffer ranges
    uint32_t n_blocks;
    uint32_t wg_begin;         // first workgroup of this item in the grid
    uint32_t blocks_per_wg;
    uint32_t tables_bytes;     // multiple of 16
    uint32_t lut_bits;
    uint32_t pad;
};

struct Buffers {
    __amdgpu_buffer_rsrc_t words, offw, raw, dst;
};

__device__ __forceinline__ Buffers make_buffers(const ItemArgs &a) {
    Buffers r;
    r.words = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(a.words), 0, int(a.words_bytes), kBufferConfig);
    r.offw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(a.offw), 0, int(a.offw_bytes), kBufferConfig);
    r.raw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.raw), 0, int(a.raw_bytes), kBufferConfig);
    r.dst = __builtin_amdgcn_make_buffer_rsrc(a.dst, 0, int(a.dst_bytes), kBufferConfig);
    return r;
}

struct BatchArgs {
    ItemArgs item[DFC_MAX_BATCH];
    uint32_t count;
    uint32_t stage_bytes;  // LDS exponent staging per wavefront (multiple of 16)
    uint32_t *status;
};

// Rounds of raw-byte octets (512 values per wavefront per round) prefetched
// into registers before decoding: enough for a block of 64 chunks at about
// 4 bits per code.
template <int C>
struct Prefetch {
    static constexpr int N = C >= 32 ? 12 : C / 2;
};

// Wavefronts per SIMD the register budget is sized for (512 VGPRs per lane
// shared by the resident wavefronts): 64 VGPRs give 8, the 32-byte chunk
// path needs more registers and settles for 5.
template <int C>
struct Occupancy {
    static constexpr int kWavesPerSimd = C >= 32 ? 5 : 8;
};

// Output range of one block and its octets (8 values, 16 output bytes).
// Octets [full0, full1) lie wholly inside [s_out, e_out); the first and the
// last octet may be shared with the neighbouring blocks.
struct BlockRange {
    uint32_t s_out, e_out;
    uint32_t h0, nh;  // first octet, number of octets
    uint32_t full0, full1;
};

__device__ __forceinline__ BlockRange block_range(uint32_t s_out, uint32_t e_out) {
    BlockRange r;
    r.s_out = s_out;
    r.e_out = e_out;
    r.h0 = s_out >> 3;
    r.nh = ((e_out + 7u) >> 3) - r.h0;
    r.full0 = (s_out & 7u) ? 1u : 0u;
    r.full1 = (e_out & 7u) ? r.nh - 1u : r.nh;
    return r;
}

// Octet i of the block (one per lane): whole octets go out as one 16-byte
// buffer store (1 KB contiguous per wavefront); a shared octet stores only
// its values inside the block, one 16-bit store each.
__device__ __forceinline__ void store_octet(const Buffers &bf, const BlockRange &br, uint32_t i, const u32x4 &o) {
    const uint32_t h = br.h0 + i;
    const bool full = i - br.full0 < br.full1 - br.full0;
    __builtin_amdgcn_raw_buffer_store_b128(o, bf.dst, full ? 16u * h : kNowhere, 0, 0);
    if (!full && i < br.nh) {
        // values [lo, hi) of the octet are the block's; value q goes out iff
        // q - lo < hi - lo (unsigned)
        const uint32_t lo = uint32_t(max(int(br.s_out) - int(8u * h), 0));
        const uint32_t span = min(br.e_out - 8u * h, 8u) - lo;
        const uint32_t v[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // (kNowhere + 14 is still past every range)
            const uint32_t at = (uint32_t(q) - lo < span ? 16u * h : kNowhere) + 2u * uint32_t(q);
            __builtin_amdgcn_raw_buffer_store_b16(uint16_t(v[q >> 1] >> (16 * (q & 1))), bf.dst, at, 0, 0);
        }
    }
}

template <int C, bool Padded>
__device__ __forceinline__ void decode_block(const ItemArgs &a, const Buffers &bf, uint32_t b, uint32_t lane,
                                             const Chunk<C> &ck, uint8_t *stage, uint32_t stage_off,
                                             uint32_t stage_bytes, const Tables &t, uint32_t *status,
                                             const u32x2 (&R)[Prefetch<C>::N], const BlockRange &br,
                                             const Chunk<C> &nxt) {
    constexpr int PF = Prefetch<C>::N;
    // Zero the staging bytes this block ORs its exponents into: lead, the
    // block's exponents, and the spill of its last lookup.
    const uint32_t nz = min((br.s_out & 7u) + (br.e_out - br.s_out) + 8u, stage_bytes);
    for (uint32_t o = 16u * lane; o + 16u <= ((nz + 15u) & ~15u); o += 16u * kWave)
        *reinterpret_cast<uint4 *>(stage + o) = make_uint4(0, 0, 0, 0);
    const uint32_t chunk = b * kWave + lane;
    // Stream bits from this lane's chunk to the end of the stream: only the
    // last block needs them per lane (a uniform 64-bit test, then 32 bits).
    const int64_t block_left = int64_t(a.total_bits) - int64_t(uint64_t(b) * (uint64_t(kWave) * 8u * C));
    const int bits_left = block_left >= int64_t(kWave) * (8 * C + 32)
                              ? (8 * C + 32)
                              : max(int(block_left) - int(lane) * (8 * C), -1);
    int start = 0, end;
    if constexpr (Padded)
        end = min(8 * C, bits_left);
    else
        chunk_span<C>(ck, chunk, bits_left, start, end);

    // The count and write passes run at a raised wave priority, so that the
    // wavefronts that are decoding get issue slots ahead of those that are
    // storing, which keeps stores queued behind the decode (1% in one-process
    // timing); the store rounds drop back to the normal priority.
    __builtin_amdgcn_s_setprio(1);
    uint32_t cnt = 0;
    if (start < end) cnt = Padded ? count_codes_padded<C>(ck, end, t) : count_codes<C>(ck, start, end, t);
    const uint32_t incl = wave_inclusive_scan(cnt);
    const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
    // A chunk of 8C bits holds at most 8C code starts; anything else (or a
    // total that disagrees with the block offsets) means a corrupt stream.
    const bool bad = (total != br.e_out - br.s_out) | (__builtin_amdgcn_ballot_w64(cnt > 8u * C) != 0);
    const uint32_t lead = br.s_out & 7u;
    if (!bad && cnt) {
        if constexpr (Padded)
            write_codes_padded<C>(ck, end, cnt, stage - stage_off, stage_off + lead + (incl - cnt), t);
        else
            write_codes<C>(ck, start, end, stage - stage_off, stage_off + lead + (incl - cnt), t);
    }
    // Everything prefetched must be in registers before the first store, on
    // every path to the next block.
    wait_for(R);
    wait_for(nxt);
    if (bad) {
        if (lane == 0 && status) atomicOr(status, kStatusCorrupt);
        return;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    __builtin_amdgcn_s_setprio(0);
    // Lanes past the block's last octet read its last staged octet again and
    // store nowhere.
    const uint32_t last = br.nh - 1u;
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        if (uint32_t(kWave * j) < br.nh) {
            const uint32_t i = lane + uint32_t(kWave * j);
            const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + 8u * min(i, last));
            store_octet(bf, br, i, assemble8(E, R[j]));
        }
    }
    for (uint32_t j0 = uint32_t(kWave * PF); j0 < br.nh; j0 += kWave) {
        const uint32_t i = lane + j0;
        const u32x2 Ri = __builtin_amdgcn_raw_buffer_load_b64(bf.raw, i < br.nh ? 8u * (br.h0 + i) : kNowhere, 0, 0);
        const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + 8u * min(i, last));
        store_octet(bf, br, i, assemble8(E, Ri));
    }
    // The next block reuses this wavefront's staging area.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int C, bool Padded>
__global__ __launch_bounds__(1024, Occupancy<C>::kWavesPerSimd) void dfc_decode_kernel(const BatchArgs args) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int PF = Prefetch<C>::N;
    const uint32_t wg = blockIdx.x;
    uint32_t it = 0;
    for (uint32_t k = 1; k < args.count; ++k)
        if (wg >= args.item[k].wg_begin) it = k;
    const ItemArgs a = args.item[it];
    const Buffers bf = make_buffers(a);
    const const_u32_ptr blockout = (const_u32_ptr)(a.blockout);

    const Tables t = stage_tables(lds, a.tables, a.tables_bytes, a.lut_bits);

    const uint32_t waves = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t stage_off = a.tables_bytes + wave * args.stage_bytes;
    uint8_t *stage = lds + stage_off;
    const uint32_t lo_b = (wg - a.wg_begin) * a.blocks_per_wg;
    const uint32_t hi_b = min(lo_b + a.blocks_per_wg, a.n_blocks);

    uint32_t b = lo_b + wave;
    if (b >= hi_b) return;
    Chunk<C> cur;
    load_chunk<C, !Padded>(bf.words, bf.offw, b * kWave + lane, cur);
    uint32_t s_out = blockout[b], e_out = blockout[b + 1];
    // Resident on entry, as it is on every later iteration (see wait_for).
    wait_for(cur);
    for (;;) {
        // the block index is the same in every lane
        b = __builtin_amdgcn_readfirstlane(b);
        const BlockRange br = block_range(s_out, e_out);
        // raw bytes of this block's first PF octets per lane (rounds past the
        // block's last octet load nothing)
        u32x2 R[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const uint32_t i = lane + uint32_t(kWave * j);
            R[j] = uint32_t(kWave * j) < br.nh
                       ? __builtin_amdgcn_raw_buffer_load_b64(bf.raw, i < br.nh ? 8u * (br.h0 + i) : kNowhere, 0, 0)
                       : u32x2{0u, 0u};
        }
        // next block's stream words, offsets and output range
        const uint32_t bn = b + waves;
        const bool more = bn < hi_b;
        Chunk<C> nxt{};
        uint32_t s_nxt = 0, e_nxt = 0;
        if (more) {
            load_chunk<C, !Padded>(bf.words, bf.offw, bn * kWave + lane, nxt);
            s_nxt = blockout[bn];
            e_nxt = blockout[bn + 1];
        }
        decode_block<C, Padded>(a, bf, b, lane, cur, stage, stage_off, args.stage_bytes, t, args.status, R, br, nxt);
        if (!more) break;
        cur = nxt;
        b = bn;
        s_out = s_nxt;
        e_out = e_nxt;
    }
}

// ------------------------------------------------------------------ launch

// Set by dfc_set_launch, read by every launch (possibly on other threads).
struct LaunchCfg {
    std::atomic<uint32_t> waves{0}, blocks_per_wave{0};
} g_launch;

// Split `slots` workgroups across items so that the largest per-workgroup
// block count is as small as possible (each item gets at least one).
std::vector<uint32_t> share_workgroups(const std::vector<uint64_t> &blocks, uint64_t slots, uint32_t per_wg_min) {
    const size_t m = blocks.size();
    std::vector<uint32_t> g(m, 1);
    uint64_t used = m;
    auto load = [&](size_t i) { return dfc::ceil_div(blocks[i], g[i]); };
    while (used < slots) {
        size_t best = 0;
        for (size_t i = 1; i < m; ++i)
            if (load(i) > load(best)) best = i;
        if (load(best) <= per_wg_min) break;
        g[best]++;
        used++;
    }
    return g;
}

template <int C, bool Padded>
dfc_status launch_group(const dfc_batch_item *items, const uint32_t *idx, uint32_t count, uint32_t *status,
                        hipStream_t stream) {
    BatchArgs args;
    std::memset(&args, 0, sizeof(args));
    uint32_t max_tables = 0, max_block = 0;
    std::vector<uint64_t> blocks;
    std::vector<uint32_t> live;
    for (uint32_t k = 0; k < count; ++k) {
        const dfc_info &in = *items[idx[k]].info;
        if (in.n_blocks == 0) continue;
        live.push_back(idx[k]);
        blocks.push_back(in.n_blocks);
        max_tables = std::max<uint32_t>(max_tables, uint32_t((in.tables_bytes + 15) & ~15ull));
        max_block = std::max(max_block, in.max_block_elems);
    }
    if (live.empty()) return DFC_OK;
    // staging: lead (< 8) + elements + spill of the last lookup, rounded to 16
    const uint32_t stage = (max_block + 32u + 15u) & ~15u;
    if (!allow_full_lds(reinterpret_cast<const void *>(&dfc_decode_kernel<C, Padded>))) return DFC_EHIP;
    // Resident workgroups per CU for w wavefronts each, under both the LDS
    // and the register budget.
    auto resident = [&](uint32_t w) -> int {
        const uint32_t lds = max_tables + w * stage;
        if (lds > kLdsBytes) return 0;
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&dfc_decode_kernel<C, Padded>),
                                                         int(w * kWave), size_t(lds)) != hipSuccess)
            per_cu = int(kLdsBytes / lds);
        return per_cu;
    };
    // waves per workgroup: the most resident wavefronts per CU, then the
    // larger workgroup (fewer table copies)
    uint32_t waves = g_launch.waves.load(std::memory_order_relaxed);
    const uint32_t blocks_per_wave = g_launch.blocks_per_wave.load(std::memory_order_relaxed);
    if (!waves) {
        uint32_t best = 0;
        for (uint32_t w = 4; w <= kMaxWaves; ++w) {
            const uint32_t r = uint32_t(std::max(0, resident(w))) * w;
            if (r >= best && r > 0) {
                best = r;
                waves = w;
            }
        }
    }
    if (!waves) waves = 1;
    while (waves > 1 && max_tables + waves * stage > kLdsBytes) --waves;
    const uint32_t lds = max_tables + waves * stage;
    if (lds > kLdsBytes) return DFC_EUNSUPPORTED;
    int per_cu = resident(waves);
    if (per_cu <= 0) per_cu = 1;
    uint64_t slots = uint64_t(per_cu) * uint64_t(device_cu_count());
    if (blocks_per_wave) {
        // fixed work per workgroup instead of filling the machine exactly
        uint64_t total = 0;
        for (uint64_t nb : blocks) total += dfc::ceil_div(nb, uint64_t(waves) * blocks_per_wave);
        slots = total;
    }
    const std::vector<uint32_t> g =
        share_workgroups(blocks, std::max<uint64_t>(slots, live.size()), waves);
    uint32_t wg = 0;
    for (size_t k = 0; k < live.size(); ++k) {
        const dfc_batch_item &bi = items[live[k]];
        const dfc_info &in = *bi.info;
        const uint8_t *base = static_cast<const uint8_t *>(bi.blob_dev);
        ItemArgs &a = args.item[k];
        a.words = reinterpret_cast<const uint32_t *>(base + in.off_words);
        a.offw = reinterpret_cast<const uint32_t *>(base + in.off_offsets);
        a.blockout = reinterpret_cast<const uint32_t *>(base + in.off_blockout);
        a.raw = base + in.off_raw;
        a.tables = base + in.off_tables;
        a.dst = bi.dst_dev;
        a.words_bytes = uint32_t(in.words_bytes);
        a.offw_bytes = uint32_t(in.offsets_bytes);
        a.raw_bytes = uint32_t(in.raw_bytes);
        a.dst_bytes = uint32_t(2 * in.n);
        a.total_bits = in.total_bits;
        a.n_blocks = uint32_t(in.n_blocks);
        a.blocks_per_wg = uint32_t(dfc::ceil_div(in.n_blocks, g[k]));
        a.wg_begin = wg;
        a.tables_bytes = uint32_t((in.tables_bytes + 15) & ~15ull);
        a.lut_bits = in.lut_bits;
        wg += uint32_t(dfc::ceil_div(in.n_blocks, a.blocks_per_wg));
    }
    args.count = uint32_t(live.size());
    args.stage_bytes = stage;
    args.status = status;
    dfc_decode_kernel<C, Padded><<<dim3(wg), dim3(waves * kWave), lds, stream>>>(args);
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
    if (in.layout == DFC_LAYOUT_ANS) return dfc::ans_check_item(it);
    if (in.layout != DFC_LAYOUT_FLAT && in.layout != DFC_LAYOUT_PADDED) return DFC_EUNSUPPORTED;
    if (in.lanes_per_block != 64) return DFC_EUNSUPPORTED;
    const uint32_t C = in.chunk_bytes;
    if (C != 4 && C != 8 && C != 16 && C != 32) return DFC_EINVAL;
    if (in.lut_bits < 8 || in.lut_bits > 12 || in.min_len < 1) return DFC_EINVAL;
    if (in.max_block_elems > 64u * dfc::ceil_div(8ull * C, in.min_len)) return DFC_EINVAL;
    // Every stream is addressed with 32-bit byte offsets below kNowhere.
    const uint64_t limit = kNowhere - 64u * 1024u;
    if (2 * in.n > limit || in.words_bytes > limit || in.offsets_bytes > limit || in.raw_bytes > limit)
        return DFC_EUNSUPPORTED;
    return DFC_OK;
}

}  // namespace

extern "C" {

dfc_status dfc_set_launch(uint32_t waves_per_group, uint32_t blocks_per_wave) {
    if (waves_per_group > kMaxWaves) return DFC_EINVAL;
    if (blocks_per_wave > 64) return DFC_EINVAL;
    g_launch.waves.store(waves_per_group, std::memory_order_relaxed);
    g_launch.blocks_per_wave.store(blocks_per_wave, std::memory_order_relaxed);
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
    {
        uint32_t idx[DFC_MAX_BATCH], m = 0;
        for (uint32_t k = 0; k < count; ++k)
            if (items[k].info->n && items[k].info->layout == DFC_LAYOUT_ANS) idx[m++] = k;
        if (m) {
            dfc_status s = dfc::ans_launch(items, idx, m, status_dev, st);
            if (s != DFC_OK) return s;
        }
    }
    // one launch per (chunk size, layout) present in the batch
    for (int pad = 0; pad < 2; ++pad) {
        const uint32_t layout = pad ? DFC_LAYOUT_PADDED : DFC_LAYOUT_FLAT;
        for (int c : sizes) {
            uint32_t idx[DFC_MAX_BATCH], m = 0;
            for (uint32_t k = 0; k < count; ++k) {
                const dfc_info &in = *items[k].info;
                if (in.n && in.chunk_bytes == uint32_t(c) && in.layout == layout) idx[m++] = k;
            }
            if (!m) continue;
            dfc_status s = DFC_OK;
            switch (c * 2 + pad) {
                case 8: s = launch_group<4, false>(items, idx, m, status_dev, st); break;
                case 9: s = launch_group<4, true>(items, idx, m, status_dev, st); break;
                case 16: s = launch_group<8, false>(items, idx, m, status_dev, st); break;
                case 17: s = launch_group<8, true>(items, idx, m, status_dev, st); break;
                case 32: s = launch_group<16, false>(items, idx, m, status_dev, st); break;
                case 33: s = launch_group<16, true>(items, idx, m, status_dev, st); break;
                case 64: s = launch_group<32, false>(items, idx, m, status_dev, st); break;
                default: s = launch_group<32, true>(items, idx, m, status_dev, st); break;
            }
            if (s != DFC_OK) return s;
        }
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
