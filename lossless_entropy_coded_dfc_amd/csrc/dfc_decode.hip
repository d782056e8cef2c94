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
//           bytes into bf16 with coalesced 16-byte stores.
//
// Work decomposition: one lane per chunk (C bytes of code stream), one
// wavefront (64 lanes) per block of 64 chunks.  Workgroups are persistent:
// the grid is sized to the resident capacity of the GPU, each workgroup owns
// a contiguous run of blocks of one matrix, and its wavefronts take those
// blocks in turn while prefetching the next block's stream words, offsets
// and raw bytes.  All decoding is integer work on bit patterns.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "dfc.h"
#include "dfc_format.h"

namespace {

constexpr int kWave = 64;
// Accumulator = (codes << 16) + (kBias + shift), shift = bits from the
// current position to the end of the current 32-bit word pair's first word.
// kBias keeps the low half from borrowing and is a multiple of 32, so the
// low 5 bits of the accumulator are the funnel-shift amount.
constexpr uint32_t kBias = 0x8000u;
constexpr uint32_t kEscape = dfc::kStepEscape;
constexpr int kMaxWaves = 16;

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
    uint32_t blocks_per_wg;
    uint32_t tables_bytes;     // multiple of 16
    uint32_t lut_bits;
    uint32_t pad;
};

struct BatchArgs {
    ItemArgs item[DFC_MAX_BATCH];
    uint32_t count;
    uint32_t stage_bytes;  // LDS exponent staging per wavefront (multiple of 16)
    uint32_t *status;
};

struct Tables {
    const uint32_t *step;  // every whole code in the window (counting pass)
    const uint2 *wsym;     // x: rotated exponents of the first <= 4 codes, y: their step
    const uint16_t *mask;
    const uint32_t *limit, *first, *base;
    const uint8_t *order;
    uint32_t kshift;  // 32 - k
    uint32_t kb;
};

__device__ __forceinline__ uint32_t lo16(uint32_t a) { return a & 0xFFFFu; }

// Codes longer than the first-level window: the smallest length l with
// window < limit[l] (left-justified 24-bit comparison), then the symbol by
// canonical rank.  Returns the length; sym receives the rotated exponent.
__device__ __forceinline__ uint32_t long_code(uint32_t w24, const Tables &t, uint32_t &sym) {
    uint32_t l = t.kb + 1;
    while (l < 24u && w24 >= t.limit[l]) ++l;
    const uint32_t e = t.order[t.base[l] + (w24 >> (24u - l)) - t.first[l]];
    sym = ((e >> 1) | (e << 7)) & 0xFFu;
    return l;
}

// Per-lane view of one chunk: its words plus two lookahead words, the start
// offset of its first code and the end of its last code (chunk-relative
// bits), and the block's output range.
template <int C>
struct Chunk {
    static constexpr int NW = C / 4;
    uint32_t w[NW + 2];
    uint32_t o0, o1;  // the two offset-array words holding this chunk's field and the next
    uint32_t meta;    // lane 0: out[b], lane 1: out[b + 1]
};

template <int C>
__device__ __forceinline__ void load_chunk(const ItemArgs &a, uint32_t b, uint32_t lane, Chunk<C> &ck) {
    const uint64_t chunk = uint64_t(b) * kWave + lane;
    const uint32_t *p = a.words + chunk * (C / 4);
    if constexpr (C == 4) {
        ck.w[0] = p[0];
        ck.w[1] = p[1];
        ck.w[2] = p[2];
    } else if constexpr (C == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        const uint2 u = *reinterpret_cast<const uint2 *>(p + 2);
        ck.w[0] = v.x;
        ck.w[1] = v.y;
        ck.w[2] = u.x;
        ck.w[3] = u.y;
    } else {
#pragma unroll
        for (int q = 0; q < C / 16; ++q) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p + 4 * q);
            ck.w[4 * q + 0] = v.x;
            ck.w[4 * q + 1] = v.y;
            ck.w[4 * q + 2] = v.z;
            ck.w[4 * q + 3] = v.w;
        }
        const uint2 u = *reinterpret_cast<const uint2 *>(p + C / 4);
        ck.w[C / 4] = u.x;
        ck.w[C / 4 + 1] = u.y;
    }
    // Only loads here: combining the words right away would make the
    // compiler wait for every load in flight, prefetches included.
    const uint32_t *o = a.offw + ((5ull * chunk) >> 5);
    ck.o0 = o[0];
    ck.o1 = o[1];
    ck.meta = a.blockout[b + min(lane, 1u)];
}

// 32 stream bits starting at chunk-relative bit pos, 0 <= pos <= 32 (NW + 1).
template <int NW>
__device__ __forceinline__ uint32_t window_at(const uint32_t (&w)[NW + 2], uint32_t pos) {
    const uint32_t j = (pos + 31) >> 5;  // pos in (32 (j - 1), 32 j]
    uint32_t hi = 0, lo = w[0];
#pragma unroll
    for (int q = 1; q <= NW + 1; ++q) {
        if (j == uint32_t(q)) {
            hi = w[q - 1];
            lo = w[q];
        }
    }
    return __builtin_amdgcn_alignbit(hi, lo, 32u * j - pos);
}

// Phase one: number of codes that start in [start, end) (chunk-relative).
// The k-loop walks the chunk one word at a time so that every window is a
// funnel shift of two registers: a code starting at pos in (32k, 32k + 32]
// lies inside words k and k + 1.  Each lookup adds step = (codes << 16) -
// bits for every whole code inside the k-bit window; the last lookup may
// count codes that start at or after `end`, which are removed with the
// boundary mask of the window that starts at `end`.
template <int C>
__device__ __forceinline__ uint32_t count_codes(const Chunk<C> &ck, int start, int end, const Tables &t) {
    constexpr int NW = C / 4;
    uint32_t acc = kBias - uint32_t(start);
#pragma unroll
    for (int k = -1; k < NW; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        // stay while shift >= 0 (pos <= 32 (k + 1)) and pos < end
        const uint16_t g = uint16_t(kBias + uint32_t(max(0, 32 * (k + 1) - end + 1)));
        for (;;) {
            while (uint16_t(acc) >= g) {
                const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
                acc += t.step[win >> t.kshift];
            }
            if (lo16(acc) >= kBias - 2048u) break;
            // escape: the code at pos is longer than the window
            acc += 0x1000u;
            uint32_t sym;
            const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
            acc += 0x10000u - long_code(win >> 8, t, sym);
        }
        acc += 32u;
    }
    uint32_t cnt = acc >> 16;
    const int pos = 32 * (NW + 1) - int(lo16(acc)) + int(kBias);
    if (pos > end) {
        const uint32_t we = window_at<NW>(ck.w, uint32_t(end));
        cnt -= __popc(uint32_t(t.mask[we >> t.kshift]) & ((1u << (pos - end)) - 1u));
    }
    return cnt;
}

// Stores the 4 bytes of v at p, one naturally aligned byte store each.  On
// gfx950 a wide LDS store to an address that is not a multiple of its width
// is carried out one lane at a time; byte stores never are.
__device__ __forceinline__ void store_4_bytes(uint8_t *p, uint32_t v) {
    p[0] = uint8_t(v);
    p[1] = uint8_t(v >> 8);
    p[2] = uint8_t(v >> 16);
    p[3] = uint8_t(v >> 24);
}

// Phase two: decode the chunk again and write its cnt (rotated) exponents to
// LDS, at most four codes per lookup.  While four or more codes remain, all
// four symbol bytes of a lookup are stored: bytes past the lookup's own codes
// fall on positions this lane overwrites with its next lookup.  The last
// < 4 codes are written exactly.
template <int C>
__device__ __forceinline__ void write_codes(const Chunk<C> &ck, int start, uint32_t cnt, uint8_t *out,
                                            const Tables &t) {
    constexpr int NW = C / 4;
    uint32_t acc = kBias - uint32_t(start);
    const uint32_t lim = cnt >= 4u ? (cnt - 3u) << 16 : 0u;  // acc < lim <=> done <= cnt - 4
#pragma unroll
    for (int k = -1; k < NW; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        for (;;) {
            while (uint16_t(acc) >= uint16_t(kBias) && acc < lim) {
                const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
                const uint2 e = t.wsym[win >> t.kshift];
                store_4_bytes(out + (acc >> 16), e.x);
                acc += e.y;
            }
            if (lo16(acc) >= kBias - 2048u) break;
            acc += 0x1000u;
            uint32_t sym;
            const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
            const uint32_t l = long_code(win >> 8, t, sym);
            out[acc >> 16] = uint8_t(sym);
            acc += 0x10000u - l;
        }
        acc += 32u;
    }
    uint32_t done = acc >> 16;
    uint32_t pos = uint32_t(32 * (NW + 1)) - lo16(acc) + kBias;
    while (done < cnt && pos < uint32_t(32 * (NW + 1))) {
        const uint32_t win = window_at<NW>(ck.w, pos);
        const uint2 e = t.wsym[win >> t.kshift];
        if (e.y == kEscape) {
            uint32_t sym;
            pos += long_code(win >> 8, t, sym);
            out[done] = uint8_t(sym);
            done += 1;
        } else {
            const uint32_t r = min((e.y >> 16) + 1u, cnt - done);
            out[done] = uint8_t(e.x);
            if (r > 1u) out[done + 1] = uint8_t(e.x >> 8);
            if (r > 2u) out[done + 2] = uint8_t(e.x >> 16);
            done += r;
            pos += 0x10000u - (e.y & 0xFFFFu);
        }
    }
}

// Inclusive prefix sum across the wavefront (DPP row shifts, then row
// broadcasts 15 and 31).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xf, 0xf, false));  // row_shr:1
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xf, 0xf, false));  // row_shr:2
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xf, 0xf, false));  // row_shr:4
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xf, 0xf, false));  // row_shr:8
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x142, 0xa, 0xf, false));  // row_bcast:15
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}

// 16 bf16 values from 16 staged (rotated) exponents and 16 raw bytes.  Per
// pair of values, x1 = [raw_a, exp_a, raw_b, exp_b] and x2 = [exp_a, raw_a,
// exp_b, raw_b] (bytes, low first); each output byte keeps bits 6..0 of x1
// and bit 7 of x2.
__device__ __forceinline__ void assemble16(const uint4 &E, const uint4 &R, uint32_t o[8]) {
    const uint32_t e[4] = {E.x, E.y, E.z, E.w};
    const uint32_t r[4] = {R.x, R.y, R.z, R.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t a1 = __builtin_amdgcn_perm(e[q], r[q], 0x05010400u);
        const uint32_t a2 = __builtin_amdgcn_perm(e[q], r[q], 0x01050004u);
        const uint32_t b1 = __builtin_amdgcn_perm(e[q], r[q], 0x07030602u);
        const uint32_t b2 = __builtin_amdgcn_perm(e[q], r[q], 0x03070206u);
        o[2 * q] = (a1 & 0x7F7F7F7Fu) | (a2 & 0x80808080u);
        o[2 * q + 1] = (b1 & 0x7F7F7F7Fu) | (b2 & 0x80808080u);
    }
}

__device__ __forceinline__ void store_group(const ItemArgs &a, uint32_t g, uint32_t s_out, uint32_t e_out,
                                            const uint32_t o[8]) {
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

// Makes the compiler wait for the loads into v now.  vmcnt also counts
// stores on this chip, and the compiler cannot count the stores of the
// divergent store paths below, so a register first used after a store would
// make it wait for every store in flight to reach memory.
template <typename T>
__device__ __forceinline__ void wait_for(const T &v) {
    static_assert(sizeof(T) % 4 == 0, "whole dwords only");
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 4; ++i) asm volatile("" ::"v"(w[i]));
}

// Raw-byte groups prefetched into registers per lane before decoding.
template <int C>
struct Prefetch {
    static constexpr int N = C >= 32 ? 6 : C / 4;
};

template <int C>
__device__ __forceinline__ void decode_block(const ItemArgs &a, uint32_t b, uint32_t lane, const Chunk<C> &ck,
                                             uint8_t *stage, const Tables &t, uint32_t *status,
                                             const uint4 (&R)[Prefetch<C>::N], uint32_t s_out, uint32_t e_out,
                                             const Chunk<C> &nxt, bool more) {
    constexpr int PF = Prefetch<C>::N;
    const uint64_t chunk = uint64_t(b) * kWave + lane;
    const uint32_t offpair = __builtin_amdgcn_alignbit(ck.o1, ck.o0, uint32_t((5ull * chunk) & 31));
    const int start = int(offpair & 31u);
    const int next_off = int((offpair >> 5) & 31u);
    const int64_t rem = int64_t(a.total_bits) - int64_t(chunk * (8ull * C));
    const int end = int(min(int64_t(8 * C + next_off), max(rem, int64_t(-1))));

    const uint32_t cnt = start < end ? count_codes<C>(ck, start, end, t) : 0u;
    const uint32_t incl = wave_inclusive_scan(cnt);
    const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
    // A chunk of 8C bits holds at most 8C code starts; anything else (or a
    // total that disagrees with the block offsets) means a corrupt stream.
    const bool bad = (total != e_out - s_out) | (__builtin_amdgcn_ballot_w64(cnt > 8u * C) != 0);
    const uint32_t lead = s_out & 15u;
    if (!bad && cnt) write_codes<C>(ck, start, cnt, stage + lead + (incl - cnt), t);
    // Everything prefetched must be in registers before the first store, on
    // every path to the next block.
    wait_for(R);
    wait_for(nxt);
    if (bad) {
        if (lane == 0 && status) atomicOr(status, 1u);
        return;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const uint32_t g0 = s_out >> 4, g1 = (e_out + 15u) >> 4;
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        const uint32_t g = g0 + lane + uint32_t(kWave * j);
        if (g < g1) {
            const uint4 E = *reinterpret_cast<const uint4 *>(stage + 16u * (g - g0));
            uint32_t o[8];
            assemble16(E, R[j], o);
            store_group(a, g, s_out, e_out, o);
        }
    }
    for (uint32_t g = g0 + lane + uint32_t(kWave * PF); g < g1; g += kWave) {
        const uint4 E = *reinterpret_cast<const uint4 *>(stage + 16u * (g - g0));
        const uint4 Rg = *reinterpret_cast<const uint4 *>(a.raw + 16ull * g);
        uint32_t o[8];
        assemble16(E, Rg, o);
        store_group(a, g, s_out, e_out, o);
    }
    // The next block reuses this wavefront's staging area.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int C>
__global__ __launch_bounds__(1024) void dfc_decode_kernel(const BatchArgs args) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int PF = Prefetch<C>::N;
    const uint32_t wg = blockIdx.x;
    uint32_t it = 0;
    for (uint32_t k = 1; k < args.count; ++k)
        if (wg >= args.item[k].wg_begin) it = k;
    const ItemArgs &a = args.item[it];

    // Stage the decode tables in LDS (16 bytes per thread per step).
    for (uint32_t o = threadIdx.x * 16u; o < a.tables_bytes; o += blockDim.x * 16u)
        *reinterpret_cast<uint4 *>(lds + o) = *reinterpret_cast<const uint4 *>(a.tables + o);
    __syncthreads();

    Tables t;
    t.kb = a.lut_bits;
    t.kshift = 32u - t.kb;
    t.step = reinterpret_cast<const uint32_t *>(lds);
    t.wsym = reinterpret_cast<const uint2 *>(lds + (4u << t.kb));
    t.mask = reinterpret_cast<const uint16_t *>(lds + (12u << t.kb));
    t.limit = reinterpret_cast<const uint32_t *>(lds + (14u << t.kb));
    t.first = t.limit + 32;
    t.base = t.limit + 64;
    t.order = lds + (14u << t.kb) + 384;

    const uint32_t waves = blockDim.x / kWave;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    uint8_t *stage = lds + a.tables_bytes + wave * args.stage_bytes;
    const uint32_t lo_b = (wg - a.wg_begin) * a.blocks_per_wg;
    const uint32_t hi_b = min(lo_b + a.blocks_per_wg, a.n_blocks);

    uint32_t b = lo_b + wave;
    if (b >= hi_b) return;
    Chunk<C> cur;
    load_chunk<C>(a, b, lane, cur);
    // Resident on entry, as it is on every later iteration (see wait_for).
    wait_for(cur);
    for (;;) {
        const uint32_t s_out = __builtin_amdgcn_readlane(cur.meta, 0);
        const uint32_t e_out = __builtin_amdgcn_readlane(cur.meta, 1);
        // raw bytes of this block's first PF groups per lane
        uint4 R[PF];
        const uint32_t g0 = s_out >> 4, g1 = (e_out + 15u) >> 4;
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const uint32_t g = g0 + lane + uint32_t(kWave * j);
            R[j] = g < g1 ? *reinterpret_cast<const uint4 *>(a.raw + 16ull * g) : make_uint4(0, 0, 0, 0);
        }
        // next block's stream words, offsets and output range
        const uint32_t bn = b + waves;
        const bool more = bn < hi_b;
        Chunk<C> nxt{};
        if (more) load_chunk<C>(a, bn, lane, nxt);
        decode_block<C>(a, b, lane, cur, stage, t, args.status, R, s_out, e_out, nxt, more);
        if (!more) break;
        cur = nxt;
        b = bn;
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

constexpr uint32_t kLdsBytes = 160u * 1024u;

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

template <int C>
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
    // staging: lead (< 16) + elements + one 16-byte group of slack, rounded to 16
    const uint32_t stage = (max_block + 32u + 15u) & ~15u;
    // waves per workgroup: the most resident wavefronts per CU under the LDS budget
    uint32_t waves = g_launch.waves;
    if (!waves) {
        uint32_t best = 0;
        for (uint32_t w = 4; w <= kMaxWaves; ++w) {
            const uint32_t per = max_tables + w * stage;
            if (per > kLdsBytes) break;
            const uint32_t resident = std::min<uint32_t>(kLdsBytes / per, 32 / w) * w;
            if (resident > best) {
                best = resident;
                waves = w;
            }
        }
    }
    if (!waves) waves = 1;
    while (waves > 1 && max_tables + waves * stage > kLdsBytes) --waves;
    const uint32_t lds = max_tables + waves * stage;
    if (lds > kLdsBytes) return DFC_EUNSUPPORTED;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(&dfc_decode_kernel<C>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsBytes)) != hipSuccess)
            return DFC_EHIP;
        attr_set = true;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&dfc_decode_kernel<C>),
                                                     int(waves * kWave), size_t(lds)) != hipSuccess ||
        per_cu <= 0)
        per_cu = int(std::max(1u, kLdsBytes / lds));
    uint64_t slots = uint64_t(per_cu) * uint64_t(device_cu_count());
    if (g_launch.blocks_per_wave) {
        // fixed work per workgroup instead of filling the machine exactly
        uint64_t total = 0;
        for (uint64_t nb : blocks) total += dfc::ceil_div(nb, uint64_t(waves) * g_launch.blocks_per_wave);
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
    if (in.max_block_elems > 64u * dfc::ceil_div(8ull * C, in.min_len)) return DFC_EINVAL;
    return DFC_OK;
}

}  // namespace

extern "C" {

dfc_status dfc_set_launch(uint32_t waves_per_group, uint32_t blocks_per_wave) {
    if (waves_per_group > kMaxWaves) return DFC_EINVAL;
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
