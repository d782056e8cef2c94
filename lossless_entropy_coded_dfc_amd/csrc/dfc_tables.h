// dfc_tables.h - decode tables derived on the GPU, in LDS, by every
// workgroup that decodes a container (internal to libdfc).
//
// DFloat11 blog ("70% Size, 100% Accuracy ... (DFloat11)"), section 03
// item 1: compact hierarchical lookup tables held in on-chip memory find the
// code boundaries.  They are a function of the code alone (the 256 code
// lengths of a canonical prefix code, or the 256 rANS frequencies), so a
// container carries only the code and each workgroup builds the tables it
// decodes with in its own LDS before its first block.  No table format ever
// leaves the library.
//
// Huffman layouts, k-bit first level (k = lut_bits, 8..12), LDS image of
// tables_bytes(k) = 14 * 2^k + 640 bytes:
//   step[2^k]  u32  every whole code inside the k-bit window w (its first bit
//                   is the next stream bit): (codes << 16) - their bits, or
//                   kStepEscape when the first code is longer than k bits;
//   wsym[2^k]  u32x2  x: the first <= 4 of those codes' exponents, rotated
//                   right by one bit, in bytes 0..3 (zero past them);
//                   y: (min(codes, 4) << 16) - their bits, or kStepEscape;
//   mask[2^k]  u16  bit j set when a code ends j + 1 bits into the window;
//   limit[32], first[32], base[32]  u32, index = code length 1..24 (other
//                   entries 0): canonical decoding of codes longer than k:
//                   the length is the smallest l with w24 < limit[l]
//                   (w24 = next 24 bits), the symbol order[base[l] + (w24 >>
//                   (24 - l)) - first[l]];
//   order[256] u8   used symbols by (length, symbol), zero after them.
// rANS layout: the slot table, u32 per slot of 2^12: rotated exponent |
// (f - 1) << 8 | (slot - cum) << 20, where slot - cum is the slot's place
// inside its symbol's range.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dfc_format.h"

namespace {

// LDS bytes derive_tables needs beside the tables: per-group length counts
// (4 x 32 u32), per-symbol ranks and lengths (2 x 256 u8), and the
// single-code table of the k-bit windows (2^k u32).
__host__ __device__ constexpr uint32_t derive_scratch_bytes(uint32_t k) { return 512u + 512u + (4u << k); }

// Slot of window j in the single-code table.  The first-level pass reads
// entry (w << o) mod 2^k for consecutive w in a wavefront's lanes, 2^o
// entries apart; XOR-ing the bank bits with the entry's 64-entry row puts
// those reads in different LDS banks (or on one address) for every o.
__device__ __forceinline__ uint32_t t1_slot(uint32_t j) { return j ^ ((j >> 6) & 63u); }

// LDS bytes derive_slot_table needs beside the slot table: cum[256] u32.
constexpr uint32_t kSlotScratchBytes = 1024u;

__device__ __forceinline__ uint32_t rotr8_1(uint32_t e) { return ((e >> 1) | (e << 7)) & 0xFFu; }

// Inclusive prefix sum across the wavefront (DPP row shifts, then row
// broadcasts 15 and 31).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xf, 0xf, false));
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xf, 0xf, false));
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xf, 0xf, false));
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xf, 0xf, false));
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x142, 0xa, 0xf, false));
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x143, 0xc, 0xf, false));
    return x;
}

// Builds the Huffman decode tables for the code whose 256 lengths are at
// `lengths` (global memory) into `tab` (LDS, tables_bytes(k) bytes) using
// `scratch` (LDS, derive_scratch_bytes(k) bytes, 4-byte aligned, disjoint
// from tab).  The code must be complete (Kraft sum 1) with lengths <= 24,
// which the host checks before any launch.  Every thread of the workgroup
// must call it (blockDim.x a multiple of 64); it ends with a barrier.
__device__ void derive_tables(uint8_t *tab, uint8_t *scratch, const uint8_t *lengths, uint32_t k) {
    const uint32_t tid = threadIdx.x, nt = blockDim.x;
    const uint32_t lane = tid % 64u, wave = tid / 64u, waves = nt / 64u;
    uint32_t *grp = reinterpret_cast<uint32_t *>(scratch);  // [4][32]: group g, length l
    uint8_t *rank = scratch + 512;                          // [256]
    uint8_t *lens = scratch + 768;                          // [256]
    uint32_t *t1 = reinterpret_cast<uint32_t *>(scratch + 1024);
    uint32_t *limit = reinterpret_cast<uint32_t *>(tab + (14u << k));
    uint32_t *first = limit + 32, *base = limit + 64;
    uint8_t *order = tab + (14u << k) + 384;
    uint32_t *step = reinterpret_cast<uint32_t *>(tab);
    uint2 *wsym = reinterpret_cast<uint2 *>(tab + (4u << k));
    uint16_t *mask = reinterpret_cast<uint16_t *>(tab + (12u << k));

    // 1. Per group of 64 symbols: the symbols of every length, and each
    //    symbol's rank among the group's symbols of its length.
    for (uint32_t g = wave; g < 4u; g += waves) {
        const uint32_t s = 64u * g + lane;
        const uint32_t l = lengths[s];
        uint32_t r = 0, mine = 0;
        for (uint32_t L = 1; L <= dfc::kMaxLen; ++L) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(l == L);
            if (l == L) r = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
            if (lane == L) mine = uint32_t(__builtin_popcountll(m));
        }
        if (lane < 32u) grp[32u * g + lane] = mine;
        rank[s] = uint8_t(r);
        lens[s] = uint8_t(l);
    }
    __syncthreads();
    // 2. Canonical tables (wavefront 0, lane = length): count[l] summed over
    //    the groups; base = exclusive prefix of the counts; with u = count <<
    //    (24 - l), limit[l] = inclusive prefix of u (the left-justified end of
    //    the codes of length <= l) and first[l] = (exclusive prefix of u) >>
    //    (24 - l) (the first code of length l), which is the canonical
    //    recurrence first[l] = (first[l - 1] + count[l - 1]) << 1 summed out.
    if (wave == 0) {
        const bool len_ok = lane >= 1u && lane <= dfc::kMaxLen;
        uint32_t c = 0;
        if (len_ok)
            for (uint32_t g = 0; g < 4u; ++g) c += grp[32u * g + lane];
        const uint32_t cin = wave_inclusive_scan(c);
        const uint32_t u = len_ok ? c << (dfc::kMaxLen - lane) : 0u;
        const uint32_t uin = wave_inclusive_scan(u);
        if (lane < 32u) {
            limit[lane] = len_ok ? uin : 0u;
            first[lane] = len_ok ? (uin - u) >> (dfc::kMaxLen - lane) : 0u;
            base[lane] = len_ok ? cin - c : 0u;
        }
        // the number of used symbols, for the zero tail of order[]
        const uint32_t used = __builtin_amdgcn_readlane(cin, 63);
        if (lane == 0) grp[0] = used;  // (group 0 has no symbols of length 0)
    }
    __syncthreads();
    // 3. order[]: symbol s of length l goes to base[l] + (symbols of length
    //    l in the groups before its own) + its rank in its group.
    {
        const uint32_t used = grp[0];
        for (uint32_t s = tid; s < 256u; s += nt) {
            const uint32_t l = lens[s];
            if (s >= used) order[s] = 0;
            if (l) {
                uint32_t at = base[l] + rank[s];
                for (uint32_t g = 1; g <= s / 64u; ++g) at += grp[32u * (g - 1u) + l];
                order[at] = uint8_t(s);
            }
        }
    }
    __syncthreads();
    // 4. The first code of every k-bit window (its low bits zero past the
    //    window): its exponent rotated right by one bit | length << 8, or 0
    //    when it is longer than k.  By the monotone limits, the length is
    //    1 + the number of l <= k with limit[l] <= w24.
    const uint32_t kmask = (1u << k) - 1u;
    for (uint32_t j = tid; j <= kmask; j += nt) {
        const uint32_t x = j << (dfc::kMaxLen - k);
        uint32_t l = 1;
#pragma unroll
        for (uint32_t i = 1; i <= 12u; ++i) l += (i <= k && x >= limit[i]) ? 1u : 0u;
        uint32_t v = 0;
        if (l <= k) v = rotr8_1(order[base[l] + (x >> (dfc::kMaxLen - l)) - first[l]]) | (l << 8);
        t1[t1_slot(j)] = v;
    }
    __syncthreads();
    // 5. First-level entries: the codes of window w decoded one after
    //    another from its first bit through the single-code table; a code
    //    read from a shifted window (zeros past its end) is the true code
    //    whenever it fits in what is left of w.
    for (uint32_t w = tid; w <= kmask; w += nt) {
        uint32_t o = 0, n = 0, o4 = 0, syms = 0, m = 0;
        for (uint32_t it = 0; it < k; ++it) {
            const uint32_t e = t1[t1_slot((w << o) & kmask)];
            const uint32_t l = e >> 8;
            if (l == 0u || o + l > k) break;
            const bool first4 = n < 4u;
            syms |= first4 ? (e & 0xFFu) << (8u * n) : 0u;
            o += l;
            o4 = first4 ? o : o4;
            m |= 1u << (o - 1u);
            ++n;
        }
        step[w] = n ? (n << 16) - o : dfc::kStepEscape;
        wsym[w] = make_uint2(syms, n ? ((n < 4u ? n : 4u) << 16) - o4 : dfc::kStepEscape);
        mask[w] = uint16_t(m);
    }
    __syncthreads();
}

// Builds the rANS slot table (2^12 u32) for the frequencies at `freqs`
// (global memory, u16[256], summing to 2^12) into `table` (LDS) using
// `scratch` (LDS, kSlotScratchBytes, 4-byte aligned).  Every thread of the
// workgroup must call it (blockDim.x a multiple of 64); it ends with a
// barrier.
__device__ void derive_slot_table(uint32_t *table, uint8_t *scratch, const uint16_t *freqs) {
    const uint32_t tid = threadIdx.x, nt = blockDim.x;
    uint32_t *cum = reinterpret_cast<uint32_t *>(scratch);
    if (tid < 64u) {
        // lane i: symbols 4i .. 4i + 3
        uint32_t f[4], t = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[q] = freqs[4u * tid + q];
            t += f[q];
        }
        uint32_t c = wave_inclusive_scan(t) - t;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cum[4u * tid + q] = c;
            c += f[q];
        }
    }
    __syncthreads();
    // the slot's symbol: the largest s with cum[s] <= slot (that symbol's
    // range holds the slot, so its frequency is not zero)
    for (uint32_t j = tid; j < dfc::kAnsSlots; j += nt) {
        uint32_t s = 0;
#pragma unroll
        for (uint32_t d = 128; d; d >>= 1) s += cum[s + d] <= j ? d : 0u;
        const uint32_t f = freqs[s];
        table[j] = rotr8_1(s) | ((f - 1u) << 8) | ((j - cum[s]) << 20);
    }
    __syncthreads();
}

}  // namespace
