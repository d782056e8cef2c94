// dfc_decode_core.h - device-side building blocks shared by the gfx950
// kernels of libdfc (the flat decoder and the fused decode + matrix product).
//
// DFloat11 blog ("70% Size, 100% Accuracy ... (DFloat11)"), section 03:
// item 1, compact hierarchical lookup tables in on-chip memory (the k-bit
// first-level tables and the per-length canonical tables, staged in LDS);
// item 2, a two-phase decode (count the codes of every chunk, scan the counts
// into write positions across the wavefront, then decode again and write).
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <set>
#include <utility>

#include <cstdint>

#include "dfc.h"
#include "dfc_format.h"
#include "dfc_tables.h"

namespace {

constexpr int kWave = 64;
// Accumulator = (codes << 16) + (kBias + shift), shift = bits from the
// current position to the end of the current 32-bit word pair's first word.
// kBias keeps the low half from borrowing and is a multiple of 32, so the
// low 5 bits of the accumulator are the funnel-shift amount.
constexpr uint32_t kBias = 0x8000u;
constexpr uint32_t kEscape = dfc::kStepEscape;
constexpr int kMaxWaves = 16;
// What a kernel ORs into the caller's status word when a block fails its
// checks: the bit pattern of DFC_ECORRUPT (every writer ORs the same value).
constexpr uint32_t kStatusCorrupt = uint32_t(DFC_ECORRUPT);

// Raw buffer resources (base, 32-bit byte range) for every stream of an
// item: loads past the range return zero and stores past it are dropped, so
// lanes without work need no branch around their memory accesses.
constexpr uint32_t kBufferConfig = 0x00020000u;  // dword 3 of a raw buffer resource on gfx9-family chips
constexpr uint32_t kNowhere = 0xFFFFFFF0u;       // byte offset past every range the launcher accepts

using u32x2 = __attribute__((ext_vector_type(2))) uint32_t;
using u32x4 = __attribute__((ext_vector_type(4))) uint32_t;
// Read-only global memory through the constant address space: uniform
// indices load with scalar instructions.
typedef const uint32_t __attribute__((address_space(4))) *const_u32_ptr;

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

// After a word's whole-window lookups: lo16(acc) >= kBias - 2048 unless the
// code at the current position is longer than the window.  Written with a
// shift rather than lo16, so that the compiler can fold the loop test's own
// low-half mask into its comparison.
__device__ __forceinline__ bool no_escape(uint32_t acc) { return (acc << 16) >= ((kBias - 2048u) << 16); }

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

// Per-lane view of one chunk: its words plus two lookahead words, and the
// two offset-array words that hold its start offset and the next chunk's.
template <int C>
struct Chunk {
    static constexpr int NW = C / 4;
    uint32_t w[NW + 2];
    uint32_t o0, o1;
};

// Chunk `chunk` of a stream: its words through the buffer resource `words`,
// its offset-array words through `offw` (none for the padded layout, whose
// chunks start with a code).
template <int C, bool Offsets = true>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t words, __amdgpu_buffer_rsrc_t offw, uint32_t chunk,
                                           Chunk<C> &ck) {
    const uint32_t at = chunk * C;
    if constexpr (C == 4) {
        ck.w[0] = __builtin_amdgcn_raw_buffer_load_b32(words, at, 0, 0);
        ck.w[1] = __builtin_amdgcn_raw_buffer_load_b32(words, at + 4u, 0, 0);
        ck.w[2] = __builtin_amdgcn_raw_buffer_load_b32(words, at + 8u, 0, 0);
    } else if constexpr (C == 8) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(words, at, 0, 0);
        const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(words, at + 8u, 0, 0);
        ck.w[0] = v.x;
        ck.w[1] = v.y;
        ck.w[2] = u.x;
        ck.w[3] = u.y;
    } else {
#pragma unroll
        for (int q = 0; q < C / 16; ++q) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(words, at + 16u * q, 0, 0);
            ck.w[4 * q + 0] = v.x;
            ck.w[4 * q + 1] = v.y;
            ck.w[4 * q + 2] = v.z;
            ck.w[4 * q + 3] = v.w;
        }
        const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(words, at + C, 0, 0);
        ck.w[C / 4] = u.x;
        ck.w[C / 4 + 1] = u.y;
    }
    // Only loads here: combining the words right away would make the
    // compiler wait for every load in flight, prefetches included.
    if constexpr (Offsets) {
        // Field `chunk` starts at bit 5 chunk of the offset array.
        const uint32_t word = (chunk >> 5) * 5u + (((chunk & 31u) * 5u) >> 5);
        ck.o0 = __builtin_amdgcn_raw_buffer_load_b32(offw, 4u * word, 0, 0);
        ck.o1 = __builtin_amdgcn_raw_buffer_load_b32(offw, 4u * word + 4u, 0, 0);
    } else {
        ck.o0 = ck.o1 = 0;
    }
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

// window_at for a chunk's end bit, which lies past 32 (NW - 1) in every
// chunk but a stream's last few: two candidate word pairs there, the full
// selection only for the others.
template <int NW>
__device__ __forceinline__ uint32_t window_at_end(const uint32_t (&w)[NW + 2], uint32_t pos) {
    if (pos > 32u * (NW - 1)) {
        const bool second = pos > 32u * NW;
        const uint32_t hi = second ? w[NW] : w[NW - 1];
        const uint32_t lo = second ? w[NW + 1] : w[NW];
        return __builtin_amdgcn_alignbit(hi, lo, (second ? 32u * (NW + 1) : 32u * NW) - pos);
    }
    return window_at<NW>(w, pos);
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
    // the lookups of word k go on while the low half of acc is at least
    // max(kBias, g0 + 32 (k + 1)): shift >= 0 and pos < end
    const int g0 = int(kBias) + 1 - end;
#pragma unroll
    for (int k = -1; k < NW; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        // stay while shift >= 0 (pos <= 32 (k + 1)) and pos < end
        const uint16_t g = uint16_t(max(int(kBias), g0 + 32 * (k + 1)));
        for (;;) {
            while (uint16_t(acc) >= g) {
                const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
                acc += t.step[win >> t.kshift];
            }
            if (no_escape(acc)) break;
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
        const uint32_t we = window_at_end<NW>(ck.w, uint32_t(end));
        cnt -= __popc(uint32_t(t.mask[we >> t.kshift]) & ((1u << (pos - end)) - 1u));
    }
    return cnt;
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

// LDS address (byte offset in the workgroup's LDS) of a pointer into it.
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
__device__ __forceinline__ uint32_t lds_address(const uint8_t *p) {
    return uint32_t(reinterpret_cast<size_t>((const lds_u8_t *)p));
}

// ORs the 4 bytes of v into the zeroed LDS staging bytes at LDS address
// [q, q + 4): two aligned dword ORs.  OR is what lets lanes overlap: a byte
// is only ever ORed with zero or with its own final value.  q is an LDS
// address, not an offset from a pointer, so that the address needs no add.
__device__ __forceinline__ void or_4_bytes(uint32_t q, uint32_t v) {
    const uint64_t x = uint64_t(v) << (8u * (q & 3u));
    lds_u32_t *d = reinterpret_cast<lds_u32_t *>(size_t(q & ~3u));
    __hip_atomic_fetch_or(d, uint32_t(x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    __hip_atomic_fetch_or(d + 1, uint32_t(x >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// Phase two: decode the chunk again and OR its (rotated) exponents into the
// zeroed staging area, from LDS address q0 on, up to four codes per lookup.  A
// table entry holds zero bytes past its own codes, and codes decoded past
// the chunk's last one are the next chunk's first codes, identical to what
// the next lane writes there; so neither needs to be cut off.  Lookups stop
// at the chunk's end bit, which bounds the spill past the block's last
// exponent to three codes.  Returns the number of codes that start in
// [start, end), as count_codes does (callers that take their positions
// from stored counts check them with it; for the others it is dead code).
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

template <int C, typename Hook = NoHook>
__device__ __forceinline__ uint32_t write_codes(const Chunk<C> &ck, int start, int end, uint32_t q0,
                                                const Tables &t, const Hook &hook = Hook()) {
    constexpr int NW = C / 4;
    // the boundary mask at `end`, looked up first so that the stream words
    // need not outlive the loop
    const uint32_t end_mask = t.mask[window_at_end<NW>(ck.w, uint32_t(end)) >> t.kshift];
    uint32_t acc = kBias - uint32_t(start);
    const int g0 = int(kBias) + 1 - end;  // as in count_codes
#pragma unroll
    for (int k = -1; k < NW; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        // stay while shift >= 0 (pos <= 32 (k + 1)) and pos < end
        const uint16_t g = uint16_t(max(int(kBias), g0 + 32 * (k + 1)));
        for (;;) {
            while (uint16_t(acc) >= g) {
                const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
                const uint2 e = t.wsym[win >> t.kshift];
                or_4_bytes(q0 + (acc >> 16), e.x);
                acc += e.y;
            }
            if (no_escape(acc)) break;
            acc += 0x1000u;
            uint32_t sym;
            const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
            const uint32_t l = long_code(win >> 8, t, sym);
            or_4_bytes(q0 + (acc >> 16), sym);
            acc += 0x10000u - l;
        }
        acc += 32u;
        hook(k + 1);
    }
    uint32_t cnt = acc >> 16;
    const int pos = 32 * (NW + 1) - int(lo16(acc)) + int(kBias);
    if (pos > end) cnt -= __popc(end_mask & ((1u << (pos - end)) - 1u));
    return cnt;
}

// Padded layout, phase one: the number of codes, decoded from the chunk's
// first bit, that end at or before `end` (<= 8C).  Whole-window lookups run
// while the k-bit window lies inside [0, end), so every code they count is
// the chunk's own.  After them, either a long code has run past `end` (it is
// the unused tail of ones, read as a code longer than the tail, and is
// dropped), or the codes that still end by `end` are read off the boundary
// mask of the window at the current position.
template <int C>
__device__ __forceinline__ uint32_t count_codes_padded(const Chunk<C> &ck, int end, const Tables &t) {
    constexpr int NW = C / 4;
    const int stop = end - int(t.kb) + 1;  // whole-window lookups start before this bit
    uint32_t acc = kBias;
    const int g0 = int(kBias) + 1 - stop;  // as in count_codes, with stop for end
#pragma unroll
    for (int k = -1; k < NW; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        // stay while shift >= 0 (pos <= 32 (k + 1)) and pos < stop
        const uint16_t g = uint16_t(max(int(kBias), g0 + 32 * (k + 1)));
        for (;;) {
            while (uint16_t(acc) >= g) {
                const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
                acc += t.step[win >> t.kshift];
            }
            if (no_escape(acc)) break;
            acc += 0x1000u;
            uint32_t sym;
            const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
            acc += 0x10000u - long_code(win >> 8, t, sym);
        }
        acc += 32u;
    }
    uint32_t cnt = acc >> 16;
    const int pos = 32 * (NW + 1) - int(lo16(acc)) + int(kBias);
    if (pos > end) return cnt - 1u;
    if (pos < end) {
        const uint32_t we = window_at<NW>(ck.w, uint32_t(pos));
        cnt += __popc(uint32_t(t.mask[we >> t.kshift]) & ((1u << (end - pos)) - 1u));
    }
    return cnt;
}

// Padded layout, phase two: the chunk's cnt codes (from the counting pass)
// ORed into the staging area from LDS address q0 on.  Nothing past them may be
// written: what follows a chunk's last code is its tail of ones and the next
// chunk's bits, not the next chunk's first codes.  Whole-window lookups need
// no cut (their codes end by `end`); a long code is written only if it is
// one of the cnt; the last few codes go out with their entry cut to the
// codes still owed.
template <int C, typename Hook = NoHook>
__device__ __forceinline__ void write_codes_padded(const Chunk<C> &ck, int end, uint32_t cnt, uint32_t q0,
                                                   const Tables &t, const Hook &hook = Hook()) {
    constexpr int NW = C / 4;
    const int stop = end - int(t.kb) + 1;
    uint32_t acc = kBias;
    const int g0 = int(kBias) + 1 - stop;  // as in count_codes, with stop for end
#pragma unroll
    for (int k = -1; k < NW; ++k) {
        const uint32_t hi = k < 0 ? 0u : ck.w[k < 0 ? 0 : k];
        const uint32_t lo = ck.w[k + 1];
        const uint16_t g = uint16_t(max(int(kBias), g0 + 32 * (k + 1)));
        for (;;) {
            while (uint16_t(acc) >= g) {
                const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
                const uint2 e = t.wsym[win >> t.kshift];
                or_4_bytes(q0 + (acc >> 16), e.x);
                acc += e.y;
            }
            if (no_escape(acc)) break;
            acc += 0x1000u;
            uint32_t sym;
            const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, acc);
            const uint32_t l = long_code(win >> 8, t, sym);
            if ((acc >> 16) < cnt) or_4_bytes(q0 + (acc >> 16), sym);
            acc += 0x10000u - l;
        }
        acc += 32u;
        hook(k + 1);
    }
    // (done << 16) + kBias - pos, advanced by the symbol entries' steps.  The
    // codes owed end within k - 1 <= 11 bits, so three entries hold them.
    uint32_t a = (acc & 0xFFFF0000u) + (kBias - uint32_t(32 * (NW + 1) - int(lo16(acc)) + int(kBias)));
#pragma unroll
    for (int it = 0; it < 3; ++it) {
        if ((a >> 16) >= cnt) break;
        const uint32_t pos = kBias - lo16(a);
        const uint2 e = t.wsym[window_at<NW>(ck.w, pos) >> t.kshift];
        const uint32_t owed = cnt - (a >> 16);
        const uint32_t keep = owed >= 4u ? 0xFFFFFFFFu : (1u << (8u * owed)) - 1u;
        or_4_bytes(q0 + (a >> 16), e.x & keep);
        a += e.y;
    }
}

// 8 bf16 values from 8 staged (rotated) exponents and 8 raw bytes.  A
// staged byte holds exponent bits 0 | 7..1 (bit 7 = the exponent's lowest
// bit), a raw byte sign | mantissa: a value's low byte is bit 7 of the one
// and bits 6..0 of the other, its high byte the other way round.  Per 4
// values, two bit-field selects make the 4 low and the 4 high bytes and two
// byte permutes interleave them.
__device__ __forceinline__ u32x4 assemble8(const u32x2 &E, const u32x2 &R) {
    const uint32_t e[2] = {E.x, E.y};
    const uint32_t r[2] = {R.x, R.y};
    constexpr uint32_t kTop = 0x80808080u;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint32_t lo = (e[q] & kTop) | (r[q] & ~kTop);
        const uint32_t hi = (r[q] & kTop) | (e[q] & ~kTop);
        o[2 * q] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
        o[2 * q + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// The decode tables of a container into LDS at `lds`: copied from `tables`
// (what dfc_derive_tables wrote for the container, tables_bytes bytes, a
// multiple of 16) when there are any, else derived from the code lengths,
// with the LDS after the tables as scratch.  Every thread of the workgroup
// calls it; it ends with a barrier.
__device__ __forceinline__ void load_or_derive_tables(uint8_t *lds, const uint8_t *tables, uint32_t tables_bytes,
                                                      const uint8_t *lengths, uint32_t lut_bits) {
    if (tables) {
        // every load of a thread is issued before its LDS writes, so the
        // copy waits for one round trip to the cache, not one per 16 bytes
        // (four per thread cover the largest tables, 57,984 bytes at k = 12,
        // from 1,024 threads; smaller workgroups loop)
        const __amdgpu_buffer_rsrc_t tr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(tables), 0, int(tables_bytes), kBufferConfig);
        const uint32_t step = blockDim.x * 16u;
        for (uint32_t o = threadIdx.x * 16u; o < tables_bytes; o += 4u * step) {
            const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(tr, o, 0, 0);
            const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(tr, o + step, 0, 0);
            const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(tr, o + 2u * step, 0, 0);
            const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(tr, o + 3u * step, 0, 0);
            *reinterpret_cast<u32x4 *>(lds + o) = a;
            if (o + step < tables_bytes) *reinterpret_cast<u32x4 *>(lds + o + step) = b;
            if (o + 2u * step < tables_bytes) *reinterpret_cast<u32x4 *>(lds + o + 2u * step) = c;
            if (o + 3u * step < tables_bytes) *reinterpret_cast<u32x4 *>(lds + o + 3u * step) = d;
        }
        __syncthreads();
    } else {
        derive_tables(lds, lds + tables_bytes, lengths, lut_bits);
    }
}

// Pointers into the LDS image of derive_tables for a k-bit first level.
__device__ __forceinline__ Tables tables_view(uint8_t *lds, uint32_t lut_bits) {
    Tables t;
    t.kb = lut_bits;
    t.kshift = 32u - t.kb;
    t.step = reinterpret_cast<const uint32_t *>(lds);
    t.wsym = reinterpret_cast<const uint2 *>(lds + (4u << t.kb));
    t.mask = reinterpret_cast<const uint16_t *>(lds + (12u << t.kb));
    t.limit = reinterpret_cast<const uint32_t *>(lds + (14u << t.kb));
    t.first = t.limit + 32;
    t.base = t.limit + 64;
    t.order = lds + (14u << t.kb) + 384;
    return t;
}

// Chunk-relative first bit of a chunk's first code and end of its codes,
// from the offset-array words and the number of stream bits left from the
// chunk's first bit to the end of its stream (or item), clamped to at most
// 8C + 32 by the caller.
template <int C>
__device__ __forceinline__ void chunk_span(const Chunk<C> &ck, uint32_t chunk, int bits_left, int &start, int &end) {
    const uint32_t offpair = __builtin_amdgcn_alignbit(ck.o1, ck.o0, (5u * chunk) & 31u);
    start = int(offpair & 31u);
    const int next_off = int((offpair >> 5) & 31u);
    end = min(8 * C + next_off, max(bits_left, -1));
}

constexpr uint32_t kLdsBytes = 160u * 1024u;

// Raises a kernel's dynamic LDS limit to kLdsBytes on the current device,
// once per (kernel, device): the attribute is per device, and concurrent
// first calls from several host threads are serialized.
inline bool allow_full_lds(const void *kernel) {
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({kernel, dev})) return true;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsBytes)) != hipSuccess)
        return false;
    done.insert({kernel, dev});
    return true;
}

inline int device_cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return cus;
}

}  // namespace
