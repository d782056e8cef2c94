// dfc_encode_gpu.hip - gfx950 encoder: the same DFC1 containers as the host
// encoder, built from bf16 data already in device memory.
//
// DFloat11 blog ("70% Size, 100% Accuracy ... (DFloat11)"), section 02: an
// entropy code from the weights' own statistics; section 03 item 2: the
// per-chunk and per-block position variables the two-phase decoder needs.
// The pages compress offline on the host; this moves the O(n) work to the
// GPU:
//   1. exponent histogram (LDS bins per workgroup, then global atomics);
//   2. on the host: code lengths, canonical codes, total bits (the histogram
//      times the lengths), section layout and header;
//   3. code bits per segment of 4096 elements, an exclusive scan over the
//      segments, then every thread packs its 16 codes at its bit position
//      (interior words stored, the two words shared with neighbours ORed)
//      and writes the raw bytes; the element whose code covers a chunk's
//      first bit writes that chunk's 5-bit offset (the next code starts where
//      it ends) and, on block boundaries, the block's output offset.
// Containers in the interleaved rANS layout (an arithmetic-family code, the
// blog's section 02) take steps 1-2 with frequencies instead of code
// lengths, then one wavefront per block runs the block's encoder twice: a
// first pass counts the block's 16-bit words, an exclusive scan over the
// blocks gives every block's first word (its total is read back to place the
// sections), and a second pass writes each word at its place in decode
// order, then the final states; the raw bytes are written by a plain
// streaming kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <vector>

#include "dfc.h"
#include "dfc_format.h"
#include "dfc_host_internal.h"

namespace {

constexpr uint32_t kSegThreads = 256;
constexpr uint32_t kPerThread = 16;
constexpr uint32_t kSegElems = kSegThreads * kPerThread;  // 4096

__device__ __forceinline__ uint32_t exponent_of(uint32_t b) { return (b >> 7) & 0xFFu; }
__device__ __forceinline__ uint32_t raw_of(uint32_t b) { return ((b >> 8) & 0x80u) | (b & 0x7Fu); }

// Exponent histogram: 16-byte loads (eight values per thread and step) into
// eight LDS sub-histograms per wavefront, one per lane mod 8, spaced 257
// words apart so that the copies of a bin lie in different banks: the few
// frequent exponents of a weight matrix then collide in at most a few lanes
// per atomic.  The copies are summed into the global counts once per
// workgroup.
constexpr uint32_t kHistCopies = 32;  // 4 wavefronts x 8
constexpr uint32_t kHistStride = 257;

__global__ __launch_bounds__(256) void histogram_kernel(const uint16_t *src, uint64_t n, uint32_t *hist) {
    __shared__ uint32_t bins[kHistCopies * kHistStride];
    const uint32_t t = threadIdx.x;
    for (uint32_t i = t; i < kHistCopies * kHistStride; i += 256) bins[i] = 0;
    __syncthreads();
    uint32_t *mine = bins + ((t / 64u) * 8u + (t & 7u)) * kHistStride;
    const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
    const uint64_t gid = uint64_t(blockIdx.x) * blockDim.x + t;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
        const uint64_t n8 = n / 8;
        for (uint64_t i = gid; i < n8; i += stride) {
            const uint4 u = reinterpret_cast<const uint4 *>(src)[i];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                atomicAdd(&mine[exponent_of(w[q])], 1u);
                atomicAdd(&mine[exponent_of(w[q] >> 16)], 1u);
            }
        }
        for (uint64_t j = 8 * n8 + gid; j < n; j += stride) atomicAdd(&mine[exponent_of(src[j])], 1u);
    } else {
        for (uint64_t j = gid; j < n; j += stride) atomicAdd(&mine[exponent_of(src[j])], 1u);
    }
    __syncthreads();
    uint32_t v = 0;
    for (uint32_t k = 0; k < kHistCopies; ++k) v += bins[k * kHistStride + t];
    if (v) atomicAdd(&hist[t], v);
}

__global__ void fill_zero_u32(uint32_t *p, uint64_t words) {
    for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < words; i += uint64_t(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

struct Book {
    uint32_t code[256];
    uint8_t len[256];
};

// Loads this thread's 16 elements (zero past n): two 16-byte loads when all
// are in range and the source is 16-byte aligned.
__device__ __forceinline__ void load16(const uint16_t *src, uint64_t n, uint64_t j0, uint16_t (&b)[kPerThread]) {
    if (j0 + kPerThread <= n && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
        const uint4 u = *reinterpret_cast<const uint4 *>(src + j0);
        const uint4 v = *reinterpret_cast<const uint4 *>(src + j0 + 8);
        const uint32_t w[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t q = 0; q < kPerThread; ++q) b[q] = uint16_t(w[q >> 1] >> (16 * (q & 1)));
    } else {
#pragma unroll
        for (uint32_t q = 0; q < kPerThread; ++q) b[q] = j0 + q < n ? src[j0 + q] : uint16_t(0);
    }
}

// The code book in LDS (256 threads), so that per-value lookups are LDS reads.
struct BookLds {
    uint32_t code[256];
    uint8_t len[256];
};

__device__ __forceinline__ void stage_book(const Book &book, BookLds &s) {
    s.code[threadIdx.x] = book.code[threadIdx.x];
    s.len[threadIdx.x] = book.len[threadIdx.x];
    __syncthreads();
}

// Block-wide exclusive scan of one u32 per thread (256 threads).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *sh, uint32_t &total) {
    const uint32_t t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (uint32_t d = 1; d < kSegThreads; d <<= 1) {
        const uint32_t add = t >= d ? sh[t - d] : 0u;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    total = sh[kSegThreads - 1];
    const uint32_t incl = sh[t];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(256) void segment_bits_kernel(const uint16_t *src, uint64_t n, Book book,
                                                           uint32_t *seg_bits) {
    __shared__ uint32_t sh[kSegThreads];
    __shared__ BookLds bk;
    stage_book(book, bk);
    const uint64_t j0 = uint64_t(blockIdx.x) * kSegElems + uint64_t(threadIdx.x) * kPerThread;
    uint16_t b[kPerThread];
    load16(src, n, j0, b);
    uint32_t bits = 0;
#pragma unroll
    for (uint32_t q = 0; q < kPerThread; ++q)
        if (j0 + q < n) bits += bk.len[exponent_of(b[q])];
    uint32_t total;
    block_exclusive_scan(bits, sh, total);
    if (threadIdx.x == 0) seg_bits[blockIdx.x] = total;
}

// Exclusive prefix over the segments (one workgroup of 1024 threads): each
// thread sums a contiguous run of segments, one workgroup scan places the
// runs, and each thread writes its run's prefixes.
__global__ __launch_bounds__(1024) void segment_scan_kernel(const uint32_t *seg_bits, uint64_t nseg,
                                                            uint64_t *seg_off) {
    __shared__ uint64_t sh[1024];
    const uint32_t t = threadIdx.x;
    const uint64_t per = (nseg + 1023) / 1024;
    const uint64_t i0 = min(uint64_t(t) * per, nseg), i1 = min(i0 + per, nseg);
    uint64_t sum = 0;
    for (uint64_t i = i0; i < i1; ++i) sum += seg_bits[i];
    sh[t] = sum;
    __syncthreads();
    for (uint32_t d = 1; d < 1024; d <<= 1) {
        const uint64_t add = t >= d ? sh[t - d] : 0;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    uint64_t run = sh[t] - sum;
    for (uint64_t i = i0; i < i1; ++i) {
        const uint64_t v = seg_bits[i];
        seg_off[i] = run;
        run += v;
    }
}

struct PackArgs {
    const uint16_t *src;
    uint64_t n;
    uint32_t *words;     // stream words (zeroed)
    uint32_t *offw;      // packed 5-bit offsets (zeroed)
    uint32_t *blockout;  // u32 out[n_blocks + 1]
    uint8_t *raw;        // raw bytes
    const uint64_t *seg_off;
    uint32_t chunk_shift;  // log2(8 C)
    uint32_t lanes_shift;  // log2(T)
};

__device__ __forceinline__ void or_word(uint32_t *words, uint64_t w, uint32_t v) {
    if (v) atomicOr(&words[w], v);
}

// A segment of 4096 values codes to at most 4096 * 24 bits: its words, and
// the 5-bit offset fields of the chunk boundaries inside it (at least 32
// bits per chunk), fit these LDS buffers.
constexpr uint32_t kSegWords = kSegElems * 24u / 32u + 2u;
constexpr uint32_t kSegOffWords = (5u * (kSegElems * 24u / 32u + 1u) + 4u) / 32u + 3u;

// One workgroup per segment of 4096 values.  The threads OR their codes and
// offset fields into LDS copies of the segment's words; the words wholly
// inside the segment then go to HBM with plain stores and only its first and
// last word of each section, which neighbouring segments share, with atomic
// ORs (onto the zeroed container).
__global__ __launch_bounds__(256) void pack_kernel(const PackArgs a, const Book book) {
    __shared__ uint32_t sh[kSegThreads];
    __shared__ BookLds bk;
    __shared__ uint32_t wbuf[kSegWords];
    __shared__ uint32_t obuf[kSegOffWords];
    stage_book(book, bk);
    const uint32_t t = threadIdx.x;
    const uint64_t j0 = uint64_t(blockIdx.x) * kSegElems + uint64_t(t) * kPerThread;
    uint16_t b[kPerThread];
    load16(a.src, a.n, j0, b);
    uint32_t bits = 0;
#pragma unroll
    for (uint32_t q = 0; q < kPerThread; ++q)
        if (j0 + q < a.n) bits += bk.len[exponent_of(b[q])];
    uint32_t seg_total;
    const uint32_t before = block_exclusive_scan(bits, sh, seg_total);
    const uint64_t seg_start = a.seg_off[blockIdx.x], seg_end = seg_start + seg_total;
    const uint64_t start = seg_start + before;

    // the segment's words [wb0, wb0 + nw) and offset words [ob0, ob0 + no)
    const uint32_t cs = a.chunk_shift;
    const uint64_t wb0 = seg_start >> 5;
    const uint32_t nw = seg_total ? uint32_t(((seg_end - 1) >> 5) - wb0 + 1) : 0u;
    const uint64_t c_lo = (seg_start >> cs) + 1, c_hi = seg_end >> cs;  // boundaries in (seg_start, seg_end]
    const uint64_t ob0 = (5 * c_lo) >> 5;
    const uint32_t no = c_lo <= c_hi ? uint32_t(((5 * c_hi + 4) >> 5) - ob0 + 1) : 0u;
    for (uint32_t i = t; i < nw; i += kSegThreads) wbuf[i] = 0u;
    for (uint32_t i = t; i < no; i += kSegThreads) obuf[i] = 0u;
    __syncthreads();

    // Raw bytes: 16 per thread, one store when all are in range.
    if (j0 + kPerThread <= a.n) {
        uint32_t r[4] = {0, 0, 0, 0};
#pragma unroll
        for (uint32_t q = 0; q < kPerThread; ++q) r[q >> 2] |= raw_of(b[q]) << (8 * (q & 3));
        *reinterpret_cast<uint4 *>(a.raw + j0) = make_uint4(r[0], r[1], r[2], r[3]);
    } else {
        for (uint32_t q = 0; q < kPerThread && j0 + q < a.n; ++q) a.raw[j0 + q] = uint8_t(raw_of(b[q]));
    }

    // Codes: MSB-first into 32-bit words.
    uint64_t pos = start;
    uint64_t acc = 0;
    uint32_t nacc = uint32_t(pos & 31);
    uint32_t w = uint32_t((pos >> 5) - wb0);
    for (uint32_t q = 0; q < kPerThread; ++q) {
        const uint64_t j = j0 + q;
        if (j >= a.n) break;
        const uint32_t e = exponent_of(b[q]);
        const uint32_t l = bk.len[e];
        // A chunk boundary inside (pos, pos + l]: the next code starts at pos + l.
        const uint64_t c = (pos >> cs) + 1;
        if ((c << cs) <= pos + l) {
            const uint32_t off = uint32_t(pos + l - (c << cs));
            const uint64_t g = 5ull * c;
            const uint64_t v = uint64_t(off) << (g & 31);
            const uint32_t o = uint32_t((g >> 5) - ob0);
            if (uint32_t(v)) atomicOr(&obuf[o], uint32_t(v));
            if (uint32_t(v >> 32)) atomicOr(&obuf[o + 1], uint32_t(v >> 32));
            if ((c & ((uint64_t(1) << a.lanes_shift) - 1)) == 0) a.blockout[c >> a.lanes_shift] = uint32_t(j + 1);
        }
        acc = (acc << l) | bk.code[e];
        nacc += l;
        pos += l;
        if (nacc >= 32) {
            nacc -= 32;
            const uint32_t v = uint32_t(acc >> nacc);
            if (v) atomicOr(&wbuf[w], v);
            ++w;
        }
    }
    if (nacc > 0) {
        const uint32_t v = uint32_t(acc << (32 - nacc));
        if (v) atomicOr(&wbuf[w], v);
    }
    __syncthreads();

    for (uint32_t i = t; i < nw; i += kSegThreads) {
        if (i == 0 || i == nw - 1) {
            if (wbuf[i]) atomicOr(&a.words[wb0 + i], wbuf[i]);
        } else {
            a.words[wb0 + i] = wbuf[i];
        }
    }
    for (uint32_t i = t; i < no; i += kSegThreads) {
        if (i == 0 || i == no - 1) {
            if (obuf[i]) atomicOr(&a.offw[ob0 + i], obuf[i]);
        } else {
            a.offw[ob0 + i] = obuf[i];
        }
    }
}

// ------------------------------------------------------------------ rANS

// Per-symbol coding constants: frequency, cumulative frequency and
// ceil(2^32 / f) (0 for f = 1), so that v / f needs no divide: the high half
// of v * magic is the quotient or one more.
struct AnsBook {
    uint16_t f[256], cum[256];
    uint32_t magic[256];
};

struct AnsArgs {
    const uint16_t *src;
    uint32_t n, steps, n_blocks;
    uint32_t *counts;        // pass 1: 16-bit words per block (counts[n_blocks] = 0)
    const uint64_t *first;   // pass 2: first word of every block (n_blocks + 1)
    uint16_t *words;         // pass 2: the words section
    uint32_t *offsets;       // pass 2: the offsets section (n_blocks + 1)
    uint32_t *states;        // pass 2: 64 initial decoder states per block
};

constexpr uint32_t kAnsEncWaves = 4;

// One wavefront per block, lane l coding the elements 64 i + l.  The steps
// run backwards (a decoder reads them forwards) and, inside a step, lanes
// 63 down to 0 emit first: a word's place in decode order is the block's
// word count minus one minus the words emitted before it.
template <bool Write>
__global__ __launch_bounds__(kAnsEncWaves * 64) void ans_encode_kernel(const AnsArgs a, const AnsBook book) {
    __shared__ uint32_t fc[256], mg[256];  // f | cum << 16, magic
    for (uint32_t s = threadIdx.x; s < 256; s += blockDim.x) {
        fc[s] = uint32_t(book.f[s]) | (uint32_t(book.cum[s]) << 16);
        mg[s] = book.magic[s];
    }
    __syncthreads();
    const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const uint32_t b = blockIdx.x * kAnsEncWaves + wave;
    if (b >= a.n_blocks) return;
    const uint32_t per = 64u * a.steps, e0 = b * per;
    const uint32_t cnt = min(per, a.n - e0), steps = (cnt + 63u) / 64u;
    uint32_t x = uint32_t(dfc::kAnsLow), emitted = 0;
    uint64_t base = 0;
    uint32_t last = 0;
    if constexpr (Write) {
        base = a.first[b];
        last = uint32_t(a.first[b + 1] - base) - 1u;  // unused when the block has no words
    }
    // Steps run from the block's last to its first, eight at a time: the eight
    // symbols are loaded first (independent loads in flight together), then
    // the eight dependent state updates run.
    for (uint32_t top = steps; top > 0;) {
        const uint32_t g = min(top, 8u);
        uint32_t syms[8];
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
            const uint32_t j = 64u * (top - 1u - k) + lane;
            syms[k] = k < g && j < cnt ? (uint32_t(a.src[e0 + j]) >> 7) & 0xFFu : 0u;
        }
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
            if (k >= g) break;
            const uint32_t j = 64u * (top - 1u - k) + lane;
            const bool live = j < cnt;
            const uint32_t sym = syms[k];
            const uint32_t e = fc[sym], f = e & 0xFFFFu, cum = e >> 16;
            // x >= f 2^20, without forming f << 20 (2^32 for a lone symbol)
            const bool emit = live && (x >> 20) >= f;
            const uint64_t m = __builtin_amdgcn_ballot_w64(emit);
            if constexpr (Write) {
                if (emit) {
                    const uint32_t above = uint32_t(__builtin_popcountll(lane == 63 ? 0ull : m >> (lane + 1)));
                    a.words[base + (last - emitted - above)] = uint16_t(x & 0xFFFFu);
                }
            }
            const uint32_t v = emit ? x >> 16 : x;
            // q = v / f, r = v mod f
            uint32_t q = f == 1u ? v : __umulhi(v, mg[sym]);
            uint32_t r = v - q * f;
            if (r >= f) {  // q was one too large
                --q;
                r += f;
            }
            if (live) x = q * uint32_t(dfc::kAnsSlots) + r + cum;
            emitted += uint32_t(__builtin_popcountll(m));
        }
        top -= g;
    }
    if constexpr (!Write) {
        if (lane == 0) {
            a.counts[b] = emitted;
            if (b == 0) a.counts[a.n_blocks] = 0u;
        }
    } else {
        a.states[64ull * b + lane] = x;
        if (lane == 0) {
            a.offsets[b] = uint32_t(base);
            if (b + 1 == a.n_blocks) a.offsets[a.n_blocks] = uint32_t(a.first[a.n_blocks]);
        }
    }
}

// Raw bytes (sign << 7 | mantissa) of n elements, 16 per thread.
__global__ __launch_bounds__(256) void raw_kernel(const uint16_t *src, uint64_t n, uint8_t *raw) {
    for (uint64_t j0 = (uint64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 16; j0 < n;
         j0 += uint64_t(gridDim.x) * blockDim.x * 16) {
        if (j0 + 16 <= n) {
            uint16_t b[16];
            load16(src, n, j0, b);
            uint32_t r[4] = {0, 0, 0, 0};
#pragma unroll
            for (uint32_t q = 0; q < 16; ++q) r[q >> 2] |= raw_of(b[q]) << (8 * (q & 3));
            *reinterpret_cast<uint4 *>(raw + j0) = make_uint4(r[0], r[1], r[2], r[3]);
        } else {
            for (uint64_t j = j0; j < n; ++j) raw[j] = uint8_t(raw_of(src[j]));
        }
    }
}

// ----------------------------------------------------------------- panels

// Panel layout: items of 32 rows x panel_k columns, row panels first; inside
// an item, element i = 512 t + 8 l + j is W[r0 + l mod 32][c0 + 16 t +
// 8 (l div 32) + j].  Every item is packed on its own from a fresh chunk.
struct PanelArgs {
    const uint16_t *src;
    uint64_t cols;
    uint32_t slices, panel_k;
    uint32_t *item_bits;    // pass 1: code bits per item
    const uint32_t *first;  // pass 2: (first chunk, first block) per item, n_items + 1 pairs
    uint32_t *words, *offw, *blockout;
    uint32_t *counts;  // one count per chunk, count_shift = log2(32 / count bits) to a word
    uint8_t *raw;
    uint32_t chunk_shift, lanes_shift;  // log2(8 C), log2(T)
    uint32_t count_shift;               // 2 (byte counts) or 1 (16-bit counts)
};

struct PanelItem {
    uint64_t row0, col0, e0;
    uint32_t nq;
};

__device__ __forceinline__ PanelItem panel_item(const PanelArgs &a, uint32_t q) {
    PanelItem it;
    const uint64_t p = q / a.slices;
    it.row0 = 32ull * p;
    it.col0 = uint64_t(a.panel_k) * (q % a.slices);
    it.nq = 32u * uint32_t(min(uint64_t(a.panel_k), a.cols - it.col0));
    it.e0 = 32ull * (p * a.cols + it.col0);
    return it;
}

// Octet o of an item (its values 8 o .. 8 o + 7 in panel order) is eight
// consecutive columns of one row (columns and slice widths are multiples of
// 16): one 16-byte load when the source is 16-byte aligned.
__device__ __forceinline__ uint4 panel_octet(const PanelArgs &a, const PanelItem &it, uint32_t o, bool vec) {
    const uint32_t t = o >> 6, l = o & 63u;
    const uint64_t at = (it.row0 + (l & 31u)) * a.cols + it.col0 + 16u * t + 8u * (l >> 5);
    if (vec) return *reinterpret_cast<const uint4 *>(a.src + at);
    uint32_t w[4];
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) w[k] = uint32_t(a.src[at + 2 * k]) | (uint32_t(a.src[at + 2 * k + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t octet_value(const uint4 &v, uint32_t j) {
    const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return (w >> (16 * (j & 1))) & 0xFFFFu;
}

constexpr uint32_t kOctBatch = 4;  // octets loaded together (independent loads in flight)

// One workgroup per item: its code bits.
__global__ __launch_bounds__(256) void panel_bits_kernel(const PanelArgs a, const Book book) {
    __shared__ uint32_t sh[kSegThreads];
    __shared__ BookLds bk;
    stage_book(book, bk);
    const PanelItem it = panel_item(a, blockIdx.x);
    const bool vec = (reinterpret_cast<uintptr_t>(a.src) & 15u) == 0;
    const uint32_t n_oct = it.nq / 8;
    uint32_t bits = 0;
    for (uint32_t ob = threadIdx.x; ob < n_oct; ob += kSegThreads * kOctBatch) {
        uint4 v[kOctBatch];
#pragma unroll
        for (uint32_t k = 0; k < kOctBatch; ++k)
            v[k] = ob + k * kSegThreads < n_oct ? panel_octet(a, it, ob + k * kSegThreads, vec) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (uint32_t k = 0; k < kOctBatch; ++k)
            if (ob + k * kSegThreads < n_oct)
#pragma unroll
                for (uint32_t j = 0; j < 8; ++j) bits += bk.len[exponent_of(octet_value(v[k], j))];
    }
    uint32_t total;
    block_exclusive_scan(bits, sh, total);
    if (threadIdx.x == 0) a.item_bits[blockIdx.x] = total;
}

// One workgroup per item: thread t packs a contiguous run of the item's
// octets at its bit position (interior words stored, the two words shared
// with neighbours ORed), writes their raw bytes (8 per octet), and, for
// every chunk of the item whose first bit its codes cover, that chunk's
// 5-bit offset (the next code starts where the covering code ends) and, on
// block boundaries, the block's first element (panel order).  Its codes
// start in consecutive chunks: it adds the number that start in each chunk
// to that chunk's count when it moves on (atomically, since the first and
// last chunk, and the word that holds several counts, may be shared).
__global__ __launch_bounds__(256) void panel_pack_kernel(const PanelArgs a, const Book book) {
    __shared__ uint32_t sh[kSegThreads];
    __shared__ BookLds bk;
    stage_book(book, bk);
    const uint32_t q = blockIdx.x;
    const PanelItem it = panel_item(a, q);
    const bool vec = (reinterpret_cast<uintptr_t>(a.src) & 15u) == 0;
    const uint32_t n_oct = it.nq / 8;
    const uint32_t per = (n_oct + kSegThreads - 1) / kSegThreads;
    const uint32_t o0 = min(threadIdx.x * per, n_oct), o1 = min(o0 + per, n_oct);
    uint32_t bits = 0;
    for (uint32_t ob = o0; ob < o1; ob += kOctBatch) {
        uint4 v[kOctBatch];
#pragma unroll
        for (uint32_t k = 0; k < kOctBatch; ++k)
            v[k] = ob + k < o1 ? panel_octet(a, it, ob + k, vec) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (uint32_t k = 0; k < kOctBatch; ++k)
            if (ob + k < o1)
#pragma unroll
                for (uint32_t j = 0; j < 8; ++j) bits += bk.len[exponent_of(octet_value(v[k], j))];
    }
    uint32_t total;
    const uint64_t start = block_exclusive_scan(bits, sh, total);
    const uint32_t c0 = a.first[2 * q], b0 = a.first[2 * q + 1];
    const uint32_t chunks = a.first[2 * q + 2] - c0;
    if (threadIdx.x == 0) a.blockout[b0] = uint32_t(it.e0);
    uint32_t *words = a.words + (uint64_t(c0) << (a.chunk_shift - 5));
    uint64_t pos = start, acc = 0;
    uint32_t nacc = uint32_t(pos & 31);
    uint64_t w = pos >> 5;
    const uint64_t first_word = w, last_word = bits ? (start + bits - 1) >> 5 : w;
    uint64_t cur = pos >> a.chunk_shift;
    uint32_t ncur = 0;
    auto flush_count = [&]() {
        if (ncur) {
            // a chunk's final count fits its field, so no carry crosses fields
            const uint64_t c = c0 + cur;
            const uint32_t per_word = 1u << a.count_shift;
            atomicAdd(a.counts + (c >> a.count_shift), ncur << ((32u / per_word) * uint32_t(c & (per_word - 1u))));
        }
    };
    for (uint32_t ob = o0; ob < o1; ob += kOctBatch) {
        uint4 v[kOctBatch];
#pragma unroll
        for (uint32_t k = 0; k < kOctBatch; ++k)
            v[k] = ob + k < o1 ? panel_octet(a, it, ob + k, vec) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (uint32_t k = 0; k < kOctBatch; ++k) {
            if (ob + k >= o1) break;
            const uint32_t o = ob + k;
            uint32_t r[2] = {0u, 0u};
#pragma unroll
            for (uint32_t j = 0; j < 8; ++j) {
                const uint32_t b = octet_value(v[k], j), i = 8u * o + j;
                r[j >> 2] |= raw_of(b) << (8 * (j & 3));
                const uint32_t e = exponent_of(b);
                const uint32_t l = bk.len[e];
                if ((pos >> a.chunk_shift) != cur) {
                    flush_count();
                    cur = pos >> a.chunk_shift;
                    ncur = 0;
                }
                ++ncur;
                const uint64_t c = (pos >> a.chunk_shift) + 1;
                if (c < chunks && (c << a.chunk_shift) <= pos + l) {
                    const uint32_t off = uint32_t(pos + l - (c << a.chunk_shift));
                    const uint64_t g = 5ull * (c0 + c);
                    const uint64_t vv = uint64_t(off) << (g & 31);
                    or_word(a.offw, g >> 5, uint32_t(vv));
                    or_word(a.offw, (g >> 5) + 1, uint32_t(vv >> 32));
                    if ((c & ((uint64_t(1) << a.lanes_shift) - 1)) == 0)
                        a.blockout[b0 + (c >> a.lanes_shift)] = uint32_t(it.e0 + i + 1);
                }
                acc = (acc << l) | bk.code[e];
                nacc += l;
                pos += l;
                if (nacc >= 32) {
                    nacc -= 32;
                    const uint32_t wv = uint32_t(acc >> nacc);
                    if (w == first_word || w == last_word) or_word(words, w, wv);
                    else words[w] = wv;
                    ++w;
                }
            }
            *reinterpret_cast<uint2 *>(a.raw + it.e0 + 8u * o) = make_uint2(r[0], r[1]);
        }
    }
    if (nacc > 0) or_word(words, w, uint32_t(acc << (32 - nacc)));
    flush_count();
}

// Host copy of a workspace layout.
// segbits/segoff hold one entry per 4096-element segment (FLAT) or per rANS
// block plus one (the smallest rANS block is 64 x 8 elements).
struct Workspace {
    uint64_t hist_off, segbits_off, segoff_off, bytes, nseg, slots;
};
Workspace workspace_layout(uint64_t n) {
    Workspace w;
    w.nseg = dfc::ceil_div(std::max<uint64_t>(n, 1), kSegElems);
    w.slots = std::max<uint64_t>(w.nseg, dfc::ceil_div(std::max<uint64_t>(n, 1), uint64_t(dfc::kAnsLanes) * 8) + 1);
    w.hist_off = 0;
    w.segbits_off = 1024;
    w.segoff_off = dfc::align256(w.segbits_off + 4 * w.slots);
    w.bytes = dfc::align256(w.segoff_off + 8 * w.slots);
    return w;
}

dfc_status hip_ok(hipError_t e) { return e == hipSuccess ? DFC_OK : DFC_EHIP; }

// The rANS layout from the device histogram: count pass, scan, section
// layout and header on the host, write pass, raw bytes.
dfc_status encode_ans_device(const uint16_t *src_dev, uint64_t n, const dfc_params &p, uint64_t rows, uint64_t cols,
                             const uint64_t hist[256], uint8_t *dst, uint64_t cap, uint8_t *work, const Workspace &ws,
                             uint64_t *written, hipStream_t st) {
    const uint32_t S = dfc::ans_steps_or_default(p.ans_steps);
    const uint64_t nb = dfc::ceil_div(n, uint64_t(dfc::kAnsLanes) * S);
    if (nb + 1 > ws.slots) return DFC_ESIZE;
    uint32_t f[256], cum[256];
    dfc::ans_frequencies(hist, f, cum);
    AnsBook book;
    for (int s = 0; s < 256; ++s) {
        book.f[s] = uint16_t(f[s]);
        book.cum[s] = uint16_t(cum[s]);
        book.magic[s] = f[s] >= 2 ? uint32_t(((uint64_t(1) << 32) + f[s] - 1) / f[s]) : 0u;
    }
    AnsArgs a;
    std::memset(&a, 0, sizeof(a));
    a.src = src_dev;
    a.n = uint32_t(n);
    a.steps = S;
    a.n_blocks = uint32_t(nb);
    a.counts = reinterpret_cast<uint32_t *>(work + ws.segbits_off);
    uint64_t *first = reinterpret_cast<uint64_t *>(work + ws.segoff_off);
    a.first = first;
    const uint32_t grid = uint32_t(dfc::ceil_div(nb, uint64_t(kAnsEncWaves)));
    uint64_t nw = 0;
    if (nb) {
        hipLaunchKernelGGL(ans_encode_kernel<false>, dim3(grid), dim3(kAnsEncWaves * 64), 0, st, a, book);
        hipLaunchKernelGGL(segment_scan_kernel, dim3(1), dim3(1024), 0, st, a.counts, nb + 1, first);
        if (hipMemcpyAsync(&nw, first + nb, sizeof(nw), hipMemcpyDeviceToHost, st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return DFC_EHIP;
    }
    if (nw >= (uint64_t(1) << 32)) return DFC_ESIZE;
    const dfc::SectionSizes sz = dfc::ans_section_sizes(n, nw, nb);
    uint64_t off[dfc::kNumSections];
    const uint64_t blob_bytes = dfc::place_sections(sz, off);
    if (cap < blob_bytes) return DFC_ESIZE;
    std::vector<uint8_t> head(dfc::head_bytes(sz, off), 0);
    dfc::ans_container_head(head.data(), n, nw, nb, S, rows, cols, sz, off, blob_bytes, f);
    hipLaunchKernelGGL(fill_zero_u32, dim3(uint32_t(std::min<uint64_t>(65535, dfc::ceil_div(blob_bytes / 4, 256)))),
                       dim3(256), 0, st, reinterpret_cast<uint32_t *>(dst), blob_bytes / 4);
    if (hipMemcpyAsync(dst, head.data(), head.size(), hipMemcpyHostToDevice, st) != hipSuccess) return DFC_EHIP;
    if (nb) {
        a.words = reinterpret_cast<uint16_t *>(dst + off[dfc::kWords]);
        a.offsets = reinterpret_cast<uint32_t *>(dst + off[dfc::kOffsets]);
        a.states = reinterpret_cast<uint32_t *>(dst + off[dfc::kBlockout]);
        hipLaunchKernelGGL(ans_encode_kernel<true>, dim3(grid), dim3(kAnsEncWaves * 64), 0, st, a, book);
        hipLaunchKernelGGL(raw_kernel, dim3(uint32_t(std::min<uint64_t>(65535, dfc::ceil_div(n, 256 * 16)))), dim3(256),
                           0, st, src_dev, n, dst + off[dfc::kRaw]);
    }
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess) return DFC_EHIP;
    *written = blob_bytes;
    return DFC_OK;
}

// The panel layout from the device histogram and the code: bits per item,
// item placement and sections on the host, then every item packed on the
// device.
dfc_status encode_panel_device(const uint16_t *src_dev, uint64_t n, const dfc_params &p, const Book &book,
                               const uint8_t len[256], uint8_t *dst, uint64_t cap, uint8_t *work,
                               const Workspace &ws, uint64_t *written, hipStream_t st) {
    dfc::PanelGeom g;
    if (!dfc::panel_geom(p.rows, p.cols, p.panel_k, g) || g.rows * g.cols != n) return DFC_EINVAL;
    // item bit counts are 32-bit on the device
    if (32ull * std::min<uint64_t>(g.panel_k, g.cols) * dfc::kMaxLen >= (uint64_t(1) << 32)) return DFC_EUNSUPPORTED;
    if (g.n_items + 1 > ws.slots) return DFC_ESIZE;
    const uint32_t C = p.chunk_bytes, T = p.lanes_per_block;
    PanelArgs a;
    std::memset(&a, 0, sizeof(a));
    a.src = src_dev;
    a.cols = g.cols;
    a.slices = uint32_t(g.slices);
    a.panel_k = uint32_t(g.panel_k);
    a.item_bits = reinterpret_cast<uint32_t *>(work + ws.segbits_off);
    a.chunk_shift = uint32_t(__builtin_ctz(8u * C));  // C and T are powers of two
    a.lanes_shift = uint32_t(__builtin_ctz(T));
    hipLaunchKernelGGL(panel_bits_kernel, dim3(uint32_t(g.n_items)), dim3(kSegThreads), 0, st, a, book);
    std::vector<uint32_t> bits(g.n_items);
    if (hipMemcpyAsync(bits.data(), a.item_bits, 4 * g.n_items, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return DFC_EHIP;
    std::vector<uint32_t> first(2 * (g.n_items + 1), 0);
    uint64_t chunks = 0, blocks = 0, total_bits = 0;
    for (uint64_t q = 0; q < g.n_items; ++q) {
        first[2 * q] = uint32_t(chunks);
        first[2 * q + 1] = uint32_t(blocks);
        const uint64_t cq = dfc::ceil_div(uint64_t(bits[q]), 8ull * C);
        chunks += cq;
        blocks += dfc::ceil_div(cq, uint64_t(T));
        total_bits += bits[q];
        if (chunks >= (uint64_t(1) << 32) || blocks >= (uint64_t(1) << 32)) return DFC_ESIZE;
    }
    first[2 * g.n_items] = uint32_t(chunks);
    first[2 * g.n_items + 1] = uint32_t(blocks);
    const dfc::SectionSizes sz = dfc::section_sizes(n, chunks, blocks, C, p.lut_bits, g.n_items);
    uint64_t off[dfc::kNumSections];
    const uint64_t blob_bytes = dfc::place_sections(sz, off);
    if (cap < blob_bytes) return DFC_ESIZE;
    std::vector<uint8_t> head(dfc::head_bytes(sz, off), 0);
    dfc::container_header(head.data(), p, n, total_bits, chunks, blocks, g.rows, g.cols, sz, off, blob_bytes, len);
    // the item table: (first chunk, first block, code bits, 0) per item and a sentinel
    std::vector<uint32_t> table(4 * (g.n_items + 1), 0);
    for (uint64_t q = 0; q <= g.n_items; ++q) {
        table[4 * q] = first[2 * q];
        table[4 * q + 1] = first[2 * q + 1];
        table[4 * q + 2] = q < g.n_items ? bits[q] : 0u;
    }
    const uint32_t n_out = uint32_t(n);
    uint32_t *first_dev = reinterpret_cast<uint32_t *>(work + ws.segoff_off);
    hipLaunchKernelGGL(fill_zero_u32, dim3(uint32_t(std::min<uint64_t>(65535, dfc::ceil_div(blob_bytes / 4, 256)))),
                       dim3(256), 0, st, reinterpret_cast<uint32_t *>(dst), blob_bytes / 4);
    if (hipMemcpyAsync(dst, head.data(), head.size(), hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(dst + off[dfc::kPanels], table.data(), 4 * table.size(), hipMemcpyHostToDevice, st) !=
            hipSuccess ||
        hipMemcpyAsync(dst + off[dfc::kBlockout] + 4 * blocks, &n_out, 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(first_dev, first.data(), 4 * first.size(), hipMemcpyHostToDevice, st) != hipSuccess)
        return DFC_EHIP;
    a.first = first_dev;
    a.words = reinterpret_cast<uint32_t *>(dst + off[dfc::kWords]);
    a.offw = reinterpret_cast<uint32_t *>(dst + off[dfc::kOffsets]);
    a.blockout = reinterpret_cast<uint32_t *>(dst + off[dfc::kBlockout]);
    a.counts = reinterpret_cast<uint32_t *>(dst + off[dfc::kCounts]);
    a.count_shift = dfc::count_width(C) == 1 ? 2u : 1u;
    a.raw = dst + off[dfc::kRaw];
    hipLaunchKernelGGL(panel_pack_kernel, dim3(uint32_t(g.n_items)), dim3(kSegThreads), 0, st, a, book);
    // the host vectors must outlive the copies above
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess) return DFC_EHIP;
    *written = blob_bytes;
    return DFC_OK;
}

// The workspace of dfc_encode_device_noalloc: a fixed array in device
// memory, one copy per GPU the library runs on, held until the process
// ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies get the address hipGetSymbolAddress
// returns for the device, kept per device below.
__device__ __align__(256) uint8_t scratch[DFC_NOALLOC_WORKSPACE_BYTES];

struct DeviceScratch {
    void *ptr = nullptr;  // this device's copy of `scratch`
    std::mutex mu;        // held for a whole call: the copy is shared
};

// The scratch of device `dev`: its address is looked up once, with that
// device current, and kept.
dfc_status device_scratch(int dev, DeviceScratch **out) {
    static std::mutex table_mu;
    static std::map<int, std::unique_ptr<DeviceScratch>> table;
    std::lock_guard<std::mutex> lock(table_mu);
    auto it = table.find(dev);
    if (it == table.end()) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return DFC_EHIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return DFC_EHIP;
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return DFC_EHIP;
        if (e != hipSuccess || !ptr) return DFC_EHIP;
        auto s = std::make_unique<DeviceScratch>();
        s->ptr = ptr;
        it = table.emplace(dev, std::move(s)).first;
    }
    *out = it->second.get();
    return DFC_OK;
}

}  // namespace

extern "C" {

dfc_status dfc_encode_device_noalloc(const uint16_t *src_dev, uint64_t n, const dfc_params *p, const dfc_codebook *cb,
                                     void *dst_dev, uint64_t cap, uint64_t *written, void *stream) {
    if (workspace_layout(n).bytes > DFC_NOALLOC_WORKSPACE_BYTES) return DFC_ESIZE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess) return DFC_EHIP;
    DeviceScratch *ds = nullptr;
    const dfc_status s = device_scratch(dev, &ds);
    if (s != DFC_OK) return s;
    // dfc_encode_device returns with its stream idle, so holding the lock
    // for the call keeps every other call on this device off the scratch
    std::lock_guard<std::mutex> lock(ds->mu);
    return dfc_encode_device(src_dev, n, p, cb, dst_dev, cap, ds->ptr, DFC_NOALLOC_WORKSPACE_BYTES, written, stream);
}

dfc_status dfc_encode_device_workspace(uint64_t n, uint64_t *bytes) {
    if (!bytes) return DFC_EINVAL;
    *bytes = workspace_layout(n).bytes;
    return DFC_OK;
}

dfc_status dfc_histogram_device(const uint16_t *src_dev, uint64_t n, uint32_t *hist_dev, void *stream) {
    if ((!src_dev && n) || !hist_dev) return DFC_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(fill_zero_u32, dim3(1), dim3(256), 0, st, hist_dev, uint64_t(256));
    if (n) {
        // about four workgroups per CU, each over many 16-byte loads, so that
        // clearing and summing the sub-histograms is paid rarely (329 -> 198 us
        // for 218 M values against 4096 workgroups)
        const uint32_t grid = uint32_t(std::min<uint64_t>(1024, dfc::ceil_div(n, 256 * 16)));
        hipLaunchKernelGGL(histogram_kernel, dim3(std::max(1u, grid)), dim3(256), 0, st, src_dev, n, hist_dev);
    }
    return hip_ok(hipGetLastError());
}

dfc_status dfc_encode_device(const uint16_t *src_dev, uint64_t n, const dfc_params *pin, const dfc_codebook *cb_in,
                             void *dst_dev, uint64_t cap, void *work_dev, uint64_t work_bytes, uint64_t *written,
                             void *stream) {
    dfc_params p;
    if (pin) p = *pin; else dfc_default_params(&p);
    if ((!src_dev && n) || !dst_dev || !written || !work_dev || !dfc::encoder_params_ok(p)) return DFC_EINVAL;
    if (p.layout == DFC_LAYOUT_PADDED) return DFC_EUNSUPPORTED;
    if (p.layout == DFC_LAYOUT_PANEL && !p.panel_k) p.panel_k = DFC_PANEL_K_DEFAULT;
    if (p.layout == DFC_LAYOUT_ANS && cb_in) return DFC_EINVAL;  // frequencies come from src's own histogram
    if ((reinterpret_cast<uintptr_t>(dst_dev) & 255u) || (reinterpret_cast<uintptr_t>(work_dev) & 255u) ||
        (reinterpret_cast<uintptr_t>(src_dev) & 1u))
        return DFC_EINVAL;
    if (n >= (uint64_t(1) << 32)) return DFC_ESIZE;
    uint64_t rows = p.rows, cols = p.cols;
    if (rows == 0 && cols == 0) {
        rows = 1;
        cols = n;
    }
    if (rows * cols != n) return DFC_EINVAL;
    const Workspace ws = workspace_layout(n);
    if (work_bytes < ws.bytes) return DFC_ESIZE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *work = static_cast<uint8_t *>(work_dev);
    uint32_t *hist_dev = reinterpret_cast<uint32_t *>(work + ws.hist_off);

    // 1. histogram -> host
    dfc_status s = dfc_histogram_device(src_dev, n, hist_dev, stream);
    if (s != DFC_OK) return s;
    uint32_t h32[256];
    if (hipMemcpyAsync(h32, hist_dev, sizeof(h32), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return DFC_EHIP;
    uint64_t hist[256];
    for (int i = 0; i < 256; ++i) hist[i] = h32[i];
    if (p.layout == DFC_LAYOUT_ANS)
        return encode_ans_device(src_dev, n, p, rows, cols, hist, static_cast<uint8_t *>(dst_dev), cap, work, ws,
                                 written, st);

    // 2. codebook, layout and header on the host
    uint8_t len[256];
    if (cb_in) {
        std::memcpy(len, cb_in->len, 256);
        uint32_t used = 0;
        for (int i = 0; i < 256; ++i) {
            if (len[i] > p.max_code_len || (hist[i] && !len[i])) return DFC_EINVAL;
            used += len[i] != 0;
        }
        if (n && (used < 2 || dfc::kraft_sum(len) != (uint64_t(1) << dfc::kMaxLen))) return DFC_EINVAL;
    } else {
        s = dfc::code_lengths(hist, p.max_code_len, len);
        if (s != DFC_OK) return s;
    }
    if (p.chunk_bytes == 0)
        p.chunk_bytes = p.layout == DFC_LAYOUT_FLAT ? dfc::choose_chunk_bytes(hist, len, p.lanes_per_block) : 16u;
    Book book;
    dfc::canonical_codes(len, book.code);
    std::memcpy(book.len, len, 256);
    if (p.layout == DFC_LAYOUT_PANEL)
        return encode_panel_device(src_dev, n, p, book, len, static_cast<uint8_t *>(dst_dev), cap, work, ws, written,
                                   st);
    uint64_t total_bits = 0;
    for (int i = 0; i < 256; ++i) total_bits += hist[i] * len[i];
    const uint32_t C = p.chunk_bytes, T = p.lanes_per_block;
    const dfc::Layout L = dfc::layout_sizes(total_bits, C, T);
    const dfc::SectionSizes sz = dfc::section_sizes(n, L.n_chunks, L.n_blocks, C, p.lut_bits);
    uint64_t off[dfc::kNumSections];
    const uint64_t blob_bytes = dfc::place_sections(sz, off);
    if (cap < blob_bytes) return DFC_ESIZE;
    std::vector<uint8_t> head(dfc::head_bytes(sz, off), 0);
    dfc::container_header(head.data(), p, n, total_bits, L.n_chunks, L.n_blocks, rows, cols, sz, off, blob_bytes, len);

    // 3. zero the container (all but the raw bytes' whole 16-byte groups,
    // which the packer writes), upload the header, pack
    uint8_t *dst = static_cast<uint8_t *>(dst_dev);
    auto zero = [&](uint64_t from, uint64_t to) {
        if (to > from)
            hipLaunchKernelGGL(fill_zero_u32, dim3(uint32_t(std::min<uint64_t>(65535, dfc::ceil_div((to - from) / 4, 256)))),
                               dim3(256), 0, st, reinterpret_cast<uint32_t *>(dst + from), (to - from) / 4);
    };
    zero(0, off[dfc::kRaw]);
    zero(off[dfc::kRaw] + (n & ~uint64_t(15)), blob_bytes);
    if (hipMemcpyAsync(dst, head.data(), head.size(), hipMemcpyHostToDevice, st) != hipSuccess) return DFC_EHIP;
    const uint32_t n_out = uint32_t(n);
    if (hipMemcpyAsync(dst + off[dfc::kBlockout] + 4 * L.n_blocks, &n_out, 4, hipMemcpyHostToDevice, st) !=
        hipSuccess)
        return DFC_EHIP;
    if (n) {
        uint32_t *seg_bits = reinterpret_cast<uint32_t *>(work + ws.segbits_off);
        uint64_t *seg_off = reinterpret_cast<uint64_t *>(work + ws.segoff_off);
        hipLaunchKernelGGL(segment_bits_kernel, dim3(uint32_t(ws.nseg)), dim3(kSegThreads), 0, st, src_dev, n, book,
                           seg_bits);
        hipLaunchKernelGGL(segment_scan_kernel, dim3(1), dim3(1024), 0, st, seg_bits, ws.nseg, seg_off);
        PackArgs a;
        a.src = src_dev;
        a.n = n;
        a.words = reinterpret_cast<uint32_t *>(dst + off[dfc::kWords]);
        a.offw = reinterpret_cast<uint32_t *>(dst + off[dfc::kOffsets]);
        a.blockout = reinterpret_cast<uint32_t *>(dst + off[dfc::kBlockout]);
        a.raw = dst + off[dfc::kRaw];
        a.seg_off = seg_off;
        a.chunk_shift = uint32_t(__builtin_ctz(8u * C));  // C and T are powers of two
        a.lanes_shift = uint32_t(__builtin_ctz(T));
        hipLaunchKernelGGL(pack_kernel, dim3(uint32_t(ws.nseg)), dim3(kSegThreads), 0, st, a, book);
    }
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess) return DFC_EHIP;
    *written = blob_bytes;
    return DFC_OK;
}

}  // extern "C"
