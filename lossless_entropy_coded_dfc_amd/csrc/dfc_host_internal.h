// dfc_host_internal.h - host-side codec steps of libdfc shared by the host
// encoder and the device encoder's launcher (internal to libdfc).
#pragma once

#include <algorithm>
#include <cstdint>
#include <thread>
#include <vector>

#include "dfc.h"
#include "dfc_format.h"

namespace dfc {

// Host worker threads for `work` elements: the request (0 = hardware threads,
// at most 16), and no more than one per ~1M elements.
inline unsigned pick_threads(uint32_t requested, uint64_t work) {
    unsigned hw = std::thread::hardware_concurrency();
    if (hw == 0) hw = 1;
    uint64_t t = requested ? requested : std::min(hw, 16u);
    uint64_t by_work = std::max<uint64_t>(1, work >> 20);  // >= ~1M elements per thread
    return unsigned(std::max<uint64_t>(1, std::min(t, by_work)));
}

template <class F>
void parallel_for(unsigned nt, F &&f) {
    if (nt <= 1) {
        f(0u);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(nt - 1);
    for (unsigned t = 1; t < nt; ++t) pool.emplace_back([&f, t] { f(t); });
    f(0u);
    for (auto &th : pool) th.join();
}

inline uint32_t exponent_of(uint16_t b) { return (b >> 7) & 0xFFu; }
inline uint8_t raw_of(uint16_t b) { return uint8_t(((b >> 8) & 0x80u) | (b & 0x7Fu)); }

inline void histogram_mt(const uint16_t *src, uint64_t n, uint64_t hist[256], unsigned nt) {
    std::vector<uint64_t> local(size_t(nt) * 256, 0);
    parallel_for(nt, [&](unsigned t) {
        uint64_t j0 = n * t / nt, j1 = n * (t + 1) / nt;
        uint64_t *h = &local[size_t(t) * 256];
        for (uint64_t j = j0; j < j1; ++j) h[exponent_of(src[j])]++;
    });
    for (int s = 0; s < 256; ++s) {
        uint64_t v = 0;
        for (unsigned t = 0; t < nt; ++t) v += local[size_t(t) * 256 + s];
        hist[s] = v;
    }
}

// Length-limited optimal code lengths (package-merge) for a histogram.
dfc_status code_lengths(const uint64_t hist[256], uint32_t limit, uint8_t len[256]);
// Canonical codes (RFC 1951 section 3.2.2) for code lengths.
void canonical_codes(const uint8_t len[256], uint32_t code[256]);
// Automatic chunk size of the flat layout: the first of 16, 32, 8, 4 bytes
// whose coded size is within 2% of the exponent-entropy bound, else the
// smallest container.
uint32_t choose_chunk_bytes(const uint64_t hist[256], const uint8_t len[256], uint32_t lanes);
// Encoder parameters in range.
bool encoder_params_ok(const dfc_params &p);
// Kraft sum of the lengths scaled by 2^24 (2^24 for a complete code).
uint64_t kraft_sum(const uint8_t len[256]);
// Header, code lengths and derived decode tables of a container.
void container_header(uint8_t *dst, const dfc_params &p, uint64_t n, uint64_t total_bits, uint64_t n_chunks,
                      uint64_t n_blocks, uint64_t rows, uint64_t cols, const SectionSizes &sz,
                      const uint64_t off[kNumSections], uint64_t blob_bytes, const uint8_t len[256]);

// Interleaved rANS layout (DFC_LAYOUT_ANS): encoder, size bound and
// container validation (the header fields shared with the other layouts are
// read by dfc_blob_info before it calls ans_blob_info).
dfc_status encode_ans(const uint16_t *src, uint64_t n, const dfc_params &p, uint64_t rows, uint64_t cols,
                      uint8_t *dst, uint64_t cap, uint64_t *written);
uint64_t ans_encode_bound(uint64_t n, uint32_t steps);
uint32_t ans_steps_or_default(uint32_t s);
// Frequencies summing to 2^12 from a histogram, and their cumulative sums.
void ans_frequencies(const uint64_t hist[256], uint32_t f[256], uint32_t cum[256]);
// Header and tables section of an ANS container (dst zeroed at least up to
// the end of the tables section).
void ans_container_head(uint8_t *dst, uint64_t n, uint64_t nw, uint64_t nb, uint32_t S, uint64_t rows,
                        uint64_t cols, const SectionSizes &sz, const uint64_t off[kNumSections], uint64_t blob_bytes,
                        const uint32_t f[256]);
dfc_status ans_blob_info(const uint8_t *b, uint64_t bytes, dfc_info &in);

}  // namespace dfc
