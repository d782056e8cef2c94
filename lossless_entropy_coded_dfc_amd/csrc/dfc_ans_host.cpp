// dfc_ans_host.cpp - host half of the interleaved rANS layout (DFC_LAYOUT_ANS):
// frequency quantisation, the block encoder and container validation.
//
// The exponent bytes are coded with range asymmetric numeral systems, an
// arithmetic-family entropy code (DFloat11 blog, section 02, names Huffman-
// and arithmetic-like coding; the VcLLM page's introduction describes an
// ANS-based decoder).  Sign and mantissa stay one raw byte as in the other
// layouts.  dfc.h states the code and the container; the encoder below runs
// each block's elements backwards (steps from last to first, lanes from 63
// down to 0, every lane starting from the state 2^16) so that the decoder
// reads the block's words forwards, lane by lane within each step.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "dfc.h"
#include "dfc_format.h"
#include "dfc_host_internal.h"

namespace dfc {
namespace {

// Frequencies summing to 2^12: proportional shares rounded down (at least 1
// for a present symbol), the missing units to the largest fractional parts
// (smaller symbol first on ties), an excess taken back one unit at a time from
// the largest share (smaller symbol first on ties).
void quantize(const uint64_t hist[256], uint32_t f[256]) {
    uint64_t total = 0;
    for (int s = 0; s < 256; ++s) total += hist[s];
    std::memset(f, 0, 256 * sizeof(uint32_t));
    if (!total) return;
    int64_t sum = 0;
    std::vector<int> present;
    for (int s = 0; s < 256; ++s) {
        if (!hist[s]) continue;
        present.push_back(s);
        f[s] = uint32_t(std::max<uint64_t>(1, hist[s] * kAnsSlots / total));
        sum += f[s];
    }
    int64_t d = int64_t(kAnsSlots) - sum;
    if (d > 0) {
        std::vector<int> order = present;
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
            const uint64_t ra = hist[a] * kAnsSlots % total, rb = hist[b] * kAnsSlots % total;
            return ra != rb ? ra > rb : a < b;
        });
        for (int64_t k = 0; k < d; ++k) f[order[size_t(k)]]++;
    }
    for (; d < 0; ++d) {
        int best = present[0];
        for (int s : present)
            if (f[s] > f[best]) best = s;  // first of the largest: smaller symbol on ties
        f[best]--;
    }
}

void cumulative(const uint32_t f[256], uint32_t cum[256]) {
    uint32_t c = 0;
    for (int s = 0; s < 256; ++s) {
        cum[s] = c;
        c += f[s];
    }
}

// One block of cnt elements: initial decoder states and words in decode order.
void encode_block(const uint16_t *src, uint64_t cnt, const uint32_t f[256], const uint32_t cum[256],
                  uint32_t states[kAnsLanes], std::vector<uint16_t> &words) {
    uint64_t x[kAnsLanes];
    for (uint32_t l = 0; l < kAnsLanes; ++l) x[l] = kAnsLow;
    words.clear();
    const uint64_t steps = ceil_div(cnt, kAnsLanes);
    for (uint64_t i = steps; i-- > 0;) {
        for (uint32_t l = kAnsLanes; l-- > 0;) {
            const uint64_t j = i * kAnsLanes + l;
            if (j >= cnt) continue;
            const uint32_t s = exponent_of(src[j]);
            const uint64_t fs = f[s];
            uint64_t v = x[l];
            if (v >= fs << (32 - kAnsProbBits)) {
                words.push_back(uint16_t(v & 0xFFFFu));
                v >>= 16;
            }
            x[l] = (v / fs) * kAnsSlots + v % fs + cum[s];
        }
    }
    std::reverse(words.begin(), words.end());
    for (uint32_t l = 0; l < kAnsLanes; ++l) states[l] = uint32_t(x[l]);
}

}  // namespace

uint32_t ans_steps_or_default(uint32_t s) { return s ? s : uint32_t(DFC_ANS_STEPS_DEFAULT); }

void ans_frequencies(const uint64_t hist[256], uint32_t f[256], uint32_t cum[256]) {
    quantize(hist, f);
    cumulative(f, cum);
}

void ans_container_head(uint8_t *dst, uint64_t n, uint64_t nw, uint64_t nb, uint32_t S, uint64_t rows,
                        uint64_t cols, const SectionSizes &sz, const uint64_t off[kNumSections], uint64_t blob_bytes,
                        const uint32_t f[256]) {
    store_le<uint32_t>(dst + hdr::magic, kMagic);
    store_le<uint32_t>(dst + hdr::version, kVersion);
    store_le<uint64_t>(dst + hdr::n, n);
    store_le<uint64_t>(dst + hdr::total_bits, 16 * nw);
    store_le<uint64_t>(dst + hdr::n_chunks, 0);
    store_le<uint64_t>(dst + hdr::n_blocks, nb);
    store_le<uint32_t>(dst + hdr::lanes, kAnsLanes);
    store_le<uint32_t>(dst + hdr::lut_bits, kAnsProbBits);
    store_le<uint32_t>(dst + hdr::layout, DFC_LAYOUT_ANS);
    store_le<uint64_t>(dst + hdr::rows, rows);
    store_le<uint64_t>(dst + hdr::cols, cols);
    store_le<uint32_t>(dst + hdr::tile_k, S);
    for (int i = 0; i < kNumSections; ++i) {
        store_le<uint64_t>(dst + hdr::section(i), off[i]);
        store_le<uint64_t>(dst + hdr::section(i) + 8, sz.bytes[i]);
    }
    store_le<uint64_t>(dst + hdr::blob_bytes, blob_bytes);
    uint8_t *tab = dst + off[kTables];
    for (int s = 0; s < 256; ++s) store_le<uint16_t>(tab + 2 * s, uint16_t(f[s]));
}

uint64_t ans_encode_bound(uint64_t n, uint32_t steps) {
    const uint64_t nb = ceil_div(n, uint64_t(kAnsLanes) * ans_steps_or_default(steps));
    uint64_t off[kNumSections];
    return place_sections(ans_section_sizes(n, n, nb), off);  // at most one word per element
}

dfc_status encode_ans(const uint16_t *src, uint64_t n, const dfc_params &p, uint64_t rows, uint64_t cols,
                      uint8_t *dst, uint64_t cap, uint64_t *written) {
    const uint32_t S = ans_steps_or_default(p.ans_steps);
    const uint64_t per = uint64_t(kAnsLanes) * S;
    const uint64_t nb = ceil_div(n, per);
    const unsigned nt = unsigned(std::min<uint64_t>(pick_threads(p.threads, n), std::max<uint64_t>(nb, 1)));
    uint64_t hist[256];
    histogram_mt(src, n, hist, nt);
    uint32_t f[256], cum[256];
    ans_frequencies(hist, f, cum);

    // Pass 1: every block's states and words.
    std::vector<uint32_t> states(nb * kAnsLanes);
    std::vector<std::vector<uint16_t>> words(nb);
    parallel_for(nt, [&](unsigned t) {
        for (uint64_t b = nb * t / nt; b < nb * (t + 1) / nt; ++b)
            encode_block(src + b * per, std::min(per, n - b * per), f, cum, &states[b * kAnsLanes], words[b]);
    });
    std::vector<uint64_t> first(nb + 1, 0);
    for (uint64_t b = 0; b < nb; ++b) first[b + 1] = first[b] + words[b].size();
    const uint64_t nw = first[nb];
    if (nw >= (uint64_t(1) << 32)) return DFC_ESIZE;

    // Pass 2: the container.
    const SectionSizes sz = ans_section_sizes(n, nw, nb);
    uint64_t off[kNumSections];
    const uint64_t blob_bytes = place_sections(sz, off);
    if (cap < blob_bytes) return DFC_ESIZE;
    std::memset(dst, 0, blob_bytes);
    ans_container_head(dst, n, nw, nb, S, rows, cols, sz, off, blob_bytes, f);
    uint8_t *wd = dst + off[kWords], *ofs = dst + off[kOffsets], *st = dst + off[kBlockout], *raw = dst + off[kRaw];
    for (uint64_t b = 0; b <= nb; ++b) store_le<uint32_t>(ofs + 4 * b, uint32_t(first[b]));
    parallel_for(nt, [&](unsigned t) {
        for (uint64_t b = nb * t / nt; b < nb * (t + 1) / nt; ++b) {
            if (!words[b].empty()) std::memcpy(wd + 2 * first[b], words[b].data(), 2 * words[b].size());
            std::memcpy(st + 4 * b * kAnsLanes, &states[b * kAnsLanes], 4 * kAnsLanes);
            const uint64_t j1 = std::min(n, (b + 1) * per);
            for (uint64_t j = b * per; j < j1; ++j) raw[j] = raw_of(src[j]);
        }
    });
    *written = blob_bytes;
    return DFC_OK;
}

dfc_status ans_blob_info(const uint8_t *b, uint64_t bytes, dfc_info &in) {
    const uint32_t S = load_le<uint32_t>(b + hdr::tile_k);
    if (in.chunk_bytes != 0 || in.lanes_per_block != kAnsLanes || in.max_code_len != 0 ||
        in.lut_bits != kAnsProbBits || load_le<uint32_t>(b + hdr::panel_rows) || load_le<uint32_t>(b + hdr::reserved))
        return DFC_ECORRUPT;
    if (S < 8 || S > 65536 || S % 8) return DFC_ECORRUPT;
    for (int i = 192; i < 512; ++i)  // header tail and the (unused) code-length area
        if (b[i]) return DFC_ECORRUPT;
    if (in.n >= (uint64_t(1) << 32) || in.rows * in.cols != in.n) return DFC_ECORRUPT;
    const uint64_t per = uint64_t(kAnsLanes) * S;
    if (in.n_chunks != 0 || in.n_blocks != ceil_div(in.n, per) || in.total_bits % 16) return DFC_ECORRUPT;
    const uint64_t nw = in.total_bits / 16;
    if (nw > in.n) return DFC_ECORRUPT;
    const SectionSizes sz = ans_section_sizes(in.n, nw, in.n_blocks);
    uint64_t off[kNumSections];
    const uint64_t blob_bytes = place_sections(sz, off);
    if (blob_bytes != in.blob_bytes) return DFC_ECORRUPT;
    for (int i = 0; i < kNumSections; ++i) {
        if (load_le<uint64_t>(b + hdr::section(i)) != off[i]) return DFC_ECORRUPT;
        if (load_le<uint64_t>(b + hdr::section(i) + 8) != sz.bytes[i]) return DFC_ECORRUPT;
    }
    if (bytes < blob_bytes) return DFC_ESIZE;

    // frequencies (the decoder derives its slot table from them)
    uint32_t f[256];
    uint64_t fsum = 0;
    uint32_t used = 0;
    for (int s = 0; s < 256; ++s) {
        f[s] = load_le<uint16_t>(b + off[kTables] + 2 * s);
        fsum += f[s];
        used += f[s] != 0;
    }
    if (fsum != (in.n ? kAnsSlots : 0)) return DFC_ECORRUPT;
    // block word offsets: from 0 to the stream length, at most one word per element
    const uint8_t *ofs = b + off[kOffsets];
    if (load_le<uint32_t>(ofs) != 0 || load_le<uint32_t>(ofs + 4 * in.n_blocks) != nw) return DFC_ECORRUPT;
    for (uint64_t k = 0; k < in.n_blocks; ++k) {
        const uint32_t a = load_le<uint32_t>(ofs + 4 * k), c = load_le<uint32_t>(ofs + 4 * k + 4);
        if (c < a || c - a > std::min(per, in.n - k * per)) return DFC_ECORRUPT;
    }
    // initial states in [2^16, 2^32)
    const uint8_t *st = b + off[kBlockout];
    for (uint64_t k = 0; k < in.n_blocks * kAnsLanes; ++k)
        if (load_le<uint32_t>(st + 4 * k) < kAnsLow) return DFC_ECORRUPT;

    in.n_used = used;
    in.min_len = in.max_len = 0;
    in.max_block_elems = uint32_t(std::min(per, in.n));
    in.ans_steps = S;
    in.ans_prob_bits = kAnsProbBits;
    in.off_tables = off[kTables];
    in.tables_bytes = sz.bytes[kTables];
    in.off_words = off[kWords];
    in.words_bytes = sz.bytes[kWords];
    in.off_offsets = off[kOffsets];
    in.offsets_bytes = sz.bytes[kOffsets];
    in.off_blockout = off[kBlockout];
    in.blockout_bytes = sz.bytes[kBlockout];
    in.off_raw = off[kRaw];
    in.raw_bytes = sz.bytes[kRaw];
    // header + frequencies + streams, offsets, states, raw
    in.coded_bytes = kHeaderBytes + sz.bytes[kTables] + sz.bytes[kWords] + sz.bytes[kOffsets] + sz.bytes[kBlockout] + sz.bytes[kRaw];
    return DFC_OK;
}

}  // namespace dfc
