// Mutation check of the container parser (dfc_blob_info) for untrusted input.
//
// Reads one container, then repeatedly applies a few seeded mutations (bit
// flips, overwritten header fields, overwritten words inside the sections,
// truncation) and calls dfc_blob_info on an exactly-sized copy.  Every call
// must return; a container it accepts must have every section inside the
// buffer, with the sizes the decode kernels index without bounds checks
// (block offsets, rANS word offsets and states, panel items).  The wrapper
// test builds this file with AddressSanitizer and UBSan, so a read past the
// buffer or undefined arithmetic in the parser aborts the run.
//
// usage: fuzz_blob_info <container file> <iterations> <seed>
// prints one JSON line of counts; exit status 0 when every check held.
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "dfc.h"

namespace {

uint64_t g_state;

// xorshift64* (Vigna, "An experimental exploration of Marsaglia's xorshift
// generators, scrambled", 2016)
uint64_t next() {
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return g_state * 0x2545F4914F6CDD1Dull;
}

uint32_t below(uint64_t n) { return n ? uint32_t(next() % n) : 0u; }

uint32_t interesting(uint32_t old) {
    switch (below(8)) {
        case 0: return 0u;
        case 1: return 1u;
        case 2: return 0xFFFFFFFFu;
        case 3: return 0x80000000u;
        case 4: return old + 1u;
        case 5: return old - 1u;
        case 6: return old << 1;
        default: return uint32_t(next());
    }
}

bool inside(uint64_t off, uint64_t bytes, uint64_t len) { return off <= len && bytes <= len - off; }

// What an accepted container must satisfy before a kernel may index it.
const char *check_accepted(const dfc_info &in, const uint8_t *blob, uint64_t len) {
    if (in.blob_bytes > len) return "blob_bytes";
    if (!inside(in.off_tables, in.tables_bytes, len)) return "tables";
    if (!inside(in.off_words, in.words_bytes, len)) return "words";
    if (!inside(in.off_offsets, in.offsets_bytes, len)) return "offsets";
    if (!inside(in.off_blockout, in.blockout_bytes, len)) return "blockout";
    if (!inside(in.off_raw, in.raw_bytes, len)) return "raw";
    if (in.n == 0) return nullptr;
    if (in.raw_bytes < in.n) return "raw size";
    if (in.layout == DFC_LAYOUT_ANS) {
        if (in.offsets_bytes < 4 * (in.n_blocks + 1)) return "ans offsets size";
        if (in.blockout_bytes < 256 * in.n_blocks) return "ans states size";
        if (uint64_t(64) * in.ans_steps * in.n_blocks < in.n) return "ans blocks";
        // per-block first 16-bit word: monotone from 0, inside the words
        uint32_t prev = 0;
        for (uint64_t b = 0; b <= in.n_blocks; ++b) {
            uint32_t v;
            std::memcpy(&v, blob + in.off_offsets + 4 * b, 4);
            if ((b == 0 && v != 0) || v < prev) return "ans word offsets";
            prev = v;
        }
        if (2ull * prev > in.words_bytes) return "ans word offsets end";
    } else {
        if (in.blockout_bytes < 4 * (in.n_blocks + 1)) return "blockout size";
        if (in.lanes_per_block == 0 || in.n_chunks > in.n_blocks * in.lanes_per_block) return "chunks";
        if (in.layout != DFC_LAYOUT_PANEL && in.n_chunks != in.n_blocks * in.lanes_per_block) return "chunks";
        if (in.words_bytes < in.n_chunks * in.chunk_bytes) return "words size";
    }
    if (in.layout == DFC_LAYOUT_PANEL) {
        if (!inside(in.off_panels, in.panels_bytes, len)) return "panels";
        if (in.panels_bytes < 16 * (in.n_items + 1)) return "panels size";
        if (in.rows * in.cols != in.n) return "shape";
        // item q covers chunks [c_q, c_q+1) and blocks [b_q, b_q+1): both
        // monotone, from 0 to n_chunks and n_blocks
        uint32_t c_prev = 0, b_prev = 0;
        for (uint64_t q = 0; q <= in.n_items; ++q) {
            uint32_t c, b;
            std::memcpy(&c, blob + in.off_panels + 16 * q, 4);
            std::memcpy(&b, blob + in.off_panels + 16 * q + 4, 4);
            if ((q == 0 && (c != 0 || b != 0)) || c < c_prev || b < b_prev) return "item order";
            c_prev = c;
            b_prev = b;
        }
        if (c_prev != in.n_chunks || b_prev != in.n_blocks) return "item end";
    }
    // block offsets (output element before each block) run from 0 to n
    if (in.layout != DFC_LAYOUT_ANS) {
        uint32_t prev = 0;
        for (uint64_t b = 0; b <= in.n_blocks; ++b) {
            uint32_t v;
            std::memcpy(&v, blob + in.off_blockout + 4 * b, 4);
            if ((b == 0 && v != 0) || v < prev || v - prev > in.max_block_elems) return "block offsets";
            prev = v;
        }
        if (prev != in.n) return "block offsets end";
    }
    return nullptr;
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 4) {
        std::fprintf(stderr, "usage: %s <container> <iterations> <seed>\n", argv[0]);
        return 2;
    }
    std::FILE *f = std::fopen(argv[1], "rb");
    if (!f) return 2;
    std::vector<uint8_t> blob;
    uint8_t buf[1 << 16];
    for (size_t k; (k = std::fread(buf, 1, sizeof(buf), f)) > 0;) blob.insert(blob.end(), buf, buf + k);
    std::fclose(f);
    const long iters = std::atol(argv[2]);
    g_state = std::strtoull(argv[3], nullptr, 10) * 0x9E3779B97F4A7C15ull + 1;

    dfc_info base;
    if (dfc_blob_info(blob.data(), blob.size(), &base) != DFC_OK) {
        std::fprintf(stderr, "the unmutated container is rejected\n");
        return 1;
    }
    const uint64_t sec_off[5] = {base.off_tables, base.off_words, base.off_offsets, base.off_blockout, base.off_raw};
    const uint64_t sec_len[5] = {base.tables_bytes, base.words_bytes, base.offsets_bytes, base.blockout_bytes,
                                 base.raw_bytes};

    long accepted = 0, rejected = 0, failures = 0;
    long by_status[8] = {0};
    for (long it = 0; it < iters; ++it) {
        std::vector<uint8_t> m = blob;
        const int muts = 1 + int(below(4));
        for (int q = 0; q < muts; ++q) {
            switch (below(4)) {
                case 0:  // one bit anywhere
                    m[below(m.size())] ^= uint8_t(1u << below(8));
                    break;
                case 1:  // one byte of the header and code lengths
                    m[below(std::min<size_t>(512, m.size()))] = uint8_t(next());
                    break;
                case 2: {  // one header field
                    const size_t at = 4 * below(std::min<size_t>(512, m.size()) / 4);
                    uint32_t v;
                    std::memcpy(&v, &m[at], 4);
                    v = interesting(v);
                    std::memcpy(&m[at], &v, 4);
                    break;
                }
                default: {  // one word inside a section
                    const int s = int(below(5));
                    if (sec_len[s] < 4) break;
                    const size_t at = sec_off[s] + 4 * below(sec_len[s] / 4);
                    uint32_t v;
                    std::memcpy(&v, &m[at], 4);
                    v = interesting(v);
                    std::memcpy(&m[at], &v, 4);
                    break;
                }
            }
        }
        size_t len = m.size();
        if (below(16) == 0) len = below(m.size() + 1);
        // an exactly-sized heap copy: any read past len is caught
        std::vector<uint8_t> exact(m.begin(), m.begin() + len);
        dfc_info in;
        std::memset(&in, 0xA5, sizeof(in));
        const dfc_status st = dfc_blob_info(len ? exact.data() : nullptr, len, &in);
        if (st == DFC_OK) {
            ++accepted;
            if (const char *why = check_accepted(in, exact.data(), len)) {
                ++failures;
                std::fprintf(stderr, "iteration %ld: accepted container fails '%s'\n", it, why);
            }
        } else {
            ++rejected;
            const int k = -int(st);
            if (k >= 0 && k < 8) ++by_status[k];
            else {
                ++failures;
                std::fprintf(stderr, "iteration %ld: unknown status %d\n", it, int(st));
            }
        }
    }
    std::printf("{\"iterations\": %ld, \"accepted\": %ld, \"rejected\": %ld, \"failures\": %ld, "
                "\"einval\": %ld, \"esize\": %ld, \"ecorrupt\": %ld, \"eunsupported\": %ld}\n",
                iters, accepted, rejected, failures, by_status[1], by_status[2], by_status[3], by_status[4]);
    return failures ? 1 : 0;
}
