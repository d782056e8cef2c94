// dfc_format.h - byte layout of the DFC1 container shared by the host codec
// and the device launcher (internal to libdfc).
//
// Container: 256-byte header, 256 code lengths, then the sections tables
// (empty in the Huffman layouts; the rANS frequencies in the ANS layout),
// words, offsets (empty in the padded layout), blockout, raw (and panels and
// counts, used by the panel layout only), each at the next multiple of 256 bytes,
// zero padding.  Little-endian.  A container holds the code and the coded
// data only: the decode tables are derived from the code by the kernels.
#pragma once

#include <algorithm>
#include <cstdint>
#include <cstring>

namespace dfc {

constexpr uint32_t kMagic = 0x31434644u;  // "DFC1"
constexpr uint32_t kVersion = 1;
constexpr uint64_t kHeaderBytes = 512;     // header + code lengths
constexpr uint32_t kMaxLen = 24;
constexpr uint32_t kGuardWords = 4;
constexpr uint32_t kOffsetBits = 5;

// Header field byte offsets.
namespace hdr {
constexpr int magic = 0, version = 4, n = 8, total_bits = 16, n_chunks = 24, n_blocks = 32;
constexpr int chunk_bytes = 40, lanes = 44, max_code_len = 48, lut_bits = 52, layout = 56;
constexpr int panel_rows = 60, rows = 64, cols = 72, tile_k = 80, reserved = 84;
constexpr int sections = 88;  // 6 x (u64 offset, u64 bytes): tables, words, offsets, blockout, raw, panels
constexpr int blob_bytes = 184;
constexpr int counts = 192;   // (u64 offset, u64 bytes) of the counts section
// Header byte offset of section i's (offset, bytes) pair.
constexpr int section(int i) { return i < 6 ? sections + 16 * i : counts; }
constexpr int lengths = 256;
}  // namespace hdr

enum Section { kTables = 0, kWords, kOffsets, kBlockout, kRaw, kPanels, kCounts, kNumSections };

// LDS image of the decode tables the kernels derive from the code lengths
// for a k-bit first level (see dfc_tables.h; never stored in a container):
// step[2^k] (u32), wsym[2^k] (u64), mask[2^k] (u16), then limit[32],
// first[32], base[32] (u32, index = code length) and order[256] (u8).
constexpr uint32_t kStepEscape = 0xFFFFF000u;
inline uint64_t tables_bytes(uint32_t k) { return 14ull * (1ull << k) + 3 * 128 + 256; }

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
// Bytes per stored chunk count (panel layout): a chunk of 8C bits starts at
// most 8C codes, so one byte up to C = 16 (128 codes), two at C = 32.
inline uint32_t count_width(uint32_t chunk_bytes) { return 8u * chunk_bytes <= 255u ? 1u : 2u; }
inline uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

struct Layout {
    uint64_t n_chunks_used, n_blocks, n_chunks;
};
inline Layout layout_sizes(uint64_t total_bits, uint32_t chunk_bytes, uint32_t lanes) {
    Layout l;
    l.n_chunks_used = ceil_div(total_bits, 8ull * chunk_bytes);
    l.n_blocks = ceil_div(l.n_chunks_used, lanes);
    l.n_chunks = l.n_blocks * lanes;
    return l;
}

struct SectionSizes {
    uint64_t bytes[kNumSections];
};
// with_offsets = false: the padded layout, whose chunks need no offsets.
inline SectionSizes section_sizes(uint64_t n, uint64_t n_chunks, uint64_t n_blocks, uint32_t chunk_bytes,
                                  uint32_t lut_bits, uint64_t n_items = 0, bool with_offsets = true) {
    SectionSizes s;
    s.bytes[kTables] = 0;
    s.bytes[kWords] = 4 * (n_chunks * (chunk_bytes / 4) + kGuardWords);
    s.bytes[kOffsets] = with_offsets ? 4 * (ceil_div(kOffsetBits * (n_chunks + 1), 32) + 1) : 0;
    s.bytes[kBlockout] = 4 * (n_blocks + 1);
    s.bytes[kRaw] = 16 * ceil_div(n, 16);
    s.bytes[kPanels] = n_items ? 16 * (n_items + 1) : 0;
    s.bytes[kCounts] = n_items ? 16 * ceil_div(count_width(chunk_bytes) * n_chunks, 16) : 0;
    return s;
}

// Interleaved rANS layout: 2^12 probability slots, states in [2^16, 2^32),
// 16-bit words, 64 lanes per block.  Sections: tables = f (u16[256]; the
// kernel derives its slot table from them); words = the streams (u16, whole 16-byte units plus one guard unit);
// offsets = the first word of every block (u32, n_blocks + 1); blockout =
// the 64 initial states of every block (u32); raw as in the other layouts.
constexpr uint32_t kAnsProbBits = 12;
constexpr uint32_t kAnsSlots = 1u << kAnsProbBits;
constexpr uint64_t kAnsLow = 1ull << 16;  // states live in [kAnsLow, 2^32)
constexpr uint32_t kAnsLanes = 64;
constexpr uint64_t kAnsTablesBytes = 2 * 256;
inline SectionSizes ans_section_sizes(uint64_t n, uint64_t n_words, uint64_t n_blocks) {
    SectionSizes s;
    s.bytes[kTables] = kAnsTablesBytes;
    s.bytes[kWords] = 2 * (ceil_div(n_words, 8) * 8 + 8);
    s.bytes[kOffsets] = 4 * (n_blocks + 1);
    s.bytes[kBlockout] = 4ull * kAnsLanes * n_blocks;
    s.bytes[kRaw] = 16 * ceil_div(n, 16);
    s.bytes[kPanels] = 0;
    s.bytes[kCounts] = 0;
    return s;
}

// Panel layout geometry: items of 32 rows x panel_k columns, row panels
// first, then column slices.  The counts section holds, per chunk
// (count_width bytes), the number of codes whose first bit lies in that chunk.
constexpr uint32_t kPanelRows = 32;
constexpr uint32_t kSubtileK = 16;
struct PanelGeom {
    uint64_t rows, cols, panel_k, slices, n_items;
    uint64_t item_row0(uint64_t q) const { return kPanelRows * (q / slices); }
    uint64_t item_col0(uint64_t q) const { return panel_k * (q % slices); }
    uint64_t item_width(uint64_t q) const { return std::min<uint64_t>(panel_k, cols - item_col0(q)); }
    uint64_t item_elem0(uint64_t q) const { return kPanelRows * (item_row0(q) / kPanelRows * cols + item_col0(q)); }
    // Row-major source index of element i of item q.
    uint64_t source(uint64_t q, uint64_t i) const {
        const uint64_t t = i >> 9, l = (i >> 3) & 63, j = i & 7;
        return (item_row0(q) + (l & 31)) * cols + item_col0(q) + kSubtileK * t + 8 * (l >> 5) + j;
    }
};
inline bool panel_geom(uint64_t rows, uint64_t cols, uint64_t panel_k, PanelGeom &g) {
    if (!rows || !cols || rows % kPanelRows || cols % kSubtileK || !panel_k || panel_k % kSubtileK) return false;
    g.rows = rows;
    g.cols = cols;
    g.panel_k = panel_k;
    g.slices = ceil_div(cols, panel_k);
    g.n_items = rows / kPanelRows * g.slices;
    return true;
}

// Places the sections after the header; returns the container size.
inline uint64_t place_sections(const SectionSizes &s, uint64_t off[kNumSections]) {
    uint64_t pos = kHeaderBytes;
    for (int i = 0; i < kNumSections; ++i) {
        pos = align256(pos);
        off[i] = s.bytes[i] ? pos : 0;
        pos += s.bytes[i];
    }
    return align256(pos);
}

// Bytes from the container's start through the end of its tables section
// (at least the header and code lengths): what a host writes before the data.
inline uint64_t head_bytes(const SectionSizes &s, const uint64_t off[kNumSections]) {
    return std::max<uint64_t>(kHeaderBytes, off[kTables] + s.bytes[kTables]);
}

template <typename T>
inline T load_le(const uint8_t *p) {
    T v;
    std::memcpy(&v, p, sizeof(T));  // little-endian host (x86-64)
    return v;
}
template <typename T>
inline void store_le(uint8_t *p, T v) {
    std::memcpy(p, &v, sizeof(T));
}

}  // namespace dfc
