// dfc_host.cpp - host half of libdfc: exponent histogram, length-limited
// canonical Huffman codebook, multithreaded encoder and container validation.
//
// DFloat11 blog ("70% Size, 100% Accuracy ... (DFloat11)"), section 02:
// frequent values get short codes and rare values long ones; section 03
// item 2: decoding threads coordinate through small per-chunk and per-block
// position variables, which this encoder writes.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "dfc.h"
#include "dfc_format.h"
#include "dfc_host_internal.h"

using namespace dfc;

namespace {

// Canonical per-length tables (index = length 1..24).
struct Canon {
    uint32_t count[kMaxLen + 1], first[kMaxLen + 1], limit[kMaxLen + 1], base[kMaxLen + 1];
    uint8_t order[256];
    uint32_t n_used;
};

void canonical(const uint8_t len[256], Canon &c, uint32_t code[256]) {
    std::memset(&c, 0, sizeof(c));
    for (int s = 0; s < 256; ++s)
        if (len[s]) c.count[len[s]]++;
    uint32_t seen = 0;
    for (uint32_t l = 1; l <= kMaxLen; ++l) {
        c.first[l] = l == 1 ? 0u : (c.first[l - 1] + c.count[l - 1]) << 1;
        c.limit[l] = (c.first[l] + c.count[l]) << (kMaxLen - l);
        c.base[l] = seen;
        seen += c.count[l];
    }
    c.n_used = seen;
    uint32_t next[kMaxLen + 1];
    std::memcpy(next, c.first, sizeof(next));
    uint32_t fill[kMaxLen + 1] = {0};
    for (int s = 0; s < 256; ++s) {
        uint32_t l = len[s];
        if (!l) {
            if (code) code[s] = 0;
            continue;
        }
        if (code) code[s] = next[l]++;
        c.order[c.base[l] + fill[l]++] = uint8_t(s);  // increasing symbol within a length
    }
}

// Package-merge (coin-collector form) with deterministic tie-breaks.
struct PMItem {
    uint64_t w;
    uint32_t kind;   // 0 = leaf, 1 = package
    uint32_t order;  // leaf rank or package index
    int32_t a, b;    // children in the previous level (packages)
    int32_t sym;     // symbol (leaves)
};

dfc_status package_merge(const uint64_t hist[256], uint32_t limit, uint8_t len[256]) {
    std::memset(len, 0, 256);
    std::vector<int> used;
    for (int s = 0; s < 256; ++s)
        if (hist[s]) used.push_back(s);
    const size_t m = used.size();
    if (m == 0) return DFC_OK;
    if (m == 1) {
        len[used[0]] = 1;
        len[(used[0] + 1) & 255] = 1;
        return DFC_OK;
    }
    if (m > (size_t(1) << limit)) return DFC_ESIZE;
    std::sort(used.begin(), used.end(), [&](int x, int y) {
        return hist[x] != hist[y] ? hist[x] < hist[y] : x < y;
    });
    std::vector<PMItem> leaves(m);
    for (size_t r = 0; r < m; ++r) leaves[r] = {hist[used[r]], 0u, uint32_t(r), -1, -1, used[r]};
    auto less = [](const PMItem &x, const PMItem &y) {
        if (x.w != y.w) return x.w < y.w;
        if (x.kind != y.kind) return x.kind < y.kind;
        return x.order < y.order;
    };
    std::vector<std::vector<PMItem>> level(limit);
    level[0] = leaves;
    for (uint32_t l = 1; l < limit; ++l) {
        const auto &prev = level[l - 1];
        std::vector<PMItem> cur = leaves;
        for (size_t j = 0; j + 1 < prev.size(); j += 2)
            cur.push_back({prev[j].w + prev[j + 1].w, 1u, uint32_t(j / 2), int32_t(j), int32_t(j + 1), -1});
        std::sort(cur.begin(), cur.end(), less);
        level[l] = std::move(cur);
    }
    uint32_t cnt[256] = {0};
    std::vector<std::pair<int, int>> stack;
    for (size_t i = 0; i < 2 * m - 2; ++i) stack.push_back({int(limit - 1), int(i)});
    while (!stack.empty()) {
        auto [l, i] = stack.back();
        stack.pop_back();
        const PMItem &it = level[l][i];
        if (it.kind == 0) {
            cnt[it.sym]++;
        } else {
            stack.push_back({l - 1, it.a});
            stack.push_back({l - 1, it.b});
        }
    }
    for (int s = 0; s < 256; ++s) len[s] = uint8_t(cnt[s]);
    return DFC_OK;
}

// Encoder parameters; chunk_bytes 0 (automatic) only when auto_chunk.
bool params_ok(const dfc_params &p, bool auto_chunk = true) {
    const uint32_t C = p.chunk_bytes, T = p.lanes_per_block;
    if (C != 4 && C != 8 && C != 16 && C != 32 && !(auto_chunk && C == 0)) return false;
    // one wavefront (64 lanes) decodes a block: the only block width the
    // decoders take, so the only one written
    if (T != 64) return false;
    if (p.max_code_len < 1 || p.max_code_len > kMaxLen) return false;
    if (p.lut_bits < 8 || p.lut_bits > 12) return false;
    if (p.layout != DFC_LAYOUT_FLAT && p.layout != DFC_LAYOUT_PANEL && p.layout != DFC_LAYOUT_PADDED &&
        p.layout != DFC_LAYOUT_ANS)
        return false;
    if (p.layout == DFC_LAYOUT_ANS) {
        if (T != kAnsLanes) return false;
        if (p.ans_steps && (p.ans_steps < 8 || p.ans_steps > 65536 || p.ans_steps % 8)) return false;
    } else if (p.ans_steps) {
        return false;
    }
    return true;
}

// Header and code lengths of a container (sections zeroed).
void write_header(uint8_t *dst, const dfc_params &p, uint64_t n, uint64_t total_bits, uint64_t n_chunks,
                  uint64_t n_blocks, uint64_t rows, uint64_t cols, const SectionSizes &sz,
                  const uint64_t off[kNumSections], uint64_t blob_bytes, const uint8_t len[256]) {
    store_le<uint32_t>(dst + hdr::magic, kMagic);
    store_le<uint32_t>(dst + hdr::version, kVersion);
    store_le<uint64_t>(dst + hdr::n, n);
    store_le<uint64_t>(dst + hdr::total_bits, total_bits);
    store_le<uint64_t>(dst + hdr::n_chunks, n_chunks);
    store_le<uint64_t>(dst + hdr::n_blocks, n_blocks);
    store_le<uint32_t>(dst + hdr::chunk_bytes, p.chunk_bytes);
    store_le<uint32_t>(dst + hdr::lanes, p.lanes_per_block);
    store_le<uint32_t>(dst + hdr::max_code_len, p.max_code_len);
    store_le<uint32_t>(dst + hdr::lut_bits, p.lut_bits);
    store_le<uint32_t>(dst + hdr::layout, p.layout);
    store_le<uint32_t>(dst + hdr::panel_rows, p.layout == DFC_LAYOUT_PANEL ? kPanelRows : 0);
    store_le<uint64_t>(dst + hdr::rows, rows);
    store_le<uint64_t>(dst + hdr::cols, cols);
    store_le<uint32_t>(dst + hdr::tile_k, p.layout == DFC_LAYOUT_PANEL ? p.panel_k : 0);
    for (int i = 0; i < kNumSections; ++i) {
        store_le<uint64_t>(dst + hdr::section(i), off[i]);
        store_le<uint64_t>(dst + hdr::section(i) + 8, sz.bytes[i]);
    }
    store_le<uint64_t>(dst + hdr::blob_bytes, blob_bytes);
    std::memcpy(dst + hdr::lengths, len, 256);
}

void zero_parallel(uint8_t *dst, uint64_t bytes, uint32_t threads) {
    const unsigned zt = pick_threads(threads, bytes / 4);
    parallel_for(zt, [&](unsigned t) {
        uint64_t a = bytes * t / zt, b = bytes * (t + 1) / zt;
        std::memset(dst + a, 0, b - a);
    });
}

// 5-bit offset fields, little-endian bit order.
void pack_offsets(const std::vector<uint8_t> &offs, uint8_t *ow) {
    for (uint64_t i = 0; i < offs.size(); ++i) {
        const uint64_t g = kOffsetBits * i;
        const uint64_t v = uint64_t(offs[i]) << (g & 31);
        uint8_t *w0 = ow + 4 * (g >> 5);
        store_le<uint32_t>(w0, load_le<uint32_t>(w0) | uint32_t(v));
        if (v >> 32) store_le<uint32_t>(w0 + 4, load_le<uint32_t>(w0 + 4) | uint32_t(v >> 32));
    }
}

// Panel layout: every item is packed on its own, from a fresh chunk, with
// its own blocks (see dfc.h).  Items are independent, so threads take whole
// items and never share a stream word.
dfc_status encode_panel(const uint16_t *src, uint64_t n, const dfc_params &p, const uint8_t len[256],
                        const uint32_t code[256], uint8_t *dst, uint64_t cap, uint64_t *written) {
    PanelGeom g;
    if (!panel_geom(p.rows, p.cols, p.panel_k, g) || g.rows * g.cols != n) return DFC_EINVAL;
    const uint32_t C = p.chunk_bytes, T = p.lanes_per_block;
    const uint64_t chunk_bits = 8ull * C;
    const unsigned nt = unsigned(std::min<uint64_t>(pick_threads(p.threads, n), g.n_items));
    // Pass 1: code bits per item.
    std::vector<uint64_t> bits(g.n_items, 0);
    parallel_for(nt, [&](unsigned t) {
        for (uint64_t q = g.n_items * t / nt; q < g.n_items * (t + 1) / nt; ++q) {
            const uint64_t nq = kPanelRows * g.item_width(q);
            uint64_t b = 0;
            for (uint64_t i = 0; i < nq; ++i) b += len[exponent_of(src[g.source(q, i)])];
            bits[q] = b;
        }
    });
    std::vector<uint64_t> first_chunk(g.n_items + 1, 0), first_block(g.n_items + 1, 0);
    uint64_t total_bits = 0;
    for (uint64_t q = 0; q < g.n_items; ++q) {
        const uint64_t chunks = ceil_div(bits[q], chunk_bits);
        first_chunk[q + 1] = first_chunk[q] + chunks;
        first_block[q + 1] = first_block[q] + ceil_div(chunks, T);
        total_bits += bits[q];
    }
    const uint64_t n_chunks = first_chunk[g.n_items], n_blocks = first_block[g.n_items];
    if (n_chunks >= (uint64_t(1) << 32) || n_blocks >= (uint64_t(1) << 32)) return DFC_ESIZE;
    SectionSizes sz = section_sizes(n, n_chunks, n_blocks, C, p.lut_bits, g.n_items);
    uint64_t off[kNumSections];
    const uint64_t blob_bytes = place_sections(sz, off);
    if (cap < blob_bytes) return DFC_ESIZE;
    zero_parallel(dst, blob_bytes, p.threads);
    write_header(dst, p, n, total_bits, n_chunks, n_blocks, g.rows, g.cols, sz, off, blob_bytes, len);

    uint8_t *words = dst + off[kWords];
    uint8_t *raw = dst + off[kRaw];
    uint8_t *blockout = dst + off[kBlockout];
    uint8_t *panels = dst + off[kPanels];
    uint8_t *counts = dst + off[kCounts];
    const uint32_t cw = count_width(C);
    std::vector<uint8_t> offs(n_chunks + 1, 0);
    // Pass 2: pack every item.
    parallel_for(nt, [&](unsigned t) {
        for (uint64_t q = g.n_items * t / nt; q < g.n_items * (t + 1) / nt; ++q) {
            const uint64_t nq = kPanelRows * g.item_width(q), e0 = g.item_elem0(q);
            const uint64_t c0 = first_chunk[q], b0 = first_block[q], chunks = first_chunk[q + 1] - c0;
            uint8_t *w = words + 4 * c0 * (C / 4);
            uint64_t pos = 0, acc = 0, wi = 0, ci = 0;
            uint32_t nacc = 0;
            for (uint64_t i = 0; i < nq; ++i) {
                const uint16_t b = src[g.source(q, i)];
                const uint32_t e = exponent_of(b);
                raw[e0 + i] = raw_of(b);
                while (ci < chunks && ci * chunk_bits <= pos) {
                    offs[c0 + ci] = uint8_t(pos - ci * chunk_bits);
                    if (ci % T == 0) store_le<uint32_t>(blockout + 4 * (b0 + ci / T), uint32_t(e0 + i));
                    ++ci;
                }
                const uint32_t l = len[e];
                if (cw == 1) {
                    ++counts[c0 + pos / chunk_bits];
                } else {
                    uint8_t *cnt = counts + 2 * (c0 + pos / chunk_bits);
                    store_le<uint16_t>(cnt, uint16_t(load_le<uint16_t>(cnt) + 1));
                }
                acc = (acc << l) | code[e];
                nacc += l;
                pos += l;
                if (nacc >= 32) {
                    nacc -= 32;
                    store_le<uint32_t>(w + 4 * wi++, uint32_t(acc >> nacc));
                }
            }
            if (nacc > 0) store_le<uint32_t>(w + 4 * wi, uint32_t(acc << (32 - nacc)));
            while (ci < chunks) {
                offs[c0 + ci] = uint8_t(bits[q] - ci * chunk_bits);
                if (ci % T == 0) store_le<uint32_t>(blockout + 4 * (b0 + ci / T), uint32_t(e0 + nq));
                ++ci;
            }
            uint8_t *row = panels + 16 * q;
            store_le<uint32_t>(row, uint32_t(c0));
            store_le<uint32_t>(row + 4, uint32_t(b0));
            store_le<uint32_t>(row + 8, uint32_t(bits[q]));
        }
    });
    store_le<uint32_t>(panels + 16 * g.n_items, uint32_t(n_chunks));
    store_le<uint32_t>(panels + 16 * g.n_items + 4, uint32_t(n_blocks));
    store_le<uint32_t>(blockout + 4 * n_blocks, uint32_t(n));
    pack_offsets(offs, dst + off[kOffsets]);
    *written = blob_bytes;
    return DFC_OK;
}

// Padded layout: no code crosses a chunk boundary (see dfc.h).  Pass 1
// places the chunk boundaries, which depend on every code before them, in
// one sequential walk over the code lengths; chunks own whole stream words,
// so pass 2 packs ranges of chunks on separate threads.
dfc_status encode_padded(const uint16_t *src, uint64_t n, const dfc_params &p, const uint8_t len[256],
                         const uint32_t code[256], uint64_t rows, uint64_t cols, uint8_t *dst, uint64_t cap,
                         uint64_t *written) {
    const uint32_t C = p.chunk_bytes, T = p.lanes_per_block;
    const uint32_t chunk_bits = 8u * C;
    // first element of every chunk that holds codes, then n
    std::vector<uint32_t> first{0};
    uint32_t fill = 0;
    for (uint64_t j = 0; j < n; ++j) {
        const uint32_t l = len[exponent_of(src[j])];
        if (fill + l > chunk_bits) {
            first.push_back(uint32_t(j));
            fill = 0;
        }
        fill += l;
    }
    const uint64_t used = n ? first.size() : 0;
    first.push_back(uint32_t(n));
    const uint64_t total_bits = used ? (used - 1) * chunk_bits + fill : 0;
    Layout L = layout_sizes(total_bits, C, T);
    if (L.n_chunks_used != used || L.n_chunks >= (uint64_t(1) << 32)) return DFC_ESIZE;
    SectionSizes sz = section_sizes(n, L.n_chunks, L.n_blocks, C, p.lut_bits, 0, false);
    uint64_t off[kNumSections];
    const uint64_t blob_bytes = place_sections(sz, off);
    if (cap < blob_bytes) return DFC_ESIZE;
    zero_parallel(dst, blob_bytes, p.threads);
    write_header(dst, p, n, total_bits, L.n_chunks, L.n_blocks, rows, cols, sz, off, blob_bytes, len);

    uint8_t *words = dst + off[kWords];
    uint8_t *raw = dst + off[kRaw];
    uint8_t *blockout = dst + off[kBlockout];
    const unsigned nt = unsigned(std::min<uint64_t>(pick_threads(p.threads, n), std::max<uint64_t>(used, 1)));
    parallel_for(nt, [&](unsigned t) {
        for (uint64_t c = used * t / nt; c < used * (t + 1) / nt; ++c) {
            uint8_t *w = words + uint64_t(C) * c;
            uint64_t acc = 0;
            uint32_t nacc = 0, wi = 0, bits = 0;
            for (uint64_t j = first[c]; j < first[c + 1]; ++j) {
                const uint16_t b = src[j];
                const uint32_t e = exponent_of(b);
                raw[j] = raw_of(b);
                const uint32_t l = len[e];
                acc = (acc << l) | code[e];
                nacc += l;
                bits += l;
                if (nacc >= 32) {
                    nacc -= 32;
                    store_le<uint32_t>(w + 4 * wi++, uint32_t(acc >> nacc));
                }
            }
            if (c + 1 < used) {
                // unused tail of a chunk followed by another: ones
                for (uint32_t r = chunk_bits - bits; r > 0;) {
                    const uint32_t k = std::min<uint32_t>(r, 32u - nacc);
                    acc = (acc << k) | ((uint64_t(1) << k) - 1u);
                    nacc += k;
                    r -= k;
                    if (nacc == 32) {
                        store_le<uint32_t>(w + 4 * wi++, uint32_t(acc));
                        nacc = 0;
                    }
                }
            }
            if (nacc > 0) store_le<uint32_t>(w + 4 * wi, uint32_t(acc << (32 - nacc)));
        }
    });
    for (uint64_t b = 0; b < L.n_blocks; ++b) {
        const uint64_t c = b * T;
        store_le<uint32_t>(blockout + 4 * b, c < used ? first[c] : uint32_t(n));
    }
    store_le<uint32_t>(blockout + 4 * L.n_blocks, uint32_t(n));
    *written = blob_bytes;
    return DFC_OK;
}

uint64_t kraft(const uint8_t len[256]) {
    uint64_t k = 0;
    for (int s = 0; s < 256; ++s)
        if (len[s]) k += uint64_t(1) << (kMaxLen - len[s]);
    return k;
}

}  // namespace

namespace dfc {

uint32_t choose_chunk_bytes(const uint64_t hist[256], const uint8_t len[256], uint32_t lanes) {
    uint64_t n = 0, total_bits = 0;
    for (int s = 0; s < 256; ++s) {
        n += hist[s];
        total_bits += hist[s] * len[s];
    }
    // exponent-entropy bound n (8 + H) / 8, H = sum (f / n) log2(n / f)
    double h = 0.0;
    for (int s = 0; s < 256; ++s)
        if (hist[s]) h += double(hist[s]) / double(n) * std::log2(double(n) / double(hist[s]));
    const double bound = double(n) * (8.0 + h) / 8.0;
    static const uint32_t order[4] = {16, 32, 8, 4};  // the decoder's fastest first
    uint32_t best = order[0];
    uint64_t best_size = ~uint64_t(0);
    for (uint32_t c : order) {
        const Layout L = layout_sizes(total_bits, c, lanes);
        const SectionSizes sz = section_sizes(n, L.n_chunks, L.n_blocks, c, 11);
        const uint64_t coded = kHeaderBytes + sz.bytes[kWords] + sz.bytes[kOffsets] + sz.bytes[kBlockout] +
                               sz.bytes[kRaw];
        if (double(coded) <= 1.02 * bound) return c;
        if (coded < best_size) {
            best_size = coded;
            best = c;
        }
    }
    return best;
}

dfc_status code_lengths(const uint64_t hist[256], uint32_t limit, uint8_t len[256]) {
    return package_merge(hist, limit, len);
}
void canonical_codes(const uint8_t len[256], uint32_t code[256]) {
    Canon c;
    canonical(len, c, code);
}
bool encoder_params_ok(const dfc_params &p) { return params_ok(p, true); }
uint64_t kraft_sum(const uint8_t len[256]) { return kraft(len); }
void container_header(uint8_t *dst, const dfc_params &p, uint64_t n, uint64_t total_bits, uint64_t n_chunks,
                      uint64_t n_blocks, uint64_t rows, uint64_t cols, const SectionSizes &sz,
                      const uint64_t off[kNumSections], uint64_t blob_bytes, const uint8_t len[256]) {
    write_header(dst, p, n, total_bits, n_chunks, n_blocks, rows, cols, sz, off, blob_bytes, len);
}

}  // namespace dfc

extern "C" {

void dfc_default_params(dfc_params *p) {
    if (!p) return;
    std::memset(p, 0, sizeof(*p));
    p->chunk_bytes = 0;  // automatic
    p->lanes_per_block = 64;
    p->max_code_len = kMaxLen;
    p->lut_bits = 11;
    p->layout = DFC_LAYOUT_FLAT;
}

const char *dfc_status_str(dfc_status s) {
    switch (s) {
        case DFC_OK: return "ok";
        case DFC_EINVAL: return "invalid argument";
        case DFC_ESIZE: return "size mismatch or buffer too small";
        case DFC_ECORRUPT: return "corrupt container";
        case DFC_EUNSUPPORTED: return "unsupported container variant";
        case DFC_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

dfc_status dfc_histogram(const uint16_t *src, uint64_t n, uint64_t hist[256]) {
    if (!hist || (!src && n)) return DFC_EINVAL;
    histogram_mt(src, n, hist, pick_threads(0, n));
    return DFC_OK;
}

dfc_status dfc_build_codebook(const uint64_t hist[256], uint32_t max_code_len, dfc_codebook *out) {
    if (!hist || !out || max_code_len < 1 || max_code_len > kMaxLen) return DFC_EINVAL;
    dfc_codebook cb;
    std::memset(&cb, 0, sizeof(cb));
    dfc_status st = package_merge(hist, max_code_len, cb.len);
    if (st != DFC_OK) return st;
    Canon c;
    canonical(cb.len, c, cb.code);
    cb.n_used = c.n_used;
    cb.min_len = cb.max_len = 0;
    for (int s = 0; s < 256; ++s) {
        if (!cb.len[s]) continue;
        if (!cb.min_len || cb.len[s] < cb.min_len) cb.min_len = cb.len[s];
        cb.max_len = std::max<uint32_t>(cb.max_len, cb.len[s]);
    }
    *out = cb;
    return DFC_OK;
}

dfc_status dfc_encode_bound(uint64_t n, const dfc_params *pin, uint64_t *max_bytes) {
    dfc_params p;
    if (pin) p = *pin; else dfc_default_params(&p);
    if (!max_bytes || !params_ok(p)) return DFC_EINVAL;
    if (p.chunk_bytes == 0) {
        // automatic: room for whichever chunk size the encoder picks
        uint64_t most = 0;
        for (uint32_t c : {4u, 8u, 16u, 32u}) {
            p.chunk_bytes = c;
            uint64_t b = 0;
            const dfc_status st = dfc_encode_bound(n, &p, &b);
            if (st != DFC_OK) return st;
            most = std::max(most, b);
        }
        *max_bytes = most;
        return DFC_OK;
    }
    const uint64_t bits = n * uint64_t(p.max_code_len);
    Layout L = layout_sizes(bits, p.chunk_bytes, p.lanes_per_block);
    SectionSizes s = section_sizes(n, L.n_chunks, L.n_blocks, p.chunk_bytes, p.lut_bits);
    if (p.layout == DFC_LAYOUT_PANEL) {
        // every item may add one partly used chunk and one partly used block
        PanelGeom g;
        if (!panel_geom(p.rows, p.cols, p.panel_k ? p.panel_k : uint32_t(DFC_PANEL_K_DEFAULT), g)) return DFC_EINVAL;
        s = section_sizes(n, L.n_chunks + g.n_items, L.n_blocks + g.n_items, p.chunk_bytes, p.lut_bits, g.n_items);
    } else if (p.layout == DFC_LAYOUT_ANS) {
        *max_bytes = ans_encode_bound(n, p.ans_steps);
        return DFC_OK;
    } else if (p.layout == DFC_LAYOUT_PADDED) {
        // every chunk but the last holds one code, or more than 8C - limit bits
        const uint64_t cb = 8ull * p.chunk_bytes, lim = p.max_code_len;
        const uint64_t chunks = std::min<uint64_t>(n, ceil_div(bits, cb - lim + 1) + 1);
        const uint64_t blocks = ceil_div(chunks, p.lanes_per_block);
        s = section_sizes(n, blocks * p.lanes_per_block, blocks, p.chunk_bytes, p.lut_bits, 0, false);
    }
    uint64_t off[kNumSections];
    *max_bytes = place_sections(s, off);
    return DFC_OK;
}

dfc_status dfc_encode(const uint16_t *src, uint64_t n, const dfc_params *pin, const dfc_codebook *cb_in,
                      void *dst_v, uint64_t cap, uint64_t *written) {
    dfc_params p;
    if (pin) p = *pin; else dfc_default_params(&p);
    if ((!src && n) || !dst_v || !written || !params_ok(p)) return DFC_EINVAL;
    if (n >= (uint64_t(1) << 32)) return DFC_ESIZE;
    if (p.layout == DFC_LAYOUT_PANEL) {
        if (!p.panel_k) p.panel_k = DFC_PANEL_K_DEFAULT;
        PanelGeom g;
        if (!panel_geom(p.rows, p.cols, p.panel_k, g) || p.rows * p.cols != n) return DFC_EINVAL;
    }
    uint64_t rows = p.rows, cols = p.cols;
    if (rows == 0 && cols == 0) {
        rows = 1;
        cols = n;
    }
    if (rows * cols != n) return DFC_EINVAL;
    uint8_t *dst = static_cast<uint8_t *>(dst_v);
    if (p.layout == DFC_LAYOUT_ANS) {
        if (cb_in) return DFC_EINVAL;  // frequencies always come from src's own histogram
        return encode_ans(src, n, p, rows, cols, dst, cap, written);
    }
    const unsigned nt = pick_threads(p.threads, n);

    uint64_t hist[256];
    histogram_mt(src, n, hist, nt);
    uint8_t len[256];
    if (cb_in) {
        std::memcpy(len, cb_in->len, 256);
        for (int s = 0; s < 256; ++s) {
            if (len[s] > p.max_code_len) return DFC_EINVAL;
            if (hist[s] && !len[s]) return DFC_EINVAL;
        }
        uint32_t used = 0;
        for (int s = 0; s < 256; ++s) used += len[s] != 0;
        if (n && (used < 2 || kraft(len) != (uint64_t(1) << kMaxLen))) return DFC_EINVAL;
    } else {
        dfc_status st = package_merge(hist, p.max_code_len, len);
        if (st != DFC_OK) return st;
    }
    if (p.chunk_bytes == 0)
        p.chunk_bytes = p.layout == DFC_LAYOUT_FLAT ? choose_chunk_bytes(hist, len, p.lanes_per_block) : 16u;
    Canon canon;
    uint32_t code[256];
    canonical(len, canon, code);
    const uint32_t lut_bits = p.lut_bits;
    if (p.layout == DFC_LAYOUT_PANEL) return encode_panel(src, n, p, len, code, dst, cap, written);
    if (p.layout == DFC_LAYOUT_PADDED) return encode_padded(src, n, p, len, code, rows, cols, dst, cap, written);

    // Pass 1: bits per thread range.
    std::vector<uint64_t> range_bits(nt + 1, 0);
    parallel_for(nt, [&](unsigned t) {
        uint64_t j0 = n * t / nt, j1 = n * (t + 1) / nt, b = 0;
        for (uint64_t j = j0; j < j1; ++j) b += len[exponent_of(src[j])];
        range_bits[t + 1] = b;
    });
    for (unsigned t = 0; t < nt; ++t) range_bits[t + 1] += range_bits[t];
    const uint64_t total_bits = range_bits[nt];
    const uint32_t C = p.chunk_bytes, T = p.lanes_per_block;
    Layout L = layout_sizes(total_bits, C, T);
    SectionSizes sz = section_sizes(n, L.n_chunks, L.n_blocks, C, lut_bits);
    uint64_t off[kNumSections];
    const uint64_t blob_bytes = place_sections(sz, off);
    if (cap < blob_bytes) return DFC_ESIZE;

    // Zero the container (padding, guard words and stream words are OR-ed).
    zero_parallel(dst, blob_bytes, p.threads);
    write_header(dst, p, n, total_bits, L.n_chunks, L.n_blocks, rows, cols, sz, off, blob_bytes, len);

    // Pass 2: pack codes, raw bytes, chunk offsets and block offsets.
    uint8_t *words = dst + off[kWords];
    uint8_t *raw = dst + off[kRaw];
    uint8_t *blockout = dst + off[kBlockout];
    std::vector<uint8_t> offs(L.n_chunks + 1, 0);
    std::vector<uint32_t> head(nt, 0);
    std::vector<uint64_t> head_idx(nt, ~uint64_t(0));
    const uint64_t chunk_bits = 8ull * C;
    parallel_for(nt, [&](unsigned t) {
        const uint64_t j0 = n * t / nt, j1 = n * (t + 1) / nt;
        uint64_t pos = range_bits[t];
        uint64_t acc = 0;
        uint32_t nacc = uint32_t(pos & 31);
        uint64_t wi = pos >> 5;
        bool first = true;
        auto emit = [&](uint64_t w, uint32_t v) {
            if (first) {
                head[t] = v;
                head_idx[t] = w;
                first = false;
            } else {
                store_le<uint32_t>(words + 4 * w, v);
            }
        };
        // Chunk boundaries whose first code start lies in this range.
        uint64_t lo = j0 == 0 ? 0 : pos - len[exponent_of(src[j0 - 1])] + 1;
        uint64_t ci = ceil_div(lo, chunk_bits);
        for (uint64_t j = j0; j < j1; ++j) {
            const uint16_t b = src[j];
            const uint32_t e = exponent_of(b);
            raw[j] = raw_of(b);
            while (ci * chunk_bits <= pos) {
                offs[ci] = uint8_t(pos - ci * chunk_bits);
                if (ci % T == 0) store_le<uint32_t>(blockout + 4 * (ci / T), uint32_t(j));
                ++ci;
            }
            const uint32_t l = len[e];
            acc = (acc << l) | code[e];
            nacc += l;
            pos += l;
            if (nacc >= 32) {
                nacc -= 32;
                emit(wi++, uint32_t(acc >> nacc));
            }
        }
        if (nacc > 0) emit(wi, uint32_t(acc << (32 - nacc)));
        if (t == nt - 1) {
            while (ci < L.n_chunks && ci * chunk_bits < total_bits) {
                offs[ci] = uint8_t(total_bits - ci * chunk_bits);
                if (ci % T == 0) store_le<uint32_t>(blockout + 4 * (ci / T), uint32_t(n));
                ++ci;
            }
        }
    });
    for (unsigned t = 0; t < nt; ++t) {
        if (head_idx[t] == ~uint64_t(0)) continue;
        uint8_t *w = words + 4 * head_idx[t];
        store_le<uint32_t>(w, load_le<uint32_t>(w) | head[t]);
    }
    store_le<uint32_t>(blockout + 4 * L.n_blocks, uint32_t(n));
    pack_offsets(offs, dst + off[kOffsets]);
    *written = blob_bytes;
    return DFC_OK;
}

dfc_status dfc_blob_info(const void *blob_v, uint64_t bytes, dfc_info *out) {
    if (!blob_v || !out) return DFC_EINVAL;
    const uint8_t *b = static_cast<const uint8_t *>(blob_v);
    if (bytes < kHeaderBytes) return DFC_ESIZE;
    if (load_le<uint32_t>(b + hdr::magic) != kMagic) return DFC_ECORRUPT;
    if (load_le<uint32_t>(b + hdr::version) != kVersion) return DFC_EUNSUPPORTED;
    dfc_info in;
    std::memset(&in, 0, sizeof(in));
    in.n = load_le<uint64_t>(b + hdr::n);
    in.total_bits = load_le<uint64_t>(b + hdr::total_bits);
    in.n_chunks = load_le<uint64_t>(b + hdr::n_chunks);
    in.n_blocks = load_le<uint64_t>(b + hdr::n_blocks);
    in.chunk_bytes = load_le<uint32_t>(b + hdr::chunk_bytes);
    in.lanes_per_block = load_le<uint32_t>(b + hdr::lanes);
    in.max_code_len = load_le<uint32_t>(b + hdr::max_code_len);
    in.lut_bits = load_le<uint32_t>(b + hdr::lut_bits);
    in.layout = load_le<uint32_t>(b + hdr::layout);
    in.rows = load_le<uint64_t>(b + hdr::rows);
    in.cols = load_le<uint64_t>(b + hdr::cols);
    in.blob_bytes = load_le<uint64_t>(b + hdr::blob_bytes);
    if (in.layout != DFC_LAYOUT_FLAT && in.layout != DFC_LAYOUT_PANEL && in.layout != DFC_LAYOUT_PADDED &&
        in.layout != DFC_LAYOUT_ANS)
        return DFC_EUNSUPPORTED;
    if (in.layout == DFC_LAYOUT_ANS) {
        dfc_status st = ans_blob_info(b, bytes, in);
        if (st == DFC_OK) *out = in;
        return st;
    }
    const bool panel = in.layout == DFC_LAYOUT_PANEL;
    const bool padded = in.layout == DFC_LAYOUT_PADDED;
    dfc_params p;
    dfc_default_params(&p);
    p.chunk_bytes = in.chunk_bytes;
    p.lanes_per_block = in.lanes_per_block;
    p.max_code_len = in.max_code_len;
    p.lut_bits = in.lut_bits;
    if (!params_ok(p, false)) return DFC_ECORRUPT;
    if (in.n >= (uint64_t(1) << 32) || in.rows * in.cols != in.n) return DFC_ECORRUPT;
    PanelGeom g{};
    if (panel) {
        in.panel_rows = load_le<uint32_t>(b + hdr::panel_rows);
        in.panel_k = load_le<uint32_t>(b + hdr::tile_k);
        if (in.panel_rows != kPanelRows || !panel_geom(in.rows, in.cols, in.panel_k, g)) return DFC_ECORRUPT;
        in.n_items = g.n_items;
    } else if (load_le<uint32_t>(b + hdr::panel_rows) || load_le<uint32_t>(b + hdr::tile_k)) {
        return DFC_ECORRUPT;
    }
    if (load_le<uint32_t>(b + hdr::reserved)) return DFC_ECORRUPT;
    for (int i = hdr::counts + 16; i < 256; ++i)
        if (b[i]) return DFC_ECORRUPT;

    // Code lengths: complete code under the limit (or empty for n == 0).
    const uint8_t *len = b + hdr::lengths;
    uint32_t used = 0, mn = 0, mx = 0;
    for (int s = 0; s < 256; ++s) {
        if (!len[s]) continue;
        if (len[s] > in.max_code_len) return DFC_ECORRUPT;
        used++;
        mn = mn ? std::min<uint32_t>(mn, len[s]) : len[s];
        mx = std::max<uint32_t>(mx, len[s]);
    }
    if (in.n) {
        if (used < 2 || kraft(len) != (uint64_t(1) << kMaxLen)) return DFC_ECORRUPT;
        // padded: every chunk boundary before the last code may add a tail
        // shorter than the longest code
        const uint64_t tails = padded ? (ceil_div(in.total_bits, 8ull * in.chunk_bytes) - 1) * (mx - 1) : 0;
        if (in.total_bits < in.n * mn || in.total_bits > in.n * mx + tails) return DFC_ECORRUPT;
    } else if (in.total_bits) {
        return DFC_ECORRUPT;
    }
    in.n_used = used;
    in.min_len = mn;
    in.max_len = mx;

    if (!panel) {
        Layout L = layout_sizes(in.total_bits, in.chunk_bytes, in.lanes_per_block);
        if (L.n_blocks != in.n_blocks || L.n_chunks != in.n_chunks) return DFC_ECORRUPT;
    } else if (in.n_chunks >= (uint64_t(1) << 32) || in.n_blocks >= (uint64_t(1) << 32)) {
        return DFC_ECORRUPT;
    }
    SectionSizes sz =
        section_sizes(in.n, in.n_chunks, in.n_blocks, in.chunk_bytes, in.lut_bits, in.n_items, !padded);
    uint64_t off[kNumSections];
    const uint64_t blob_bytes = place_sections(sz, off);
    if (blob_bytes != in.blob_bytes) return DFC_ECORRUPT;
    for (int i = 0; i < kNumSections; ++i) {
        if (load_le<uint64_t>(b + hdr::section(i)) != off[i]) return DFC_ECORRUPT;
        if (load_le<uint64_t>(b + hdr::section(i) + 8) != sz.bytes[i]) return DFC_ECORRUPT;
    }
    if (bytes < blob_bytes) return DFC_ESIZE;
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
    in.off_panels = off[kPanels];
    in.panels_bytes = sz.bytes[kPanels];
    in.off_counts = off[kCounts];
    in.counts_bytes = sz.bytes[kCounts];
    in.coded_bytes = kHeaderBytes + sz.bytes[kWords] + sz.bytes[kOffsets] + sz.bytes[kBlockout] + sz.bytes[kRaw] +
                     sz.bytes[kPanels] + sz.bytes[kCounts];

    // Panel table: chunk and block counts follow from every item's bits.
    std::vector<uint64_t> item_block;  // first block of every item (+ sentinel)
    if (panel) {
        const uint8_t *pt = b + off[kPanels];
        const uint64_t chunk_bits = 8ull * in.chunk_bytes;
        uint64_t bits_sum = 0;
        item_block.resize(g.n_items + 1);
        if (load_le<uint32_t>(pt) != 0 || load_le<uint32_t>(pt + 4) != 0) return DFC_ECORRUPT;
        for (uint64_t q = 0; q <= g.n_items; ++q) {
            const uint8_t *r = pt + 16 * q;
            item_block[q] = load_le<uint32_t>(r + 4);
            if (load_le<uint32_t>(r + 12)) return DFC_ECORRUPT;
            if (q == g.n_items) {
                if (load_le<uint32_t>(r) != in.n_chunks || item_block[q] != in.n_blocks || load_le<uint32_t>(r + 8))
                    return DFC_ECORRUPT;
                break;
            }
            const uint64_t bits = load_le<uint32_t>(r + 8), nq = kPanelRows * g.item_width(q);
            const uint64_t chunks = uint64_t(load_le<uint32_t>(r + 16)) - load_le<uint32_t>(r);
            const uint64_t blocks = uint64_t(load_le<uint32_t>(r + 20)) - item_block[q];
            if (bits < nq * mn || bits > nq * mx) return DFC_ECORRUPT;
            if (chunks != ceil_div(bits, chunk_bits) || blocks != ceil_div(chunks, in.lanes_per_block))
                return DFC_ECORRUPT;
            bits_sum += bits;
        }
        if (bits_sum != in.total_bits) return DFC_ECORRUPT;
    }
    // Chunk offsets: at most (longest code - 1) for live chunks, 0 elsewhere.
    if (!padded) {
        const uint8_t *ow = b + off[kOffsets];
        const uint64_t chunk_bits = 8ull * in.chunk_bytes;
        const uint32_t max_off = mx ? mx - 1 : 0;
        for (uint64_t i = 0; i <= in.n_chunks; ++i) {
            const uint64_t g = kOffsetBits * i;
            uint64_t pair = load_le<uint32_t>(ow + 4 * (g >> 5)) |
                            (uint64_t(load_le<uint32_t>(ow + 4 * (g >> 5) + 4)) << 32);
            const uint32_t v = uint32_t(pair >> (g & 31)) & 31u;
            const bool live = i < in.n_chunks && (panel || i * chunk_bits < in.total_bits);
            if (live ? v > max_off : v != 0) return DFC_ECORRUPT;
        }
    }
    // Block offsets: 0 .. n, non-decreasing, each block within LDS staging capacity.
    {
        const uint8_t *bo = b + off[kBlockout];
        if (load_le<uint32_t>(bo) != 0 || load_le<uint32_t>(bo + 4 * in.n_blocks) != in.n) return DFC_ECORRUPT;
        const uint64_t cap = in.n ? uint64_t(in.lanes_per_block) * ceil_div(8ull * in.chunk_bytes, mn) : 0;
        uint32_t prev = 0, widest = 0;
        for (uint64_t k = 1; k <= in.n_blocks; ++k) {
            uint32_t v = load_le<uint32_t>(bo + 4 * k);
            if (v < prev || v - prev > cap) return DFC_ECORRUPT;
            widest = std::max(widest, v - prev);
            prev = v;
        }
        // every item's blocks start at its first element
        for (uint64_t q = 0; panel && q < g.n_items; ++q)
            if (load_le<uint32_t>(bo + 4 * item_block[q]) != g.item_elem0(q)) return DFC_ECORRUPT;
        in.max_block_elems = widest;
    }
    // Panel chunk counts: at most the codes one chunk can start, and every
    // block's counts add up to its block offsets' difference, so a decoder
    // that places codes by prefix sums of them stays inside its block.
    if (panel) {
        const uint8_t *pt = b + off[kPanels], *cn = b + off[kCounts], *bo = b + off[kBlockout];
        const uint64_t max_count = mn ? ceil_div(8ull * in.chunk_bytes, mn) : 0;
        const uint32_t cw = count_width(in.chunk_bytes);
        for (uint64_t q = 0; q < g.n_items; ++q) {
            const uint64_t c0 = load_le<uint32_t>(pt + 16 * q), c1 = load_le<uint32_t>(pt + 16 * q + 16);
            for (uint64_t k = item_block[q]; k < item_block[q + 1]; ++k) {
                const uint64_t lo = c0 + uint64_t(in.lanes_per_block) * (k - item_block[q]);
                const uint64_t hi = std::min<uint64_t>(c1, lo + in.lanes_per_block);
                uint64_t sum = 0;
                for (uint64_t c = lo; c < hi; ++c) {
                    const uint32_t v = cw == 1 ? cn[c] : load_le<uint16_t>(cn + 2 * c);
                    if (v > max_count) return DFC_ECORRUPT;
                    sum += v;
                }
                if (sum != uint64_t(load_le<uint32_t>(bo + 4 * (k + 1))) - load_le<uint32_t>(bo + 4 * k))
                    return DFC_ECORRUPT;
            }
        }
        for (uint64_t i = cw * in.n_chunks; i < sz.bytes[kCounts]; ++i)
            if (cn[i]) return DFC_ECORRUPT;
    }
    *out = in;
    return DFC_OK;
}

}  // extern "C"
