// dfc_host_internal.h - host-side codec steps of libdfc shared by the host
// encoder and the device encoder's launcher (internal to libdfc).
#pragma once

#include <cstdint>

#include "dfc.h"
#include "dfc_format.h"

namespace dfc {

// Length-limited optimal code lengths (package-merge) for a histogram.
dfc_status code_lengths(const uint64_t hist[256], uint32_t limit, uint8_t len[256]);
// Canonical codes (RFC 1951 section 3.2.2) for code lengths.
void canonical_codes(const uint8_t len[256], uint32_t code[256]);
// Encoder parameters in range.
bool encoder_params_ok(const dfc_params &p);
// Kraft sum of the lengths scaled by 2^24 (2^24 for a complete code).
uint64_t kraft_sum(const uint8_t len[256]);
// Header, code lengths and derived decode tables of a container.
void container_header(uint8_t *dst, const dfc_params &p, uint64_t n, uint64_t total_bits, uint64_t n_chunks,
                      uint64_t n_blocks, uint64_t rows, uint64_t cols, const SectionSizes &sz,
                      const uint64_t off[kNumSections], uint64_t blob_bytes, const uint8_t len[256]);

}  // namespace dfc
