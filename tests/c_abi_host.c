/* A plain C99 user of the library's host entry points, compiled with
 * -std=c99 -pedantic -Werror against include/dfc.h and linked to libdfc.so:
 * the header must be valid C and the exported names must resolve without
 * C++ name mangling.
 *
 * It encodes a small deterministic bf16 tensor through the C ABI, reads the
 * container back with dfc_blob_info, checks the fields it can check without
 * a GPU, checks the codebook's Kraft sum, and exercises the error returns.
 * Exit status 0 on success; the failing check is printed otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dfc.h"

#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                   \
        }                                                               \
    } while (0)

/* bf16 patterns with a spread of exponents: sign and mantissa from a linear
 * congruential sequence, exponent 120 + (k mod 9) - (k mod 4). */
static void fill(uint16_t *x, uint64_t n) {
    uint32_t s = 12345u;
    uint64_t k;
    for (k = 0; k < n; ++k) {
        s = s * 1103515245u + 12345u;
        x[k] = (uint16_t)(((s >> 16) & 0x807Fu) | ((uint32_t)(120 + (int)(k % 9) - (int)(k % 4)) << 7));
    }
}

int main(void) {
    const uint64_t n = 100003; /* not a multiple of anything useful */
    uint16_t *x = (uint16_t *)malloc(n * sizeof(uint16_t));
    uint64_t hist[256], bound = 0, written = 0, total = 0, used = 0;
    uint64_t kraft_num = 0;
    dfc_params p;
    dfc_codebook cb;
    dfc_info info;
    void *blob;
    int s;
    CHECK(x != NULL);
    fill(x, n);

    CHECK(dfc_histogram(x, n, hist) == DFC_OK);
    for (s = 0; s < 256; ++s) {
        total += hist[s];
        used += hist[s] ? 1u : 0u;
    }
    CHECK(total == n);

    CHECK(dfc_build_codebook(hist, 24, &cb) == DFC_OK);
    CHECK(cb.n_used >= used && cb.max_len <= 24 && cb.min_len >= 1);
    /* a complete prefix code: sum of 2^(24 - len) over used symbols is 2^24 */
    for (s = 0; s < 256; ++s)
        if (cb.len[s]) kraft_num += (uint64_t)1 << (24 - cb.len[s]);
    CHECK(kraft_num == ((uint64_t)1 << 24));

    dfc_default_params(&p);
    CHECK(p.chunk_bytes == 0 && p.lanes_per_block == 64 && p.max_code_len == 24); /* 0: automatic */
    CHECK(dfc_encode_bound(n, &p, &bound) == DFC_OK && bound > n);
    blob = malloc((size_t)bound);
    CHECK(blob != NULL);
    CHECK(dfc_encode(x, n, &p, NULL, blob, bound, &written) == DFC_OK);
    CHECK(written > 0 && written <= bound && written % 256 == 0);
    const uint64_t container = written;

    memset(&info, 0, sizeof(info));
    CHECK(dfc_blob_info(blob, written, &info) == DFC_OK);
    CHECK(info.n == n && info.blob_bytes == written && info.layout == DFC_LAYOUT_FLAT);
    CHECK(info.chunk_bytes == 16 && info.lanes_per_block == 64);
    CHECK(info.n_chunks == info.n_blocks * 64 && info.raw_bytes >= n);
    CHECK(info.coded_bytes < 2 * n); /* it compresses */

    /* the error returns of the boundary */
    CHECK(dfc_blob_info(blob, written - 256, &info) == DFC_ESIZE);
    CHECK(dfc_encode(x, n, &p, NULL, blob, 16, &written) == DFC_ESIZE);
    p.chunk_bytes = 12;
    CHECK(dfc_encode_bound(n, &p, &bound) == DFC_EINVAL);
    CHECK(dfc_status_str(DFC_ECORRUPT) != NULL && strlen(dfc_status_str(DFC_ECORRUPT)) > 0);

    free(blob);
    free(x);
    printf("c abi ok: %llu weights -> %llu container bytes\n", (unsigned long long)n,
           (unsigned long long)container);
    return 0;
}
