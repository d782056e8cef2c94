/*
 * dfc.h - C ABI of libdfc: lossless exponent-Huffman coding of bf16 weights
 * and its GPU decoder for AMD Instinct MI355X (gfx950).
 *
 * Method (DFloat11 blog post, "70% Size, 100% Accuracy: Lossless LLM
 * Compression for Efficient GPU Inference via Dynamic-Length Float
 * (DFloat11)"):
 *   section 02  bf16 weights have a low-entropy distribution; an entropy code
 *               gives frequent values short codes and rare values long ones,
 *               and decoding returns the original bits exactly;
 *   section 03, item 1  decoding uses compact hierarchical lookup tables held
 *               in on-chip memory;
 *   section 03, item 2  a two-phase kernel: threads first agree on read and
 *               write positions through small auxiliary variables, then
 *               rebuild the weights.
 *
 * What is coded: only the 8 exponent bits of every bf16 value, with a
 * canonical (RFC 1951 section 3.2.2) prefix code of at most 24 bits built by
 * package-merge from the matrix's own exponent histogram.  Sign and mantissa
 * stay one raw byte (sign << 7 | mantissa).  The code stream is cut into
 * fixed-size chunks of C bytes, one per GPU lane; each chunk carries a 5-bit
 * start offset (bits from the chunk start to its first code) and each block
 * of T chunks carries a 32-bit output offset (number of codes before it).
 *
 * A container holds the code (the 256 code lengths, or the rANS
 * frequencies) and the coded data, nothing derived: every GPU workgroup that
 * decodes derives its lookup tables from the code in its own LDS.
 *
 * Every entry point is re-entrant and keeps no state between calls, with one
 * exception: dfc_set_launch sets a process-wide launch shape that later
 * Huffman decode launches read.  The library never allocates device memory:
 * the caller owns every buffer.  Host functions take host pointers; device
 * functions take device pointers and enqueue work on the given HIP stream (a
 * hipStream_t passed as void*, NULL = the default stream) and return before
 * it runs; only dfc_encode_device waits for its stream (it reads the
 * histogram back).  No C++ exception crosses this interface.
 */
#ifndef DFC_H
#define DFC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFC_OK = 0,
    DFC_EINVAL = -1,       /* bad argument (null pointer, bad parameter value, misaligned buffer) */
    DFC_ESIZE = -2,        /* a buffer is too small, or n does not match the container */
    DFC_ECORRUPT = -3,     /* the container fails validation (or a decoded block count mismatched) */
    DFC_EUNSUPPORTED = -4, /* valid container, but this library cannot decode that variant */
    DFC_EHIP = -5          /* a HIP runtime call failed */
} dfc_status;

/* Element order of a container.  FLAT: row-major.  PANEL: the order the
 * fused decode + matrix product consumes (dfc_decode_gemm): the matrix is cut
 * into items of 32 rows x panel_k columns (row panels in order, then column
 * slices; the last slice may be narrower); inside an item come 32 x 16
 * sub-tiles, columns ascending, and inside a sub-tile element 8 l + j
 * (l = 0..63, j = 0..7) is W[32 p + l % 32][c0 + 16 t + 8 (l / 32) + j], the
 * A-operand order of a 32x32x16 bf16 matrix instruction.  Every item's codes
 * start on a fresh chunk and form their own blocks; a table of first chunk,
 * first block and code bits per item travels in the container, and so does
 * the number of codes whose first bit lies in each chunk (one byte per chunk
 * for C <= 16, two for C = 32), an
 * auxiliary variable of the two-phase decode (DFloat11 blog, section 03
 * item 2) that gives a decoding lane its write position by a prefix sum
 * instead of a counting pass over its chunk.
 * PADDED: row-major like FLAT, but no code crosses a chunk boundary: a code
 * that does not fit in what is left of its chunk opens the next chunk, and
 * the unused tail is set to ones.  Every chunk then decodes from its first
 * bit, keeping the codes that end inside it, and the container has no
 * chunk offsets (a reading of the two-phase decode of the DFloat11 blog,
 * section 03 item 2, with one auxiliary variable fewer).  The tail stops the
 * decode because it is shorter than the longest code and, in a complete
 * canonical code, no codeword is a prefix of a run of ones that short. */
/* ANS: row-major; the exponents are coded with interleaved rANS instead of
 * the prefix code (an arithmetic-family code of the kind the DFloat11 blog's
 * section 02 names, as in the ANS decoder of the VcLLM page's introduction).
 * The exponent histogram is quantised to frequencies f[s] summing to 2^12
 * (proportional shares rounded down, at least 1 for a present symbol, the
 * remaining units to the largest fractional parts, an excess taken back from
 * the largest shares); states are 32-bit integers in [2^16, 2^32) and the
 * stream is 16-bit words: decoding slot = x mod 2^12 gives the symbol s with
 * cum[s] <= slot < cum[s] + f[s], then x = f[s] (x >> 12) + slot - cum[s], and
 * if x < 2^16 the next word w enters as x = (x << 16) | w.  A block is 64
 * lanes x S steps: element i * 64 + l of the block belongs to lane l, and at
 * every step the lanes that need a word take the block's next words in lane
 * order.  The container keeps f (u16[256]) in its tables section (the
 * decoder derives its slot table from them), all blocks' word streams in the
 * words section, the first
 * word of every block (u32, n_blocks + 1) in the offsets section and the 64
 * initial states of every block (u32) in the blockout section; chunk_bytes
 * and n_chunks are 0, lut_bits holds 12, tile_k holds S. */
enum { DFC_LAYOUT_FLAT = 0, DFC_LAYOUT_PANEL = 1, DFC_LAYOUT_PADDED = 2, DFC_LAYOUT_ANS = 3 };
enum { DFC_ANS_STEPS_DEFAULT = 512, DFC_ANS_PROB_BITS = 12 };
enum { DFC_PANEL_ROWS = 32, DFC_PANEL_K_DEFAULT = 1024 };
enum { DFC_MAX_BATCH = 32 };

/* Encoder parameters; dfc_default_params fills the defaults. */
typedef struct {
    uint32_t chunk_bytes;     /* C: bytes of code stream per lane: 4, 8, 16 or 32 (default 16) */
    uint32_t lanes_per_block; /* T: chunks per block: 64 (one wavefront; the only value accepted) */
    uint32_t max_code_len;    /* code length limit, 1..24 (default 24) */
    uint32_t lut_bits;        /* k: bits indexed by the first-level decode table the GPU derives,
                                 8..12 (default 11); recorded in the header for the decoder */
    uint32_t layout;          /* DFC_LAYOUT_FLAT (row-major), _PANEL, _PADDED or _ANS */
    uint32_t threads;         /* host encoder threads; 0 = min(hardware threads, 16) */
    uint32_t panel_k;         /* PANEL: columns per item, a multiple of 16 (0 = 1024) */
    uint32_t ans_steps;       /* ANS: steps per block S, a multiple of 8 in 8..65536 (0 = 512);
                                 must be 0 for the other layouts.  ANS ignores chunk_bytes,
                                 max_code_len and lut_bits (they must still be valid) and
                                 needs lanes_per_block = 64 */
    uint64_t rows, cols;      /* matrix shape recorded in the header; 0,0 = 1 x n (FLAT only);
                                 PANEL needs rows % 32 == 0 and cols % 16 == 0 */
} dfc_params;

/* A codebook: code length and canonical code of every exponent value. */
typedef struct {
    uint8_t len[256];    /* 0 = unused; otherwise 1..24 */
    uint32_t code[256];  /* canonical code, right-aligned in len bits */
    uint32_t n_used;     /* symbols with len > 0 (2 or more for a non-empty histogram) */
    uint32_t min_len, max_len;
} dfc_codebook;

/* Validated description of a container (filled by dfc_blob_info). */
typedef struct {
    uint64_t n;            /* elements */
    uint64_t rows, cols;
    uint64_t blob_bytes;   /* whole container */
    uint64_t coded_bytes;  /* header + lengths + stream + offsets + block offsets + raw
                              (+ the panel table and chunk counts in the panel layout;
                              excludes derived decode tables and alignment padding) */
    uint64_t total_bits;   /* code stream length */
    uint64_t n_chunks, n_blocks;
    uint64_t off_tables, tables_bytes;  /* Huffman layouts: 0, 0; ANS: the frequencies f (512 B) */
    uint64_t off_words, words_bytes;
    uint64_t off_offsets, offsets_bytes;
    uint64_t off_blockout, blockout_bytes;
    uint64_t off_raw, raw_bytes;
    uint32_t chunk_bytes, lanes_per_block, max_code_len, lut_bits, layout;
    uint32_t n_used, min_len, max_len;
    uint32_t max_block_elems;  /* most elements any one block decodes */
    uint32_t panel_rows, panel_k;  /* PANEL: 32 and columns per item; 0 for FLAT */
    uint64_t n_items;              /* PANEL: items (32-row x panel_k-column slices) */
    uint64_t off_panels, panels_bytes;  /* PANEL: per-item table, (n_items + 1) x 4 u32 */
    uint32_t ans_steps;                 /* ANS: steps per block S; 0 otherwise */
    uint32_t ans_prob_bits;             /* ANS: 12 (frequencies sum to 2^12); 0 otherwise */
    uint64_t off_counts, counts_bytes;  /* PANEL: codes starting in every chunk, n_chunks x u8
                                           (u16 when C = 32), padded to 16 bytes; 0, 0 otherwise */
} dfc_info;

/* One matrix of a batched decode. */
typedef struct {
    const void *blob_dev;  /* device copy of the whole container (256-byte aligned) */
    const dfc_info *info;  /* host description of that container (from dfc_blob_info) */
    uint16_t *dst_dev;     /* n bf16 outputs (16-byte aligned), row-major */
    uint64_t n;            /* must equal info->n */
    const void *tables_dev; /* NULL, or this container's decode tables from dfc_derive_tables
                               (16-byte aligned): see dfc_decode */
} dfc_batch_item;

/* Fills *p with the defaults (C = 16, T = 64, limit 24, k = 11, flat). */
void dfc_default_params(dfc_params *p);

/* 256-bin histogram of the exponent bits (bits 14..7) of n bf16 values.
 * Host.  src: n uint16 bf16 bit patterns (may be NULL when n == 0).
 * hist: 256 counts, overwritten.  DFC_EINVAL on a null pointer. */
dfc_status dfc_histogram(const uint16_t *src, uint64_t n, uint64_t hist[256]);

/* Length-limited optimal code lengths (package-merge) and canonical codes for
 * an exponent histogram (DFloat11 blog, section 02: short codes for frequent
 * values).  Host.  Ties between equally good length vectors are broken
 * deterministically (equal weights: leaves before packages, leaves by
 * (count, symbol)).  One used symbol gets length 1 plus a phantom symbol
 * ((s + 1) mod 256) of length 1; an all-zero histogram gives an empty book.
 * DFC_EINVAL: null pointer or max_code_len outside 1..24; DFC_ESIZE: more
 * used symbols than 2^max_code_len. */
dfc_status dfc_build_codebook(const uint64_t hist[256], uint32_t max_code_len, dfc_codebook *out);

/* Upper bound on the container size dfc_encode can produce for n elements.
 * Host.  DFC_EINVAL on bad parameters. */
dfc_status dfc_encode_bound(uint64_t n, const dfc_params *p, uint64_t *max_bytes);

/* Encode n bf16 values into a container (DFloat11 blog, section 03 item 2:
 * the auxiliary per-chunk and per-block position variables are written here).
 * Host, multithreaded.  src: n bf16 bit patterns, row-major.  p: NULL =
 * defaults.  cb: NULL = build from src's own histogram with p->max_code_len;
 * otherwise every exponent present in src must have a code (DFC_EINVAL if
 * not).  dst: cap bytes, written from offset 0; *written receives the
 * container size (a multiple of 256).  DFC_ESIZE if cap is too small (use
 * dfc_encode_bound) or n >= 2^32.  The output is deterministic. */
dfc_status dfc_encode(const uint16_t *src, uint64_t n, const dfc_params *p,
                      const dfc_codebook *cb, void *dst, uint64_t cap, uint64_t *written);

/* Validate a host copy of a container and describe it.  Host.  Checks the
 * header, section placement, code lengths (complete code, limit 24; or the
 * rANS frequencies, summing to 2^12), every chunk offset and every block
 * offset.  DFC_ECORRUPT on any inconsistency, DFC_EUNSUPPORTED on an
 * unknown version/layout, DFC_ESIZE if bytes < the declared size. */
dfc_status dfc_blob_info(const void *blob, uint64_t bytes, dfc_info *out);

/* Decode one container on the GPU (DFloat11 blog, section 03: the two-phase
 * kernel with lookup tables in on-chip memory).  Device, asynchronous on
 * stream.  blob_dev: device copy of the container described by info (256-byte
 * aligned), in the FLAT, PADDED or ANS layout.  tables_dev: NULL, or the
 * decode tables dfc_derive_tables wrote for this container (16-byte aligned):
 * every workgroup then copies them into LDS instead of deriving them from
 * the code (a few microseconds per workgroup, which matters for small
 * launches; prepare them once per container and reuse them).  Tables of
 * another container give wrong values or a corrupt-block status; bytes that
 * dfc_derive_tables did not write are not allowed.  dst_dev: n uint16 outputs
 * (16-byte aligned), receives the original bf16 bit patterns, row-major.
 * status_dev: NULL, or one device uint32 that the kernel sets to DFC_ECORRUPT
 * (its two's-complement bit pattern) when a block fails its check: a decoded
 * code count that disagrees with the block offsets (FLAT, PADDED; the block's
 * outputs are then left unwritten), or lanes that do not end at the start
 * state or words not consumed exactly (ANS; the block's outputs are then
 * undefined).  The caller clears it beforehand and reads it after the stream
 * completes.  Synchronous errors: DFC_EINVAL (null/misaligned pointers),
 * DFC_ESIZE (n != info->n), DFC_EUNSUPPORTED (lanes_per_block != 64, a
 * PANEL container, streams past 4 GiB), DFC_EHIP (launch failure).  The ANS
 * layout is the interleaved rANS variant (see DFC_LAYOUT_ANS above). */
dfc_status dfc_decode(const void *blob_dev, const dfc_info *info, const void *tables_dev, uint16_t *dst_dev,
                      uint64_t n, uint32_t *status_dev, void *stream);

/* Decode up to DFC_MAX_BATCH containers with one kernel launch (the
 * whole-model, matrix-by-matrix decode just before use that the DFloat11
 * blog's introduction calls online decompression).  Same contract as
 * dfc_decode for every item; status_dev is shared.  count == 0 is a no-op. */
dfc_status dfc_decode_batch(const dfc_batch_item *items, uint32_t count, uint32_t *status_dev,
                            void *stream);

enum { DFC_GEMM_MAX_BATCH = 64 };

/* Fused decode + matrix product Y = W X (DFloat11 blog, introduction:
 * weights are decompressed on the GPU just before use; here the decoded
 * weights go from LDS straight into bf16 matrix instructions and never reach
 * HBM).  Device, asynchronous on stream.
 * w_blob_dev: device copy (256-byte aligned) of a DFC_LAYOUT_PANEL container
 * of W (M x K bf16, M = info->rows, K = info->cols), described by info.
 * tables_dev: NULL or its decode tables from dfc_derive_tables, as in
 * dfc_decode.
 * x_dev: B activation vectors of K bf16 each, x_dev[b K + k] (i.e. X is
 * K x B column-major), 16-byte aligned.  batch: B, 1..DFC_GEMM_MAX_BATCH.
 * y_dev: B output vectors of M fp32, y_dev[b M + m] (Y = W X, M x B
 * column-major), 4-byte aligned; every element is overwritten.  Products of
 * bf16 pairs are exact and accumulate in fp32; the partial sums of a panel's
 * column slices are added in a fixed order, so the same inputs give the
 * same bits on every run.  Exception: a matrix with more than 8 column
 * slices per panel and too few 32-row panels to occupy the GPU has each
 * panel shared by several workgroups, whose sums are added into Y (zeroed
 * first, on the stream) with fp32 atomics; with three or more per panel the
 * last bits of Y may then differ between runs.
 * workspace_dev: NULL, or workspace_bytes >= dfc_gemm_workspace_bytes(B, K)
 * bytes of device memory (16-byte aligned) that nothing else touches until
 * this call's work has run on the stream.  With it, a batch above 32 first
 * copies X there in the order the matrix instructions read it (one 1 KB run
 * per 16 columns and 32 vectors), and the products read X from the copy;
 * without it, they gather each operand from X in place (32-byte pieces of
 * 32 vectors), which is slower.  Batches up to 32 never use it.
 * status_dev: as in dfc_decode (nonzero if a block's stored chunk counts
 * disagree with its block offsets or with the codes in its chunks; Y is then
 * unspecified).  Errors before launch: DFC_EINVAL (null or misaligned
 * pointers, batch out of range, bad decode parameters), DFC_ESIZE (a
 * workspace smaller than needed), DFC_EUNSUPPORTED (not a panel-layout
 * container, lanes_per_block != 64, streams or Y past 4 GiB), DFC_EHIP
 * (launch failure). */
dfc_status dfc_decode_gemm(const void *w_blob_dev, const dfc_info *info, const void *tables_dev, const uint16_t *x_dev,
                           uint32_t batch, float *y_dev, void *workspace_dev, uint64_t workspace_bytes,
                           uint32_t *status_dev, void *stream);

/* Device bytes of the workspace dfc_decode_gemm can use for B vectors of K
 * values: 0 for B <= 32, else 2 x 64 x K rounded up to 16-column steps (X in
 * operand order, two tiles of 32 vectors).  Host. */
uint64_t dfc_gemm_workspace_bytes(uint32_t batch, uint64_t cols);

/* Workspace bytes dfc_encode_device needs for n elements.  Host. */
dfc_status dfc_encode_device_workspace(uint64_t n, uint64_t *bytes);

/* 256-bin exponent histogram of n bf16 values in device memory (bits 14..7),
 * as 32-bit counts into hist_dev (256 device uint32, overwritten; a bin's
 * count wraps past 2^32 - 1, so n below 2^32 is exact).  Device,
 * asynchronous on stream.  DFC_EINVAL on null pointers. */
dfc_status dfc_histogram_device(const uint16_t *src_dev, uint64_t n, uint32_t *hist_dev, void *stream);

/* Encode n bf16 values already in device memory into a container in device
 * memory, byte-identical to what dfc_encode writes for the same values and
 * parameters (FLAT, PANEL or ANS layout).  The histogram is taken on the device and
 * read back (the call synchronizes the stream), the code and the container
 * layout are set on the host (FLAT: the stream length is the histogram
 * times the code lengths), and the code bits, chunk offsets, block offsets
 * and raw bytes are written by kernels.  ANS: the frequencies are set on the
 * host, one wavefront per block counts the block's words, their scan is read
 * back to place the sections, and a second pass writes the words, word
 * offsets and states.  PANEL: one workgroup per item sums the item's code
 * bits, the host places the items and the sections, and a second pass packs
 * every item from its first chunk.  The call returns after the stream is
 * idle.
 * src_dev: n uint16 (2-byte aligned).  cb: NULL = the data's own code.
 * dst_dev: cap bytes (256-byte aligned), use dfc_encode_bound.
 * work_dev: work_bytes >= dfc_encode_device_workspace(n) (256-byte aligned).
 * *written (host) receives the container size.  Errors: DFC_EINVAL (null or
 * misaligned pointers, bad parameters, an exponent without a code, a
 * codebook with ANS), DFC_ESIZE (cap or workspace too small, n >= 2^32),
 * DFC_EUNSUPPORTED (PADDED layout, PANEL items wider than 5.5 M columns),
 * DFC_EHIP. */
dfc_status dfc_encode_device(const uint16_t *src_dev, uint64_t n, const dfc_params *p, const dfc_codebook *cb,
                             void *dst_dev, uint64_t cap, void *work_dev, uint64_t work_bytes, uint64_t *written,
                             void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * encoder as dfc_encode_device, with the same arguments except the
 * workspace, which is a fixed array of DFC_NOALLOC_WORKSPACE_BYTES (16 MiB)
 * in device memory that the library holds on every GPU it runs on until the
 * process ends.  The call allocates no device memory.  It takes inputs up to
 * dfc_encode_device_workspace(n) <= DFC_NOALLOC_WORKSPACE_BYTES, that is
 * n <= 715,000,000 weights; larger inputs return DFC_ESIZE before any work.
 * Calls on one GPU share its array: the library serializes them (each call
 * holds that GPU's array until its stream is idle, which is when it
 * returns), so concurrent calls from several host threads wait for each
 * other rather than race.  The array keeps the last call's contents; what
 * must start at zero (the histogram) is cleared by every call.  The GPU is
 * the one the stream belongs to (the current device for the NULL stream).
 * Errors as dfc_encode_device, plus DFC_ESIZE for n above the limit. */
enum { DFC_NOALLOC_WORKSPACE_BYTES = 16 << 20 };
dfc_status dfc_encode_device_noalloc(const uint16_t *src_dev, uint64_t n, const dfc_params *p, const dfc_codebook *cb,
                                     void *dst_dev, uint64_t cap, uint64_t *written, void *stream);

/* Launch tuning knob for benchmarks (Huffman layouts): wavefronts per
 * workgroup (1..16), wave-blocks each wavefront decodes (1..64), when a
 * wavefront stores the first complete output rounds of each block
 * (DFC_STORES_DEFERRED holds them in registers and stores them while it
 * decodes its next block, 4 wavefronts per SIMD; DFC_STORES_IMMEDIATE
 * stores them at once, 8 per SIMD, 5 for 32-byte chunks), and the blocks
 * per run (1..64): a matrix's blocks are cut into runs of that many
 * consecutive blocks, dealt out to its wavefronts in turn.  0 = automatic
 * for each (the most resident wavefronts, in the smallest workgroup that
 * holds that many; immediate for 4- and 8-byte chunks; for 16-byte chunks
 * deferred once the immediate build would give each of its wavefronts at
 * least 24 blocks in sequence; for 32-byte chunks deferred unless that
 * doubles the blocks a wavefront decodes in sequence; runs of about 6,144
 * output values, 2 to 16 blocks, at most a quarter of a wavefront's share,
 * so 1 for a matrix that gives its wavefronts fewer than 4 blocks each).
 * Returns DFC_EINVAL for
 * other values.  The library's only process-wide state: each value is read
 * atomically by every later decode launch, on any thread, so a caller that
 * changes it while other threads decode changes their launch shape (never
 * their results). */
enum { DFC_STORES_AUTO = 0, DFC_STORES_DEFERRED = 1, DFC_STORES_IMMEDIATE = 2 };
dfc_status dfc_set_launch(uint32_t waves_per_group, uint32_t blocks_per_wave, uint32_t stores,
                          uint32_t run_blocks);

/* Bytes of the decode tables the GPU kernels derive from a container's code
 * (dfc_derive_tables writes that many).  Host.  Huffman layouts: the k-bit
 * first level (step u32, symbols u64, boundary mask u16 per window) and the
 * canonical per-length tables, 14 * 2^k + 640 bytes; ANS: the slot table,
 * 4 * 2^12 bytes.  DFC_EINVAL / DFC_EUNSUPPORTED on a bad info. */
dfc_status dfc_derived_tables_bytes(const dfc_info *info, uint64_t *bytes);

/* The decode tables of a container (DFloat11 blog, section 03 item 1:
 * compact lookup tables in on-chip memory), derived from its code by one
 * workgroup of `threads` threads (a multiple of 64, at most 1024; 0 = 1024)
 * with the same device code every decoding workgroup runs when it is given
 * no tables, and written to dst_dev (cap >= dfc_derived_tables_bytes,
 * 16-byte aligned).  Device, asynchronous.  Pass them to dfc_decode,
 * dfc_decode_batch (tables_dev of the item) or dfc_decode_gemm to skip the
 * derivation in every launch.  Their layout is private to the library (and
 * may change with it); tests read them to check the derivation.  Errors:
 * DFC_EINVAL (null or misaligned pointers, bad thread count, an empty
 * container), DFC_ESIZE (cap), DFC_EHIP. */
dfc_status dfc_derive_tables(const void *blob_dev, const dfc_info *info, uint32_t threads, void *dst_dev,
                             uint64_t cap, void *stream);

/* Human-readable name of a status code. */
const char *dfc_status_str(dfc_status s);

#ifdef __cplusplus
}
#endif

#endif /* DFC_H */
