"""Serialized container ("DFC1") of the flat and padded layouts (oracle).

The container is one contiguous byte buffer so that one host-to-device copy
moves it.  All integers are little-endian.

Header (bytes 0..255)::

      0 u32 magic 0x31434644 ("DFC1")      4 u32 version = 1
      8 u64 n                               16 u64 total_bits
     24 u64 n_chunks                        32 u64 n_blocks
     40 u32 chunk_bytes C                   44 u32 lanes_per_block T
     48 u32 max_code_len (builder limit)    52 u32 lut_bits k
     56 u32 layout (0 = flat)               60 u32 panel_rows
     64 u64 rows                            72 u64 cols
     80 u32 tile_k                          84 u32 reserved (0)
     88 u64 off_tables    96 u64 tables_bytes
    104 u64 off_words    112 u64 words_bytes
    120 u64 off_offsets  128 u64 offsets_bytes
    136 u64 off_blockout 144 u64 blockout_bytes
    152 u64 off_raw      160 u64 raw_bytes
    168 u64 off_panels   176 u64 panels_bytes
    184 u64 blob_bytes
    192 u64 off_counts   200 u64 counts_bytes (panel layout; 0 otherwise;
                         one count per chunk, u8 for C <= 16, u16 for C = 32)
    208..255 zero

Bytes 256..511 hold the code length of every exponent value (0 = unused).
Sections follow in the order tables, words, offsets, blockout, raw, panels;
each starts at the next multiple of 256 bytes and padding is zero:

* words: n_chunks * C / 4 + 4 uint32 (the stream, zero-padded, 4 guard words)
* offsets: 5-bit fields off[0..n_chunks] packed as in ``stream.pack_offsets``
* blockout: uint32 out[0..n_blocks]
* raw: the raw bytes (sign << 7 | mantissa), padded to a multiple of 16
* tables: empty (offset and size 0) in the Huffman layouts.

A container holds the code (the code lengths) and the coded data only.  The
lookup tables a decoder uses to find code boundaries quickly (the DFloat11
blog's section 03 item 1) are a function of the code lengths, built by the
decoder itself, and never written here; ``lut_bits`` only records the width
of the first-level window the decoder should use.
"""
from __future__ import annotations

import struct

import numpy as np

from . import codebook as cb
from . import stream as st

MAGIC = 0x31434644
VERSION = 1
HEADER_BYTES = 512
LAYOUT_FLAT = 0


def _align(x: int, a: int = 256) -> int:
    return -(-x // a) * a


# ----------------------------------------------------------------- container

def section_sizes(enc):
    n = enc["n"]
    return {
        "tables": 0,
        "words": 4 * enc["words"].size,
        "offsets": 0 if enc.get("off") is None else 4 * (-(-5 * (enc["n_chunks"] + 1) // 32) + 1),
        "blockout": 4 * (enc["n_blocks"] + 1),
        "raw": 16 * (-(-n // 16)),
        "panels": 0,
    }


def write_blob(enc, lut_bits: int = 11, rows: int | None = None, cols: int | None = None,
               layout: int = LAYOUT_FLAT) -> bytes:
    """Container of a flat encoding (``stream.encode``), or of a padded one
    (``padded.encode_padded``, layout 2: no offsets section)."""
    n = enc["n"]
    if rows is None or cols is None:
        rows, cols = 1, n
    if rows * cols != n:
        raise ValueError("rows * cols != n")
    if not 8 <= lut_bits <= 12:
        raise ValueError("lut_bits must be in 8..12")
    sizes = section_sizes(enc)
    offsets = {}
    pos = HEADER_BYTES
    for name in ("tables", "words", "offsets", "blockout", "raw", "panels"):
        pos = _align(pos)
        offsets[name] = pos if sizes[name] else 0
        pos += sizes[name]
    blob_bytes = _align(pos)
    buf = bytearray(blob_bytes)
    struct.pack_into("<IIQQQQIIIIIIQQII", buf, 0,
                     MAGIC, VERSION, n, enc["total_bits"], enc["n_chunks"], enc["n_blocks"],
                     enc["chunk_bytes"], enc["lanes"], enc["max_len_limit"], lut_bits,
                     layout, 0, rows, cols, 0, 0)
    fields = []
    for name in ("tables", "words", "offsets", "blockout", "raw", "panels"):
        fields += [offsets[name], sizes[name]]
    struct.pack_into("<12QQ", buf, 88, *fields, blob_bytes)
    buf[256:512] = np.asarray(enc["lengths"], dtype=np.uint8).tobytes()

    def put(name, data: bytes):
        o = offsets[name]
        buf[o: o + len(data)] = data

    put("words", np.asarray(enc["words"], dtype="<u4").tobytes())
    if sizes["offsets"]:
        put("offsets", st.pack_offsets(enc["off"]).astype("<u4").tobytes())
    put("blockout", np.asarray(enc["out"], dtype="<u4").tobytes())
    put("raw", np.asarray(enc["raw"], dtype=np.uint8).tobytes())
    return bytes(buf)


def parse_blob(blob: bytes):
    """Header fields and section views of a container."""
    b = bytes(blob)
    (magic, version, n, total_bits, n_chunks, n_blocks, chunk_bytes, lanes, max_len,
     lut_bits, layout, panel_rows, rows, cols, tile_k, _r) = struct.unpack_from(
        "<IIQQQQIIIIIIQQII", b, 0)
    if magic != MAGIC or version != VERSION:
        raise ValueError("not a DFC1 container")
    vals = struct.unpack_from("<12QQ", b, 88)
    names = ("tables", "words", "offsets", "blockout", "raw", "panels")
    sec = {nm: (vals[2 * i], vals[2 * i + 1]) for i, nm in enumerate(names)}
    sec["counts"] = struct.unpack_from("<QQ", b, 192)
    lengths = np.frombuffer(b, dtype=np.uint8, count=256, offset=256).copy()

    def view(name, dtype):
        o, s = sec[name]
        return np.frombuffer(b, dtype=dtype, count=s // np.dtype(dtype).itemsize, offset=o).copy()

    words = view("words", "<u4")
    # 5-bit chunk offsets in the flat and panel layouts (the padded layout
    # has none; the ANS layout keeps block stream offsets there instead)
    five_bit = sec["offsets"][1] and layout in (0, 1)
    offsets = st.unpack_offsets(view("offsets", "<u4"), n_chunks + 1) if five_bit else None
    out = view("blockout", "<u4")
    raw = view("raw", np.uint8)[:n]
    counts = (view("counts", "<u2" if 8 * chunk_bytes > 255 else np.uint8)[:n_chunks].astype(np.uint16)
              if sec["counts"][1] else None)
    return {
        "n": n, "total_bits": total_bits, "n_chunks": n_chunks, "n_blocks": n_blocks,
        "chunk_bytes": chunk_bytes, "lanes": lanes, "max_len_limit": max_len,
        "lut_bits": lut_bits, "layout": layout, "panel_rows": panel_rows,
        "rows": rows, "cols": cols, "tile_k": tile_k, "sections": sec,
        "blob_bytes": vals[12], "lengths": lengths, "words": words, "off": offsets,
        "out": out, "raw": raw, "counts": counts,
    }


def decode_blob(blob: bytes) -> np.ndarray:
    """Original bf16 bit patterns from a container (chunk-parallel decoder)."""
    from .fields import merge
    p = parse_blob(blob)
    if p["layout"] == 2:
        from .padded import decode_padded_blob
        return decode_padded_blob(blob)
    e = st.decode_chunked(p["words"], p["off"], p["total_bits"], p["chunk_bytes"],
                          p["n_chunks"], p["lengths"])
    if e.size != p["n"]:
        raise ValueError("decoded count does not match n")
    return merge(e, p["raw"])


# ----------------------------------------------------------- size accounting

def coded_bytes(p) -> int:
    """Bytes a reader must store: header, code lengths, stream, offsets, block
    offsets and raw bytes.  Alignment padding is not counted."""
    s = p["sections"]
    return HEADER_BYTES + sum(s[nm][1] for nm in ("words", "offsets", "blockout", "raw", "panels", "counts"))


def entropy_bound_bytes(hist) -> float:
    """n (8 + H_e) / 8: raw byte plus the exponent entropy per element."""
    n = float(np.asarray(hist, dtype=np.float64).sum())
    return n * (8.0 + cb.entropy_bits(hist)) / 8.0


# Chunk sizes in the order an automatic choice tries them: the decoder's
# fastest first (16 bytes per lane), then the larger chunk with half the
# offset overhead, then the smaller ones.
AUTO_CHUNK_ORDER = (16, 32, 8, 4)
AUTO_SIZE_TARGET = 1.02


def flat_coded_bytes(n: int, total_bits: int, chunk_bytes: int, lanes: int = 64) -> int:
    """Coded size of a flat container, written out from n, the stream length
    and the chunk geometry alone: 512-byte header and code lengths, the
    stream words (whole blocks plus 4 guard words), the 5-bit chunk offsets
    (n_chunks + 1 fields in 32-bit words plus one word of slack), the block
    offsets (n_blocks + 1 words) and the raw bytes (n rounded up to 16)."""
    _, n_blocks, n_chunks = st.layout_sizes(total_bits, chunk_bytes, lanes)
    return (HEADER_BYTES + (n_chunks * chunk_bytes + 16) + 4 * (-(-5 * (n_chunks + 1) // 32) + 1) +
            4 * (n_blocks + 1) + 16 * (-(-n // 16)))


def choose_chunk_bytes(hist, lengths, lanes: int = 64) -> int:
    """Automatic chunk size of the flat layout: the first of AUTO_CHUNK_ORDER
    whose coded size is within 2% of the exponent-entropy bound, else the one
    with the smallest coded size (the earlier one on a tie)."""
    h = np.asarray(hist, dtype=np.int64)
    n = int(h.sum())
    total_bits = int((h * np.asarray(lengths, dtype=np.int64)).sum())
    bound = entropy_bound_bytes(h)
    sizes = [(flat_coded_bytes(n, total_bits, c, lanes), c) for c in AUTO_CHUNK_ORDER]
    for size, c in sizes:
        if size <= AUTO_SIZE_TARGET * bound:
            return c
    return min(sizes, key=lambda t: t[0])[1]

