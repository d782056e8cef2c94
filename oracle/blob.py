"""Serialized container ("DFC1") and its derived decode tables (oracle).

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
    184 u64 blob_bytes   192..255 zero

Bytes 256..511 hold the code length of every exponent value (0 = unused).
Sections follow in the order tables, words, offsets, blockout, raw, panels;
each starts at the next multiple of 256 bytes and padding is zero:

* words: n_chunks * C / 4 + 4 uint32 (the stream, zero-padded, 4 guard words)
* offsets: 5-bit fields off[0..n_chunks] packed as in ``stream.pack_offsets``
* blockout: uint32 out[0..n_blocks]
* raw: the raw bytes (sign << 7 | mantissa), padded to a multiple of 16
* tables: derived from the code lengths alone (see ``decode_tables``).

The decode tables are the "compact hierarchical lookup tables" of the
DFloat11 blog (section 03 item 1): a first level indexed by the next k stream
bits that resolves every whole code inside those k bits at once, and
canonical per-length tables that resolve the rare codes longer than k bits.
They are stored in the container so that a decoder only has to copy them
into on-chip memory.
"""
from __future__ import annotations

import math
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


# ------------------------------------------------------------ decode tables

ESCAPE = 0xFFFFF000


def rotate_exponent(e: int) -> int:
    """The byte a decoder stages for exponent e: e rotated right by one bit
    (bit 0 moves to bit 7).  With the raw byte sign << 7 | mantissa, the two
    bytes of a bf16 value are then (e' & 0x80 | raw & 0x7F, raw & 0x80 |
    e' & 0x7F), i.e. a byte-wise merge under a constant mask."""
    return ((e >> 1) | ((e & 1) << 7)) & 0xFF


def window_codes(window: int, k: int, tables):
    """Codes that fit in a k-bit window (next k stream bits, first bit most
    significant), decoded one after another from its first bit: a list of
    (symbol, length)."""
    out = []
    o = 0
    while o < k:
        found = None
        for l in range(1, k - o + 1):
            v = (window >> (k - o - l)) & ((1 << l) - 1)
            if v < tables["first"][l] + tables["count"][l]:
                found = (tables["order"][tables["base"][l] + v - tables["first"][l]], l)
                break
        if found is None:
            break
        out.append(found)
        o += found[1]
    return out


def step_value(codes) -> int:
    """(c << 16) - b as a uint32 for c codes of total length b; 0xFFFFF000
    when there are none.  Adding it to an accumulator (count << 16) + (bias -
    position) advances both the code count and the bit position."""
    if not codes:
        return ESCAPE
    return ((len(codes) << 16) - sum(l for _, l in codes)) & 0xFFFFFFFF


def lut_entry(window: int, k: int, tables):
    """(step, wsym, mask) for one k-bit window.

    step: step_value of every whole code inside the window (counting pass).
    wsym: uint64; bits 0..31 hold rotate_exponent of the first min(c, 4)
          codes (byte j = code j, 0 past them), bits 32..63 the step_value of
          those codes (symbol pass).
    mask: uint16, bit j set when a code ends exactly j + 1 bits in.
    """
    codes = window_codes(window, k, tables)
    first4 = codes[:4]
    syms = 0
    for j, (s, _) in enumerate(first4):
        syms |= rotate_exponent(int(s)) << (8 * j)
    wsym = syms | (step_value(first4) << 32)
    mask = 0
    o = 0
    for _, l in codes:
        o += l
        mask |= 1 << (o - 1)
    return step_value(codes), wsym, mask


def decode_tables(lengths, lut_bits: int) -> bytes:
    """The tables section for a window of k = lut_bits bits: step[2^k]
    (uint32), wsym[2^k] (uint64), mask[2^k] (uint16), then limit[32],
    first[32], base[32] (uint32, index = code length; entries 0 and 25..31
    are 0) and the 256-byte list of used symbols ordered by (length,
    symbol)."""
    t = cb.canonical_tables(lengths)
    if not 8 <= lut_bits <= 12:
        raise ValueError("lut_bits must be in 8..12")
    n = 1 << lut_bits
    step = np.zeros(n, dtype=np.uint32)
    wsym = np.zeros(n, dtype=np.uint64)
    mask = np.zeros(n, dtype=np.uint16)
    for w in range(n):
        step[w], wsym[w], mask[w] = lut_entry(w, lut_bits, t)
    limit = np.zeros(32, dtype=np.uint32)
    first = np.zeros(32, dtype=np.uint32)
    base = np.zeros(32, dtype=np.uint32)
    for l in range(1, cb.MAX_LEN + 1):
        limit[l] = t["limit"][l]
        first[l] = t["first"][l]
        base[l] = t["base"][l]
    order = np.zeros(256, dtype=np.uint8)
    order[: len(t["order"])] = t["order"]
    return (step.astype("<u4").tobytes() + wsym.astype("<u8").tobytes() + mask.astype("<u2").tobytes() +
            limit.astype("<u4").tobytes() + first.astype("<u4").tobytes() + base.astype("<u4").tobytes() +
            order.tobytes())


def tables_bytes(lut_bits: int) -> int:
    return 14 * (1 << lut_bits) + 3 * 128 + 256


# ----------------------------------------------------------------- container

def section_sizes(enc, lut_bits: int):
    n = enc["n"]
    return {
        "tables": tables_bytes(lut_bits),
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
    sizes = section_sizes(enc, lut_bits)
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

    put("tables", decode_tables(enc["lengths"], lut_bits))
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
    return {
        "n": n, "total_bits": total_bits, "n_chunks": n_chunks, "n_blocks": n_blocks,
        "chunk_bytes": chunk_bytes, "lanes": lanes, "max_len_limit": max_len,
        "lut_bits": lut_bits, "layout": layout, "panel_rows": panel_rows,
        "rows": rows, "cols": cols, "tile_k": tile_k, "sections": sec,
        "blob_bytes": vals[12], "lengths": lengths, "words": words, "off": offsets,
        "out": out, "raw": raw,
        "tables": b[sec["tables"][0]: sec["tables"][0] + sec["tables"][1]],
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
    offsets and raw bytes.  Alignment padding and the derived decode tables
    (a pure function of the code lengths) are not counted."""
    s = p["sections"]
    return HEADER_BYTES + sum(s[nm][1] for nm in ("words", "offsets", "blockout", "raw", "panels"))


def entropy_bound_bytes(hist) -> float:
    """n (8 + H_e) / 8: raw byte plus the exponent entropy per element."""
    n = float(np.asarray(hist, dtype=np.float64).sum())
    return n * (8.0 + cb.entropy_bits(hist)) / 8.0


def log2(x):
    return math.log2(x)
