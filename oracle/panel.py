"""Panel layout of a weight matrix for the fused decode + GEMM path (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe decoding weights on the GPU just before they are used
(DFloat11 blog post, introduction: online decompression); they give no
layout for decoding straight into a matrix product.  The reading taken here:

* W (M x K, row-major bf16, M a multiple of 32, K a multiple of 16) is cut
  into *items*: rows [32p, 32p + 32) x columns [s*Kp, min(K, (s+1)*Kp)),
  item index q = p * ceil(K / Kp) + s (row panels in order, then column
  slices);
* inside an item the elements come in 32 x 16 sub-tiles, columns ascending;
  inside a sub-tile, element 8*l + j (l = 0..63, j = 0..7) is
  W[32p + l % 32, c0 + 16t + 8*(l // 32) + j] -- the order in which one
  wavefront holds the A operand of a 32x32x16 bf16 matrix instruction;
* one codebook for the whole matrix (its own exponent histogram); every
  item's codes start on a fresh chunk, the bits between an item's last code
  and the next chunk boundary are zero;
* chunk offsets are item-relative: off[i] = (first code start >= the chunk's
  first bit, or the item's end if none) - the chunk's first bit;
* each item has ceil(chunks / T) blocks of its own (the last one may be
  short); out[b] = index, in panel order, of the first element whose code
  starts at or after the block's first bit; out[n_blocks] = n;
* a table of items + 1 entries (first chunk, first block, code bits of the
  item, 0), the last entry (n_chunks, n_blocks, 0, 0);
* per chunk, the number of codes whose first bit lies in it (a ``counts``
  section, one byte per chunk for C <= 16 -- a chunk of 8C <= 128 bits
  starts at most 128 codes -- and two bytes for C = 32): one more auxiliary
  variable of the two-phase
  decode (DFloat11 blog, section 03 item 2), with which a decoding lane
  learns its output position from a prefix sum of stored counts instead of
  decoding its chunk once more to count them.

Everything else (codebook, bit order, raw bytes) is the flat layout's,
applied to the permuted sequence.
"""
from __future__ import annotations

import struct

import numpy as np

from . import blob as bl
from . import codebook as cb
from . import stream as st
from .fields import merge, split

PANEL_ROWS = 32
SUBTILE_K = 16
LAYOUT_PANEL = 1


def count_width(chunk_bytes: int) -> int:
    """Bytes per stored chunk count: enough for 8C codes (codes of one bit)."""
    return 1 if 8 * chunk_bytes <= 255 else 2


def panel_items(rows: int, cols: int, panel_k: int):
    """(first row, first column, width) of every item, in item order."""
    if rows % PANEL_ROWS or cols % SUBTILE_K or panel_k % SUBTILE_K or panel_k <= 0:
        raise ValueError("rows must be a multiple of 32, cols and panel_k multiples of 16")
    items = []
    for p in range(rows // PANEL_ROWS):
        for c0 in range(0, cols, panel_k):
            items.append((PANEL_ROWS * p, c0, min(panel_k, cols - c0)))
    return items


def panel_order(rows: int, cols: int, panel_k: int) -> np.ndarray:
    """Row-major source index of every element, in panel order."""
    parts = []
    for r0, c0, w in panel_items(rows, cols, panel_k):
        t = np.arange(w // SUBTILE_K)[:, None, None]
        l = np.arange(64)[None, :, None]
        j = np.arange(8)[None, None, :]
        r = r0 + l % 32
        c = c0 + SUBTILE_K * t + 8 * (l // 32) + j
        parts.append((r * cols + c).ravel())
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def encode_panel(bits: np.ndarray, panel_k: int = 1024, chunk_bytes: int = 16, lanes: int = 64,
                 max_len: int = cb.MAX_LEN, lengths=None):
    """Encode a bf16 matrix (uint16, M x K) in the panel layout."""
    bits = np.asarray(bits, dtype=np.uint16)
    rows, cols = bits.shape
    items = panel_items(rows, cols, panel_k)
    seq = bits.ravel()[panel_order(rows, cols, panel_k)]
    exponent, raw = split(seq)
    n = seq.size
    hist = cb.histogram(exponent)
    if lengths is None:
        lengths = cb.package_merge_lengths(hist, max_len)
    lengths = np.asarray(lengths, dtype=np.uint8)
    if n and (lengths[exponent] == 0).any():
        raise ValueError("an exponent has no code")
    codes = cb.canonical_codes(lengths)
    words, offs, outs, table, counts = [], [], [], [], []
    chunk_base = block_base = elem_base = total_bits = 0
    for _, _, w in items:
        nq = PANEL_ROWS * w
        e = exponent[elem_base: elem_base + nq]
        starts, bits_q = st.code_starts(lengths.astype(np.int64)[e])
        chunks_q = -(-bits_q // (8 * chunk_bytes))
        blocks_q = -(-chunks_q // lanes)
        wq = st.pack_words(e, lengths, codes, chunks_q * (chunk_bytes // 4))
        words.append(wq)
        offs.append(st.chunk_offsets(starts, bits_q, chunk_bytes, chunks_q)[:chunks_q])
        counts.append(np.bincount(np.asarray(starts, dtype=np.int64) // (8 * chunk_bytes), minlength=chunks_q)
                      if nq else np.zeros(chunks_q, dtype=np.int64))
        first = np.arange(blocks_q, dtype=np.int64) * (8 * chunk_bytes * lanes)
        outs.append(elem_base + np.searchsorted(starts, first, side="left"))
        table.append((chunk_base, block_base, bits_q, 0))
        chunk_base += chunks_q
        block_base += blocks_q
        elem_base += nq
        total_bits += bits_q
    table.append((chunk_base, block_base, 0, 0))
    words.append(np.zeros(st.GUARD_WORDS, dtype=np.uint32))
    offs.append(np.zeros(1, dtype=np.uint8))
    outs.append(np.array([n], dtype=np.int64))
    return {
        "n": n, "rows": rows, "cols": cols, "panel_k": panel_k,
        "chunk_bytes": chunk_bytes, "lanes": lanes, "max_len_limit": max_len,
        "hist": hist, "lengths": lengths, "codes": codes, "total_bits": total_bits,
        "n_chunks": chunk_base, "n_blocks": block_base, "n_items": len(items),
        "words": np.concatenate(words).astype(np.uint32),
        "off": np.concatenate(offs).astype(np.uint8),
        "out": np.concatenate(outs).astype(np.uint32),
        "items": np.array(table, dtype=np.uint32),
        "counts": (np.concatenate(counts) if counts else np.zeros(0)).astype(np.uint16),
        "count_width": count_width(chunk_bytes),
        "raw": raw,
    }


def write_panel_blob(enc, lut_bits: int = 11) -> bytes:
    """The DFC1 container of a panel-layout encoding."""
    n = enc["n"]
    if not 8 <= lut_bits <= 12:
        raise ValueError("lut_bits must be in 8..12")
    sizes = {
        "tables": 0,
        "words": 4 * enc["words"].size,
        "offsets": 4 * (-(-5 * (enc["n_chunks"] + 1) // 32) + 1),
        "blockout": 4 * (enc["n_blocks"] + 1),
        "raw": 16 * (-(-n // 16)),
        "panels": 16 * (enc["n_items"] + 1),
        "counts": 16 * (-(-enc["count_width"] * enc["n_chunks"] // 16)),
    }
    names = ("tables", "words", "offsets", "blockout", "raw", "panels", "counts")
    offsets = {}
    pos = bl.HEADER_BYTES
    for name in names:
        pos = -(-pos // 256) * 256
        offsets[name] = pos if sizes[name] else 0
        pos += sizes[name]
    blob_bytes = -(-pos // 256) * 256
    buf = bytearray(blob_bytes)
    struct.pack_into("<IIQQQQIIIIIIQQII", buf, 0,
                     bl.MAGIC, bl.VERSION, n, enc["total_bits"], enc["n_chunks"], enc["n_blocks"],
                     enc["chunk_bytes"], enc["lanes"], enc["max_len_limit"], lut_bits,
                     LAYOUT_PANEL, PANEL_ROWS, enc["rows"], enc["cols"], enc["panel_k"], 0)
    fields = []
    for name in names[:6]:
        fields += [offsets[name], sizes[name]]
    struct.pack_into("<12QQ", buf, 88, *fields, blob_bytes)
    struct.pack_into("<QQ", buf, 192, offsets["counts"], sizes["counts"])
    buf[256:512] = np.asarray(enc["lengths"], dtype=np.uint8).tobytes()

    def put(name, data: bytes):
        o = offsets[name]
        buf[o: o + len(data)] = data

    put("words", np.asarray(enc["words"], dtype="<u4").tobytes())
    put("offsets", st.pack_offsets(enc["off"]).astype("<u4").tobytes())
    put("blockout", np.asarray(enc["out"], dtype="<u4").tobytes())
    put("raw", np.asarray(enc["raw"], dtype=np.uint8).tobytes())
    put("panels", np.asarray(enc["items"], dtype="<u4").tobytes())
    put("counts", np.asarray(enc["counts"], dtype="<u2" if enc["count_width"] == 2 else np.uint8).tobytes())
    return bytes(buf)


def decode_panel_blob(blob: bytes) -> np.ndarray:
    """Decode a panel-layout container back to the row-major matrix: every
    item with the chunk-parallel decoder over its own chunks, then the
    inverse permutation."""
    p = bl.parse_blob(blob)
    if p["layout"] != LAYOUT_PANEL:
        raise ValueError("not a panel-layout container")
    b = bytes(blob)
    o, s = p["sections"]["panels"]
    table = np.frombuffer(b, dtype="<u4", count=s // 4, offset=o).reshape(-1, 4).astype(np.int64)
    C = p["chunk_bytes"]
    wpc = C // 4
    exps = []
    for q in range(table.shape[0] - 1):
        c0, c1, bits_q = table[q, 0], table[q + 1, 0], table[q, 2]
        nch = c1 - c0
        words = np.concatenate([p["words"][c0 * wpc: c1 * wpc], np.zeros(st.GUARD_WORDS, dtype=np.uint32)])
        off = np.append(p["off"][c0:c1], 0)
        e, cnt = st.decode_chunked(words, off, int(bits_q), C, int(nch), p["lengths"], return_counts=True)
        if p["counts"] is None or not np.array_equal(p["counts"][c0:c1], cnt):
            raise ValueError("stored chunk code counts do not match the stream")
        exps.append(e)
    exponent = np.concatenate(exps) if exps else np.zeros(0, dtype=np.uint8)
    seq = merge(exponent, p["raw"])
    out = np.empty(p["n"], dtype=np.uint16)
    out[panel_order(p["rows"], p["cols"], p["tile_k"])] = seq
    return out.reshape(p["rows"], p["cols"])
