"""Test-side reader of the decode tables the library derives on the GPU
(the bytes ``dfc.derive_tables`` returns) and a decoder that walks them.

The byte layout is the library's own (compact lookup tables in on-chip
memory, DFloat11 blog, section 03 item 1): a k-bit first level with, per
window, the step over every whole code (``(codes << 16) - bits``, or an
escape when the first code is longer than k), up to four exponents rotated
right by one bit plus their step, and a mask of code ends; then the canonical
per-length tables for long codes.  ``table_walk_decode`` uses nothing but
those tables and the container's stream and chunk offsets, the way a GPU lane
does, so equality with the original exponents pins the tables the kernels
build.  It shares no code with the library or the oracle's decoders.
"""
import numpy as np

ESC = 0xFFFFF000


def parse_lut(tables: bytes, k: int):
    tables = bytes(tables)
    n = 1 << k
    step = np.frombuffer(tables, dtype="<u4", count=n)
    wsym = np.frombuffer(tables, dtype="<u8", count=n, offset=4 * n)
    mask = np.frombuffer(tables, dtype="<u2", count=n, offset=12 * n)
    rest = tables[14 * n:]
    limit = np.frombuffer(rest, dtype="<u4", count=32, offset=0)
    first = np.frombuffer(rest, dtype="<u4", count=32, offset=128)
    base = np.frombuffer(rest, dtype="<u4", count=32, offset=256)
    order = np.frombuffer(rest, dtype=np.uint8, count=256, offset=384)
    return step, wsym, mask, limit, first, base, order


def rotate(e: int) -> int:
    """The staged byte of exponent e: e rotated right by one bit."""
    return ((e >> 1) | ((e & 1) << 7)) & 0xFF


def unrotate(b):
    return ((b << 1) | (b >> 7)) & 0xFF


def table_walk_decode(p, tables: bytes):
    """Decode every chunk of a parsed flat container (``oracle.blob.parse_blob``)
    using only the tables: a counting pass that adds step entries into one
    accumulator (count in the high half, bit position in the low half) and
    corrects the last lookup's overshoot with the boundary mask of the window
    that starts at the chunk's end, then a symbol pass that takes up to four
    symbols per lookup (advancing by the entry's own step value) and falls
    back to the per-length tables for codes longer than k bits."""
    k = p["lut_bits"]
    step, wsym, mask, limit, first, base, order = parse_lut(tables, k)
    words = [int(w) for w in p["words"]]
    C = p["chunk_bytes"]
    BIAS = 0x8000

    def window(pos, nbits):
        v = 0
        for b in range(pos, pos + nbits):
            k_ = b >> 5
            v = (v << 1) | (((words[k_] >> (31 - (b & 31))) & 1) if k_ < len(words) else 0)
        return v

    def long_code(pos):
        w24 = window(pos, 24)
        for l in range(k + 1, 25):
            if w24 < int(limit[l]):
                return int(order[int(base[l]) + (w24 >> (24 - l)) - int(first[l])]), l
        raise AssertionError("no code")

    out = []
    for i in range(p["n_chunks"]):
        start = 8 * C * i + int(p["off"][i])
        end = min(8 * C * (i + 1) + int(p["off"][i + 1]), p["total_bits"])
        if start >= end:
            continue
        # counting pass: acc = (count << 16) + (BIAS - (pos - start))
        acc = BIAS
        pos = start
        while pos < end:
            d = int(step[window(pos, k)])
            if d == ESC:
                d = (1 << 16) - long_code(pos)[1]
            acc = (acc + d) & 0xFFFFFFFF
            pos = start + BIAS - (acc & 0xFFFF)
        cnt = acc >> 16
        if pos > end:
            cnt -= bin(int(mask[window(end, k)]) & ((1 << (pos - end)) - 1)).count("1")
        # symbol pass
        acc = BIAS
        pos, got = start, []
        while len(got) < cnt:
            e = int(wsym[window(pos, k)])
            d = e >> 32
            if d == ESC:
                s, l = long_code(pos)
                got.append(s)
                d = (1 << 16) - l
            else:
                c = (d >> 16) + 1
                take = min(c, cnt - len(got))
                got += [unrotate((e >> (8 * j)) & 0xFF) for j in range(take)]
            acc = (acc + d) & 0xFFFFFFFF
            pos = start + BIAS - (acc & 0xFFFF)
        out += got
    return np.array(out, dtype=np.uint8)
