"""Offset-free padded-chunk layout of the code stream (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The two-phase decode of the DFloat11 blog (section 03 item 2) lets the
lanes agree on where to read through small auxiliary variables.  In the flat
layout one of them is a 5-bit start offset per chunk, because a code may
begin in one chunk and end in the next.  This layout removes the offsets by
never letting a code cross a chunk boundary.  It is a reading of that
passage, not something the pages spell out:

* codes are placed in element order, each right after the previous one,
  except that a code which would run past the end of its chunk (bit 8C(i+1))
  is placed at the first bit of the next chunk instead;
* the r bits it leaves unused at the end of the chunk are set to one;
* ``total_bits`` is the end of the last code; the bits after it are zero;
  chunk and block counts follow from it as in the flat layout (blocks of T
  chunks, the stream zero-padded to whole blocks), and ``out[b]`` is again
  the number of codes that start before bit 8CTb, ``out[n_blocks] = n``;
* there are no chunk offsets: the container's offsets section is empty.

A lane then decodes its chunk from the chunk's first bit and keeps every code
that ends at or before min(8C(i+1), total_bits).  It stops at the right place
because the unused tail is shorter than the code that moved (r < l <= L, L the
longest code length): in a complete canonical code the last codeword is L
ones, so no codeword can be a prefix of r ones (it would be a proper prefix of
another codeword), and whatever the tail and the next chunk's bits decode to
is longer than r and ends past the chunk.

Everything else (code, bit order, raw bytes, header) is the flat
layout's; the header's layout field is 2.
"""
from __future__ import annotations

import numpy as np

from . import blob as bl
from . import codebook as cb
from . import stream as st
from .fields import merge, split

LAYOUT_PADDED = 2


def place_codes(lengths_per_element, chunk_bytes: int):
    """Start bit of every code in the padded layout, and the stream length.

    Walks the chunks in order: a chunk takes the codes that follow in element
    order for as long as their lengths add up to at most 8C bits."""
    l = np.asarray(lengths_per_element, dtype=np.int64)
    bits = 8 * chunk_bytes
    if l.size and l.max() > bits:
        raise ValueError("a code is longer than a chunk")
    flat_start, _ = st.code_starts(l)
    flat_end = flat_start + l
    starts = np.empty(l.size, dtype=np.int64)
    first, chunk = 0, 0
    while first < l.size:
        # elements first..last-1 are the longest run whose codes fit in 8C bits
        last = int(np.searchsorted(flat_end, flat_start[first] + bits, side="right"))
        starts[first:last] = chunk * bits + (flat_start[first:last] - flat_start[first])
        first, chunk = last, chunk + 1
    total_bits = int(starts[-1] + l[-1]) if l.size else 0
    return starts, total_bits


def tail_gaps(starts, lengths_per_element, chunk_bytes: int):
    """(first bit, length) of every unused chunk tail before the last code:
    the bits between the last code of a chunk and the chunk's end, for every
    chunk followed by another chunk that holds codes."""
    l = np.asarray(lengths_per_element, dtype=np.int64)
    s = np.asarray(starts, dtype=np.int64)
    bits = 8 * chunk_bytes
    if s.size < 2:
        return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64)
    ends = s[:-1] + l[:-1]
    moved = (s[1:] % bits == 0) & (s[1:] != ends)
    g0 = ends[moved]
    return g0, s[1:][moved] - g0


def pack_at(starts, values, lengths, n_words: int) -> np.ndarray:
    """Words holding bit strings ``values`` (right-aligned, ``lengths`` bits,
    at most 32) at stream bits ``starts``, MSB first, none overlapping.

    A string of length l <= 32 that starts at bit p lies inside the 64-bit
    pair of words p // 32 and p // 32 + 1; adding the two shifted halves into
    the word array equals OR-ing the bits because no two strings share a bit
    (float64 sums are exact below 2^53)."""
    s = np.asarray(starts, dtype=np.int64)
    l = np.asarray(lengths, dtype=np.int64)
    v = np.asarray(values, dtype=np.uint64)
    r = (s & 31).astype(np.uint64)
    x = v << (np.uint64(64) - r - l.astype(np.uint64))
    hi = (x >> np.uint64(32)).astype(np.float64)
    lo = (x & np.uint64(0xFFFFFFFF)).astype(np.float64)
    k = s >> 5
    acc = np.bincount(k, weights=hi, minlength=n_words + 1)
    acc[1:] += np.bincount(k, weights=lo, minlength=n_words)[:n_words]
    out = acc[:n_words].astype(np.uint64)
    if (out > 0xFFFFFFFF).any():
        raise AssertionError("overlapping bit strings")
    return out.astype(np.uint32)


def encode_padded(bits, chunk_bytes: int = 16, lanes: int = 64, max_len: int = cb.MAX_LEN,
                  lengths=None):
    """Like ``stream.encode`` for the padded layout; ``off`` is None."""
    if chunk_bytes not in (4, 8, 16, 32):
        raise ValueError("chunk size must be 4, 8, 16 or 32 bytes")
    if lanes not in (64, 128, 256):
        raise ValueError("lanes per block must be 64, 128 or 256")
    exponent, raw = split(bits)
    n = exponent.size
    hist = cb.histogram(exponent)
    if lengths is None:
        lengths = cb.package_merge_lengths(hist, max_len)
    lengths = np.asarray(lengths, dtype=np.uint8)
    if n and (lengths[exponent] == 0).any():
        raise ValueError("an exponent has no code")
    codes = cb.canonical_codes(lengths)
    l = lengths.astype(np.int64)[exponent]
    starts, total_bits = place_codes(l, chunk_bytes)
    _, n_blocks, n_chunks = st.layout_sizes(total_bits, chunk_bytes, lanes)
    n_words = n_chunks * (chunk_bytes // 4) + st.GUARD_WORDS
    g0, gl = tail_gaps(starts, l, chunk_bytes)
    ones = (np.uint64(1) << gl.astype(np.uint64)) - np.uint64(1)
    words = pack_at(np.concatenate([starts, g0]),
                    np.concatenate([np.asarray(codes, dtype=np.uint64)[exponent], ones]),
                    np.concatenate([l, gl]), n_words)
    out = st.block_out(starts, n, chunk_bytes, lanes, n_blocks)
    return {
        "n": n,
        "chunk_bytes": chunk_bytes,
        "lanes": lanes,
        "max_len_limit": max_len,
        "hist": hist,
        "lengths": lengths,
        "codes": codes,
        "total_bits": total_bits,
        "n_blocks": n_blocks,
        "n_chunks": n_chunks,
        "words": words,
        "off": None,
        "out": out,
        "raw": raw,
        "starts": starts,
    }


def write_padded_blob(enc, lut_bits: int = 11, rows: int | None = None, cols: int | None = None) -> bytes:
    """The container of a padded-layout encoding (offsets section empty)."""
    return bl.write_blob(enc, lut_bits, rows, cols, layout=LAYOUT_PADDED)


# ------------------------------------------------------------------ decoders

def decode_padded_plain(words, total_bits: int, chunk_bytes: int, n_chunks: int, lengths) -> np.ndarray:
    """Chunk by chunk, one code at a time (pure Python; small inputs only)."""
    t = cb.canonical_tables(lengths)
    ws = [int(x) for x in np.asarray(words)]
    bits = 8 * chunk_bytes
    out = []
    for i in range(n_chunks):
        pos, end = i * bits, min((i + 1) * bits, total_bits)
        while pos < end:
            sym, l = cb.decode_window(st._read_bits(ws, pos, cb.MAX_LEN), t)
            if pos + l > end:
                break
            out.append(sym)
            pos += l
    return np.array(out, dtype=np.uint8)


def decode_padded(words, total_bits: int, chunk_bytes: int, n_chunks: int, lengths,
                  return_counts: bool = False):
    """The same decode vectorised across chunks with numpy (one code per
    chunk per iteration); per-chunk outputs concatenated in chunk order."""
    t = cb.canonical_tables(lengths)
    limit = np.array(t["limit"][1:], dtype=np.int64)          # index l - 1
    first = np.array(t["first"], dtype=np.int64)
    base = np.array(t["base"], dtype=np.int64)
    order = np.array(t["order"] if t["order"] else [0], dtype=np.uint8)
    w = np.asarray(words, dtype=np.uint64)
    bits = 8 * chunk_bytes
    i = np.arange(n_chunks, dtype=np.int64)
    pos = i * bits
    end = np.minimum((i + 1) * bits, total_bits)
    active = pos < end
    syms, valid = [], []
    last_word = w.size - 2
    while active.any():
        k = np.minimum(pos >> 5, last_word)
        pair = (w[k] << np.uint64(32)) | w[k + 1]
        shift = (np.int64(40) - (pos & 31)).astype(np.uint64)
        w24 = ((pair >> shift) & np.uint64(0xFFFFFF)).astype(np.int64)
        # the first length whose limit exceeds the window; past every limit
        # (bits no code starts with) the window counts as 24 bits long
        below = w24[:, None] < limit[None, :]
        l = np.where(below.any(axis=1), np.argmax(below, axis=1) + 1, cb.MAX_LEN)
        idx = np.clip(base[l] + (w24 >> (cb.MAX_LEN - l)) - first[l], 0, order.size - 1)
        active = active & (pos + l <= end)
        syms.append(np.where(active, order[idx], 0).astype(np.uint8))
        valid.append(active.copy())
        pos = np.where(active, pos + l, pos)
        active = active & (pos < end)
    if syms:
        s = np.stack(syms, axis=1)
        v = np.stack(valid, axis=1)
        result = s[v]
        counts = v.sum(axis=1)
    else:
        result = np.zeros(0, dtype=np.uint8)
        counts = np.zeros(n_chunks, dtype=np.int64)
    return (result, counts) if return_counts else result


def decode_padded_blob(blob: bytes) -> np.ndarray:
    """Original bf16 bit patterns from a padded-layout container."""
    p = bl.parse_blob(blob)
    if p["layout"] != LAYOUT_PADDED:
        raise ValueError("not a padded-layout container")
    e = decode_padded(p["words"], p["total_bits"], p["chunk_bytes"], p["n_chunks"], p["lengths"])
    if e.size != p["n"]:
        raise ValueError("decoded count does not match n")
    return merge(e, p["raw"])
