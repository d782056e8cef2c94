"""Bitstream packing, chunk/block metadata and the two reference decoders
(oracle).

Layout (DFloat11 blog, section 03 item 2: a first phase in which threads
agree on read and write positions through small auxiliary variables, so that
many threads decode one stream in parallel).  Readings that fix the details:

* codes are concatenated in element order, most significant bit first; stream
  bit b is bit (31 - b mod 32) of 32-bit word b // 32, words little-endian;
* the stream is cut into chunks of C bytes (8C bits); chunk i covers stream
  bits [8Ci, 8C(i+1)); a code belongs to the chunk that holds its first bit
  and may run up to 23 bits into the next chunk;
* ``off[i]`` (5 bits) is the distance from the chunk's first bit to the start
  of its first code: (first code start >= 8Ci, or total_bits if there is
  none) - 8Ci for chunks that start before total_bits, and 0 for chunks that
  start at or after it;
* a block is T consecutive chunks; ``out[b]`` (32 bits) is the number of
  codes that start before bit 8CTb, and ``out[n_blocks] = n``;
* the stream is zero-padded to a whole number of blocks, so the number of
  chunks is a multiple of T.

Chunk i therefore decodes the codes that start in
[8Ci + off[i], min(8C(i+1) + off[i+1], total_bits)).
"""
from __future__ import annotations

import numpy as np

from . import codebook as cb
from .fields import split

GUARD_WORDS = 4


def layout_sizes(total_bits: int, chunk_bytes: int, lanes: int):
    """(chunks that hold stream bits, blocks, chunks after padding)."""
    bits = 8 * chunk_bytes
    used = -(-total_bits // bits)
    blocks = -(-used // lanes)
    return used, blocks, blocks * lanes


def code_starts(code_len_per_element: np.ndarray):
    """Start bit of every code and the total number of bits."""
    l = np.asarray(code_len_per_element, dtype=np.int64)
    starts = np.zeros(l.size, dtype=np.int64)
    if l.size:
        np.cumsum(l[:-1], out=starts[1:])
    return starts, int(l.sum())


def pack_bits_plain(exponent, lengths, codes, n_words: int):
    """Bit-by-bit packer (pure Python; small inputs only)."""
    words = [0] * n_words
    pos = 0
    for e in np.asarray(exponent).ravel():
        l = int(lengths[int(e)])
        c = int(codes[int(e)])
        for k in range(l):
            bit = (c >> (l - 1 - k)) & 1
            if bit:
                words[pos >> 5] |= 1 << (31 - (pos & 31))
            pos += 1
    return np.array(words, dtype=np.uint32)


def pack_words(exponent, lengths, codes, n_words: int) -> np.ndarray:
    """Vectorised packer.

    A code of length l <= 24 that starts at bit p lies inside the 64-bit pair
    formed by words p//32 and p//32 + 1.  Shifting it to its place in that
    pair and adding the two halves into the word array gives the same words as
    OR-ing bits, because codes never share a bit.  Sums are accumulated in
    float64, which is exact below 2^53.
    """
    e = np.asarray(exponent, dtype=np.uint8).ravel()
    l = np.asarray(lengths, dtype=np.int64)[e]
    c = np.asarray(codes, dtype=np.uint64)[e]
    starts, _ = code_starts(l)
    r = (starts & 31).astype(np.uint64)
    v = c << (np.uint64(64) - r - l.astype(np.uint64))
    hi = (v >> np.uint64(32)).astype(np.float64)
    lo = (v & np.uint64(0xFFFFFFFF)).astype(np.float64)
    k = starts >> 5
    acc = np.bincount(k, weights=hi, minlength=n_words + 1)
    acc[1:] += np.bincount(k, weights=lo, minlength=n_words)[: n_words]
    out = acc[:n_words].astype(np.uint64)
    if (out > 0xFFFFFFFF).any():
        raise AssertionError("overlapping codes")
    return out.astype(np.uint32)


def chunk_offsets(starts: np.ndarray, total_bits: int, chunk_bytes: int,
                  n_chunks: int) -> np.ndarray:
    """off[0..n_chunks] (uint8, the extra last entry is 0)."""
    bits = 8 * chunk_bytes
    off = np.zeros(n_chunks + 1, dtype=np.uint8)
    chunk_first = np.arange(n_chunks, dtype=np.int64) * bits
    live = chunk_first < total_bits
    # The first code start at or after each live chunk's first bit; past the
    # last code that is total_bits.
    idx = np.searchsorted(starts, chunk_first[live], side="left")
    first_start = np.append(starts, total_bits)[idx]
    off[: n_chunks][live] = (first_start - chunk_first[live]).astype(np.uint8)
    return off


def block_out(starts: np.ndarray, n: int, chunk_bytes: int, lanes: int,
              n_blocks: int) -> np.ndarray:
    """out[0..n_blocks] (uint32): codes starting before each block."""
    block_first = np.arange(n_blocks, dtype=np.int64) * (8 * chunk_bytes * lanes)
    out = np.empty(n_blocks + 1, dtype=np.uint64)
    out[:n_blocks] = np.searchsorted(starts, block_first, side="left")
    out[n_blocks] = n
    return out.astype(np.uint32)


def pack_offsets(off: np.ndarray) -> np.ndarray:
    """5-bit fields, field i at bits [5i, 5i+5) of a little-endian bit array of
    uint32 words (bit k of a word is its 2^k bit); one zero word of slack."""
    off = np.asarray(off, dtype=np.uint64)
    n_words = -(-5 * off.size // 32) + 1
    words = np.zeros(n_words, dtype=np.uint64)
    for k in range(5):
        g = 5 * np.arange(off.size, dtype=np.int64) + k
        bit = (off >> np.uint64(k)) & np.uint64(1)
        np.add.at(words, g >> 5, bit << (g & 31).astype(np.uint64))
    return words.astype(np.uint32)


def unpack_offsets(words: np.ndarray, count: int) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint64)
    g = 5 * np.arange(count, dtype=np.int64)
    pair = w[g >> 5] | (w[(g >> 5) + 1] << np.uint64(32))
    return ((pair >> (g & 31).astype(np.uint64)) & np.uint64(31)).astype(np.uint8)


def encode(bits, chunk_bytes: int = 16, lanes: int = 64, max_len: int = cb.MAX_LEN,
           lengths=None):
    """Split, histogram, build the code (unless ``lengths`` is given), pack and
    compute the metadata.  Returns a dict of numpy arrays and sizes."""
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
    starts, total_bits = code_starts(lengths.astype(np.int64)[exponent])
    _, n_blocks, n_chunks = layout_sizes(total_bits, chunk_bytes, lanes)
    n_words = n_chunks * (chunk_bytes // 4) + GUARD_WORDS
    words = pack_words(exponent, lengths, codes, n_words)
    off = chunk_offsets(starts, total_bits, chunk_bytes, n_chunks)
    out = block_out(starts, n, chunk_bytes, lanes, n_blocks)
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
        "off": off,
        "out": out,
        "raw": raw,
    }


# ------------------------------------------------------------------ decoders

def _read_bits(words, pos: int, nbits: int) -> int:
    """nbits stream bits starting at pos (zero past the end of ``words``)."""
    v = 0
    for b in range(pos, pos + nbits):
        k = b >> 5
        bit = (int(words[k]) >> (31 - (b & 31))) & 1 if k < len(words) else 0
        v = (v << 1) | bit
    return v


def decode_sequential(words, n: int, lengths) -> np.ndarray:
    """Metadata-free decoder: from bit 0 read n codes one after another
    (pure Python; small inputs only)."""
    t = cb.canonical_tables(lengths)
    ws = [int(x) for x in np.asarray(words)]
    pos = 0
    out = np.empty(n, dtype=np.uint8)
    for j in range(n):
        sym, l = cb.decode_window(_read_bits(ws, pos, cb.MAX_LEN), t)
        out[j] = sym
        pos += l
    return out


def decode_chunked(words, off, total_bits: int, chunk_bytes: int, n_chunks: int,
                   lengths, return_counts: bool = False):
    """Chunk-parallel decoder driven by the metadata.

    Every chunk decodes its own codes independently (vectorised across chunks
    with numpy: one code per chunk per iteration); the per-chunk outputs are
    concatenated in chunk order.
    """
    t = cb.canonical_tables(lengths)
    limit = np.array(t["limit"][1:], dtype=np.int64)          # index l - 1
    first = np.array(t["first"], dtype=np.int64)
    base = np.array(t["base"], dtype=np.int64)
    order = np.array(t["order"] if t["order"] else [0], dtype=np.uint8)
    w = np.asarray(words, dtype=np.uint64)
    off = np.asarray(off, dtype=np.int64)
    bits = 8 * chunk_bytes
    i = np.arange(n_chunks, dtype=np.int64)
    pos = i * bits + off[:n_chunks]
    end = np.minimum((i + 1) * bits + off[1: n_chunks + 1], total_bits)
    active = pos < end
    syms, valid = [], []
    last_word = w.size - 2
    while active.any():
        k = np.minimum(pos >> 5, last_word)
        pair = (w[k] << np.uint64(32)) | w[k + 1]
        shift = (np.int64(40) - (pos & 31)).astype(np.uint64)
        w24 = ((pair >> shift) & np.uint64(0xFFFFFF)).astype(np.int64)
        l = np.argmax(w24[:, None] < limit[None, :], axis=1) + 1
        idx = base[l] + (w24 >> (cb.MAX_LEN - l)) - first[l]
        idx = np.clip(idx, 0, order.size - 1)
        syms.append(np.where(active, order[idx], 0).astype(np.uint8))
        valid.append(active.copy())
        pos = np.where(active, pos + l, pos)
        active = pos < end
    if syms:
        s = np.stack(syms, axis=1)
        v = np.stack(valid, axis=1)
        result = s[v]
        counts = v.sum(axis=1)
    else:
        result = np.zeros(0, dtype=np.uint8)
        counts = np.zeros(n_chunks, dtype=np.int64)
    return (result, counts) if return_counts else result
