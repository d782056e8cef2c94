"""Interleaved rANS coding of the exponent bytes (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the entropy-coding family the method belongs to -- Huffman-
or arithmetic-like coding adapted for real-time GPU use (DFloat11 blog,
section 02) -- and the ANS-based decoder bridge of the VcLLM page's
introduction.  This module is the range variant of asymmetric numeral
systems (rANS), with the readings below; where the pages give no detail the
plainest standard choice is taken.

* Sign and mantissa stay one raw byte, exactly as in the Huffman layouts; only
  the 8-bit exponent is coded.
* Probabilities are the exponent histogram quantised to integers f[s] that
  sum to M = 2^12 (``quantize_freqs``: proportional shares rounded down, at
  least 1 for a present symbol, the remainder to the largest fractional
  parts, an excess taken back from the largest shares); cum[s] is the sum of
  f over the symbols below s.
* State x is an integer in [L, 2^32) with L = 2^16; the stream is 16-bit
  words.  Encoding symbol s: if x >= f[s] * 2^20, emit x mod 2^16 and set
  x = x // 2^16 (at most once); then x = (x // f[s]) * M + x mod f[s] +
  cum[s].  Decoding inverts it: slot = x mod M, s is the symbol with cum[s]
  <= slot < cum[s] + f[s], x = f[s] * (x // M) - cum[s] + slot, and if x < L
  the next word w is read: x = x * 2^16 + w.
* Interleaving: a block is W = 64 lanes x S steps of elements; element
  j = i * W + l of the block (step i, lane l) is coded by lane l's state.
  All lanes of a block share one word stream, read in decode order: step 0
  lanes 0..W-1 (each lane that needs a word takes the next one), then
  step 1, and so on.  The encoder runs the same sequence backwards (steps
  from last to first, lanes from W-1 down to 0, every lane starting from
  x = L) and reverses its output; the lanes' final encoder states are the
  decoder's initial states.  In a block's last step only the lanes whose
  element exists take part.
* Container (header layout field 3): the code-lengths area is zero; the
  tables section holds f[256] (u16), from which a decoder builds whatever
  slot lookup it uses; the words section holds every block's stream (u16) back to back, the offsets
  section the first word of every block (u32, n_blocks + 1 entries), the
  blockout section the W initial states of every block (u32), the raw
  section the raw bytes.  Header: chunk_bytes = 0, lanes_per_block = W,
  tile_k = S, total_bits = 16 * stream words, n_chunks = 0.
"""
from __future__ import annotations

import struct

import numpy as np

from . import blob as bl
from . import codebook as cb
from .fields import merge, split

LAYOUT_ANS = 3
PROB_BITS = 12
M = 1 << PROB_BITS
L = 1 << 16
WORD_BITS = 16
LANES = 64


def quantize_freqs(hist, prob_bits: int = PROB_BITS) -> np.ndarray:
    """Integer frequencies summing to 2^prob_bits, >= 1 for every present
    symbol and 0 for the others (all zero for an empty histogram)."""
    h = [int(v) for v in np.asarray(hist, dtype=np.uint64)]
    total = sum(h)
    m = 1 << prob_bits
    f = [0] * 256
    if total == 0:
        return np.zeros(256, dtype=np.uint32)
    present = [s for s in range(256) if h[s] > 0]
    if len(present) > m:
        raise ValueError("more symbols than probability slots")
    for s in present:
        f[s] = max(1, h[s] * m // total)
    d = m - sum(f)
    if d > 0:
        # largest remainders of h * m / total first, smaller symbol on ties
        order = sorted(present, key=lambda s: (-(h[s] * m % total), s))
        for s in order[:d]:
            f[s] += 1
    while d < 0:
        # take one from the largest share (smaller symbol on ties)
        s = max(present, key=lambda t: (f[t], -t))
        f[s] -= 1
        d += 1
    return np.array(f, dtype=np.uint32)


def cumulative(f) -> np.ndarray:
    f = np.asarray(f, dtype=np.int64)
    c = np.zeros(256, dtype=np.int64)
    c[1:] = np.cumsum(f)[:-1]
    return c


def symbol_of_slot(f) -> np.ndarray:
    f = np.asarray(f, dtype=np.int64)
    return np.repeat(np.arange(256), f).astype(np.int64)


# ----------------------------------------------------------- one lane (plain)

def encode_symbol(x: int, s: int, f, c, out: list) -> int:
    fs, cs = int(f[s]), int(c[s])
    if x >= fs << (32 - PROB_BITS):          # f * 2^20: the state would overflow
        out.append(x & 0xFFFF)
        x >>= WORD_BITS
    return (x // fs) * M + x % fs + cs


def decode_symbol(x: int, f, c, sym_of_slot, words, pos: int):
    """(symbol, new state, new read position)."""
    slot = x % M
    s = int(sym_of_slot[slot])
    x = int(f[s]) * (x // M) + slot - int(c[s])
    if x < L:
        x = (x << WORD_BITS) | int(words[pos])
        pos += 1
    return s, x, pos


# ------------------------------------------------------------- interleaved

def encode_block_plain(symbols, f, lanes: int = LANES):
    """One block, pure Python: (initial decoder states, words in decode order)."""
    c = cumulative(f)
    sym = [int(v) for v in symbols]
    n = len(sym)
    steps = -(-n // lanes)
    x = [L] * lanes
    out = []
    for i in range(steps - 1, -1, -1):
        for l in range(lanes - 1, -1, -1):
            j = i * lanes + l
            if j < n:
                x[l] = encode_symbol(x[l], sym[j], f, c, out)
    out.reverse()
    return x, out


def decode_block_plain(states, words, n: int, f, lanes: int = LANES):
    c = cumulative(f)
    sos = symbol_of_slot(f)
    x = [int(v) for v in states]
    pos = 0
    out = [0] * n
    for i in range(-(-n // lanes)):
        for l in range(lanes):
            j = i * lanes + l
            if j < n:
                out[j], x[l], pos = decode_symbol(x[l], f, c, sos, words, pos)
    if pos != len(words):
        raise ValueError("stream not fully consumed")
    return np.array(out, dtype=np.uint8), x


def encode_ans(bits, steps: int = 1024, lanes: int = LANES, freqs=None):
    """Split, quantise, and code every block (blocks of lanes * steps
    elements).  Returns a dict of numpy arrays."""
    if lanes != LANES:
        raise ValueError("64 lanes per block")
    if steps <= 0 or steps % 8:
        raise ValueError("steps per block must be a positive multiple of 8")
    exponent, raw = split(bits)
    n = exponent.size
    hist = cb.histogram(exponent)
    f = quantize_freqs(hist) if freqs is None else np.asarray(freqs, dtype=np.uint32)
    if n and (f[exponent] == 0).any():
        raise ValueError("an exponent has no probability slot")
    per = lanes * steps
    n_blocks = -(-n // per)
    states = np.zeros((n_blocks, lanes), dtype=np.uint32)
    parts, offsets = [], [0]
    for b in range(n_blocks):
        x, w = encode_block_stream(exponent[b * per: (b + 1) * per], f, lanes)
        states[b] = x
        parts.append(w)
        offsets.append(offsets[-1] + w.size)
    words = np.concatenate(parts).astype(np.uint16) if parts else np.zeros(0, dtype=np.uint16)
    return {
        "n": n, "lanes": lanes, "steps": steps, "hist": hist, "freqs": f,
        "n_blocks": n_blocks, "states": states, "offsets": np.array(offsets, dtype=np.uint32),
        "words": words, "raw": raw,
    }


def encode_block_stream(symbols, f, lanes: int = LANES):
    """``encode_block_plain`` with numpy across lanes: the lanes of one step
    are independent except for the order of their words, which is fixed
    afterwards (each lane emits at most one word per step)."""
    f64 = np.asarray(f, dtype=np.uint64)
    c64 = cumulative(f).astype(np.uint64)
    sym = np.asarray(symbols, dtype=np.int64)
    n = sym.size
    steps = -(-n // lanes)
    x = np.full(lanes, L, dtype=np.uint64)
    out = []
    for i in range(steps - 1, -1, -1):
        j = i * lanes + np.arange(lanes)
        live = j < n
        s = np.where(live, sym[np.minimum(j, n - 1)], 0)
        fs, cs = f64[s], c64[s]
        emit = live & (x >= (fs << np.uint64(32 - PROB_BITS)))
        # words of this step, lanes W-1 .. 0 (encoder order)
        out.append((x[emit] & np.uint64(0xFFFF))[::-1])
        x = np.where(emit, x >> np.uint64(WORD_BITS), x)
        fs1 = np.where(live, fs, np.uint64(1))
        x = np.where(live, (x // fs1) * np.uint64(M) + x % fs1 + cs, x)
    w = np.concatenate(out)[::-1] if out else np.zeros(0, dtype=np.uint64)
    return x.astype(np.uint32), w.astype(np.uint16)


def decode_ans(enc) -> np.ndarray:
    """Exponent bytes of every block, numpy across blocks and lanes, one step
    at a time; each needing lane takes the next word of its block's stream in
    lane order (its rank among the block's needing lanes)."""
    f = np.asarray(enc["freqs"], dtype=np.int64)
    c = cumulative(f)
    sos = symbol_of_slot(f) if f.sum() else np.zeros(M, dtype=np.int64)
    n, lanes, steps = enc["n"], enc["lanes"], enc["steps"]
    nb = enc["n_blocks"]
    out = np.zeros(nb * lanes * steps, dtype=np.uint8)
    if nb == 0:
        return out[:0]
    words = np.asarray(enc["words"], dtype=np.int64)
    x = np.asarray(enc["states"], dtype=np.int64).copy()
    pos = np.asarray(enc["offsets"], dtype=np.int64)[:-1].copy()
    per = lanes * steps
    count = np.minimum(per, n - per * np.arange(nb))[:, None]
    lane = np.arange(lanes)[None, :]
    for i in range(steps):
        live = i * lanes + lane < count
        if not live.any():
            break
        slot = x % M
        s = sos[slot]
        xn = f[s] * (x // M) + slot - c[s]
        need = live & (xn < L)
        rank = np.cumsum(need, axis=1) - need
        idx = np.minimum(pos[:, None] + rank, max(words.size - 1, 0))
        w = words[idx] if words.size else np.zeros_like(idx)
        xn = np.where(need, (xn << WORD_BITS) | w, xn)
        x = np.where(live, xn, x)
        pos += need.sum(axis=1)
        blk = np.arange(nb)[:, None] * per + i * lanes + lane
        out[blk[live]] = s[live]
    if not np.array_equal(pos, np.asarray(enc["offsets"], dtype=np.int64)[1:]):
        raise ValueError("a block's stream was not consumed exactly")
    return out[:n]


# ---------------------------------------------------------------- container

def tables_bytes() -> int:
    return 2 * 256


def write_ans_blob(enc, rows: int | None = None, cols: int | None = None) -> bytes:
    n = enc["n"]
    if rows is None or cols is None:
        rows, cols = 1, n
    if rows * cols != n:
        raise ValueError("rows * cols != n")
    nw = int(enc["words"].size)
    sizes = {
        "tables": tables_bytes(),
        "words": 2 * (-(-nw // 8) * 8 + 8),          # whole 16-byte units + one guard unit
        "offsets": 4 * (enc["n_blocks"] + 1),
        "blockout": 4 * enc["lanes"] * enc["n_blocks"],
        "raw": 16 * (-(-n // 16)),
        "panels": 0,
    }
    names = ("tables", "words", "offsets", "blockout", "raw", "panels")
    offsets = {}
    pos = bl.HEADER_BYTES
    for name in names:
        pos = bl._align(pos)
        offsets[name] = pos if sizes[name] else 0
        pos += sizes[name]
    blob_bytes = bl._align(pos)
    buf = bytearray(blob_bytes)
    struct.pack_into("<IIQQQQIIIIIIQQII", buf, 0,
                     bl.MAGIC, bl.VERSION, n, WORD_BITS * nw, 0, enc["n_blocks"],
                     0, enc["lanes"], 0, PROB_BITS, LAYOUT_ANS, 0, rows, cols, enc["steps"], 0)
    fields = []
    for name in names:
        fields += [offsets[name], sizes[name]]
    struct.pack_into("<12QQ", buf, 88, *fields, blob_bytes)

    def put(name, data: bytes):
        o = offsets[name]
        buf[o: o + len(data)] = data

    put("tables", np.asarray(enc["freqs"], dtype="<u2").tobytes())
    put("words", np.asarray(enc["words"], dtype="<u2").tobytes())
    put("offsets", np.asarray(enc["offsets"], dtype="<u4").tobytes())
    put("blockout", np.asarray(enc["states"], dtype="<u4").tobytes())
    put("raw", np.asarray(enc["raw"], dtype=np.uint8).tobytes())
    return bytes(buf)


def parse_ans_blob(blob: bytes):
    p = bl.parse_blob(blob)
    if p["layout"] != LAYOUT_ANS:
        raise ValueError("not an ANS container")
    b = bytes(blob)
    sec = p["sections"]
    to, _ = sec["tables"]
    freqs = np.frombuffer(b, dtype="<u2", count=256, offset=to).astype(np.uint32)
    nw = p["total_bits"] // WORD_BITS
    words = np.frombuffer(b, dtype="<u2", count=nw, offset=sec["words"][0]).copy() if nw else np.zeros(0, np.uint16)
    nb = p["n_blocks"]
    offsets = np.frombuffer(b, dtype="<u4", count=nb + 1, offset=sec["offsets"][0]).copy()
    states = (np.frombuffer(b, dtype="<u4", count=nb * p["lanes"], offset=sec["blockout"][0]).reshape(nb, p["lanes"])
              if nb else np.zeros((0, p["lanes"]), dtype=np.uint32))
    return {"n": p["n"], "lanes": p["lanes"], "steps": p["tile_k"], "freqs": freqs, "n_blocks": nb,
            "states": states, "offsets": offsets, "words": words, "raw": p["raw"]}


def decode_ans_blob(blob: bytes) -> np.ndarray:
    p = parse_ans_blob(blob)
    return merge(decode_ans(p), p["raw"])


def coded_bytes(enc) -> int:
    """Header, frequencies and the words, offsets, states and raw sections
    (alignment padding between sections is not counted)."""
    nw = int(enc["words"].size)
    return (bl.HEADER_BYTES + 512 + 2 * (-(-nw // 8) * 8 + 8) + 4 * (enc["n_blocks"] + 1) +
            4 * enc["lanes"] * enc["n_blocks"] + 16 * (-(-int(enc["n"]) // 16)))
