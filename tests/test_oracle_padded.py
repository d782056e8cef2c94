"""Pins for the oracle's offset-free padded-chunk layout: a hand-worked
golden stream, the unpadded concatenation against the flat layout's stream,
the padding rule checked bit by bit, the prefix property the decoder's stop
rests on, a plain one-code-at-a-time decoder and exact round trips."""
import json
import os

import numpy as np
import pytest

from lossless_entropy_coded_dfc_amd import synth
from oracle import blob as bl
from oracle import codebook as cb
from oracle import padded as pd
from oracle import stream as st

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "padded32.json")
CHUNKS = (4, 8, 16, 32)


def stream_bits(words, n_bits):
    """The first n_bits stream bits as a 0/1 array (MSB first per word)."""
    b = np.asarray(words, dtype=">u4").tobytes()
    return np.unpackbits(np.frombuffer(b, dtype=np.uint8))[:n_bits]


def golden_cases():
    g = json.load(open(GOLDEN))
    lengths = np.zeros(256, dtype=np.uint8)
    for s, l in g["lengths"].items():
        lengths[int(s)] = l
    return g, lengths


@pytest.mark.parametrize("case", ["pad1", "exact"])
def test_golden(case):
    g, lengths = golden_cases()
    c = g["cases"][case]
    e = np.array(c["exponent"], dtype=np.uint16)
    raw = np.arange(e.size, dtype=np.uint16) % 128 if c["raw"] == "index" else np.zeros(e.size, np.uint16)
    bits = (e << 7) | raw
    enc = pd.encode_padded(bits, g["chunk_bytes"], g["lanes"], lengths=lengths)
    assert enc["total_bits"] == c["total_bits"]
    assert enc["words"].size == c["n_words"]
    want = np.zeros(c["n_words"], dtype=np.uint32)
    want[: len(c["words_hex"])] = [int(h, 16) for h in c["words_hex"]]
    assert np.array_equal(enc["words"], want)
    assert enc["out"].tolist() == c["out"]
    g0, gl = pd.tail_gaps(enc["starts"], lengths[e.astype(np.uint8)], g["chunk_bytes"])
    assert [[int(a), int(b)] for a, b in zip(g0, gl)] == c["gaps"]
    for dec in (pd.decode_padded_plain(enc["words"], enc["total_bits"], 4, enc["n_chunks"], lengths),
                pd.decode_padded(enc["words"], enc["total_bits"], 4, enc["n_chunks"], lengths)):
        assert np.array_equal(dec, e.astype(np.uint8))
    _, counts = pd.decode_padded(enc["words"], enc["total_bits"], 4, enc["n_chunks"], lengths,
                                 return_counts=True)
    want_counts = np.zeros(enc["n_chunks"], dtype=np.int64)
    for i, k in c["chunk_counts"].items():
        want_counts[int(i)] = k
    assert np.array_equal(counts, want_counts)
    blob = pd.write_padded_blob(enc)
    assert np.array_equal(bl.decode_blob(blob), bits)


def inputs():
    shape = (97, 613)
    yield "outliers", synth.gaussian_with_outliers(shape, 0.02, (40,))
    yield "ladder", synth.exponent_ladder(shape, (41,))
    yield "uniform", synth.uniform_bits(shape, (42,))
    yield "t", synth.student_t(shape, 3.0, 0.02, (43,))
    yield "bimodal", synth.bimodal(shape, 0.02, (44,))


@pytest.mark.parametrize("C", CHUNKS)
def test_used_bits_concatenate_to_the_flat_stream(C):
    """Dropping every chunk's unused tail gives exactly the flat layout's
    stream (which the flat layout's own pins fix)."""
    for name, x in inputs():
        enc = pd.encode_padded(x, C)
        flat = st.encode(x, C)
        exponent = (np.asarray(x, dtype=np.uint16).ravel() >> 7) & 0xFF
        l = enc["lengths"].astype(np.int64)[exponent]
        bits = stream_bits(enc["words"], enc["words"].size * 32)
        used = np.zeros(bits.size, dtype=bool)
        for s, n in zip(enc["starts"], l):
            used[s: s + n] = True
        got = bits[used]
        want = stream_bits(flat["words"], flat["total_bits"])
        assert got.size == flat["total_bits"], name
        assert np.array_equal(got, want), name


@pytest.mark.parametrize("C", CHUNKS)
def test_padding_rule_bit_by_bit(C):
    """No code crosses a chunk boundary; every unused tail before the last
    code is all ones and shorter than the code that opens the next chunk;
    a chunk's codes start at its first bit; nothing follows total_bits."""
    W = 8 * C
    for name, x in inputs():
        enc = pd.encode_padded(x, C)
        exponent = (np.asarray(x, dtype=np.uint16).ravel() >> 7) & 0xFF
        l = enc["lengths"].astype(np.int64)[exponent]
        s = enc["starts"]
        assert ((s % W) + l <= W).all(), name
        assert (np.diff(s) >= l[:-1]).all(), name
        bits = stream_bits(enc["words"], enc["words"].size * 32)
        chunk_of = s // W
        # every chunk up to the last one that holds codes has a code at bit 0
        assert set(np.unique(chunk_of)) == set(range(int(chunk_of[-1]) + 1)), name
        firsts = np.flatnonzero(np.diff(chunk_of)) + 1
        assert (s[firsts] % W == 0).all() and s[0] == 0, name
        for j in firsts:
            gap0, gap1 = s[j - 1] + l[j - 1], s[j]
            assert gap1 - gap0 < l[j], name                  # the moved code did not fit
            assert bits[gap0:gap1].all(), name               # tail set to ones
        assert not bits[enc["total_bits"]:].any(), name
        assert enc["total_bits"] == s[-1] + l[-1]


def test_ones_prefix_never_ends_a_code():
    """The stop rule: for complete canonical codes, a window that starts with
    r ones (r below the longest length) holds a code longer than r, whatever
    follows."""
    rng = np.random.default_rng(45)
    hists = [rng.integers(0, 1000, 256) * (rng.random(256) < p) for p in (0.02, 0.1, 0.5, 1.0)]
    hists.append(np.r_[np.zeros(200), 2.0 ** np.arange(56)][:256][::-1])   # long codes
    hists.append(np.eye(256)[77] * 5)                                     # one symbol
    for h in hists:
        if h.sum() == 0:
            continue
        lengths = cb.package_merge_lengths(h.astype(np.int64), 24)
        t = cb.canonical_tables(lengths)
        L = int(lengths.max())
        for r in range(L):
            for _ in range(40):
                tail = int(rng.integers(0, 1 << (24 - r))) if r < 24 else 0
                w = (((1 << r) - 1) << (24 - r)) | tail
                _, got = cb.decode_window(w, t)
                assert got > r


@pytest.mark.parametrize("C", CHUNKS)
def test_vectorised_decoder_matches_plain(C):
    for name, x in inputs():
        x = x[:7, :211]
        enc = pd.encode_padded(x, C)
        exponent = ((np.asarray(x, dtype=np.uint16).ravel() >> 7) & 0xFF).astype(np.uint8)
        a = pd.decode_padded_plain(enc["words"], enc["total_bits"], C, enc["n_chunks"], enc["lengths"])
        b = pd.decode_padded(enc["words"], enc["total_bits"], C, enc["n_chunks"], enc["lengths"])
        assert np.array_equal(a, exponent), name
        assert np.array_equal(b, exponent), name


@pytest.mark.parametrize("T", [64, 128, 256])
def test_block_offsets_count_codes_before_each_block(T):
    x = synth.gaussian_with_outliers((300, 700), 0.02, (46, T))
    for C in CHUNKS:
        enc = pd.encode_padded(x, C, T)
        _, counts = pd.decode_padded(enc["words"], enc["total_bits"], C, enc["n_chunks"], enc["lengths"],
                                     return_counts=True)
        per_block = counts.reshape(-1, T).sum(axis=1)
        assert enc["out"].tolist() == np.r_[0, np.cumsum(per_block)].tolist()
        bound = 8 * C * T * np.arange(enc["n_blocks"])
        assert enc["out"][:-1].tolist() == [int((enc["starts"] < b).sum()) for b in bound]


def test_padding_costs_less_than_offsets():
    """Bits lost to padding stay below the longest code per chunk boundary,
    and on Gaussian-like weights below the 5-bit offsets they replace."""
    x = synth.gaussian_with_outliers((512, 1024), 0.02, (47,))
    for C in CHUNKS:
        enc = pd.encode_padded(x, C)
        flat = st.encode(x, C)
        waste = enc["total_bits"] - flat["total_bits"]
        used_chunks = -(-enc["total_bits"] // (8 * C))
        assert 0 <= waste <= (used_chunks - 1) * (int(enc["lengths"].max()) - 1)
        assert waste < 5 * (used_chunks + 1)


@pytest.mark.parametrize("n", [0, 1, 2, 15, 16, 17, 1000])
def test_edge_sizes_round_trip(n):
    for C in CHUNKS:
        x = synth.gaussian((n,), 0.02, (48, n))
        enc = pd.encode_padded(x, C)
        blob = pd.write_padded_blob(enc)
        p = bl.parse_blob(blob)
        assert p["layout"] == pd.LAYOUT_PADDED
        assert p["sections"]["offsets"] == (0, 0)
        assert np.array_equal(bl.decode_blob(blob), x.ravel())


def test_specials_constant_and_foreign_lengths():
    specials = np.array([0x7FC1, 0xFF81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16)
    for C in CHUNKS:
        for x in (np.tile(specials, 501), np.full(3001, 0x3F80, dtype=np.uint16)):
            assert np.array_equal(bl.decode_blob(pd.write_padded_blob(pd.encode_padded(x, C))), x)
    # a 24-bit-limited code over all 256 exponents, lengths from another tensor
    lengths = cb.package_merge_lengths((np.arange(256) + 1) ** 3, 24)
    x = synth.uniform_bits((50, 400), (49,))
    for C in CHUNKS:
        enc = pd.encode_padded(x, C, lengths=lengths)
        assert np.array_equal(bl.decode_blob(pd.write_padded_blob(enc)), x.ravel())
