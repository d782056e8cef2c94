"""Pins for the oracle's interleaved rANS coder of the exponent bytes:
hand-worked states and words (one and two lanes), hand-worked frequency
quantisation cases, the largest-remainder rule by brute force, a plain
one-symbol-at-a-time decoder, the
information the stream and final states carry against the ideal code
length, and exact round trips."""
import json
import math
import os

import numpy as np
import pytest

from lossless_entropy_coded_dfc_amd import synth
from oracle import ans
from oracle import blob as bl
from oracle import codebook as cb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rans_two_symbols.json")


def golden():
    g = json.load(open(GOLDEN))
    f = np.zeros(256, dtype=np.uint32)
    for s, v in g["freqs"].items():
        f[int(s)] = v
    return g, f


@pytest.mark.parametrize("case", ["no_word", "one_word", "two_lanes"])
def test_golden_states_and_words(case):
    g, f = golden()
    c = g["cases"][case]
    want_w = [int(h, 16) for h in c["words_hex"]]
    x, w = ans.encode_block_plain(c["symbols"], f, c["lanes"])
    assert x == c["states"] and w == want_w
    xs, ws = ans.encode_block_stream(c["symbols"], f, c["lanes"])
    assert xs.tolist() == c["states"] and ws.tolist() == want_w
    d, end = ans.decode_block_plain(c["states"], want_w, len(c["symbols"]), f, c["lanes"])
    assert d.tolist() == c["symbols"]
    assert end == [ans.L] * c["lanes"]         # every lane returns to the encoder's start


def test_quantize_hand_cases():
    def q(pairs):
        h = np.zeros(256, dtype=np.uint64)
        for s, v in pairs.items():
            h[s] = v
        f = ans.quantize_freqs(h)
        return {s: int(f[s]) for s in range(256) if f[s]}

    assert q({0: 3, 1: 1}) == {0: 3072, 1: 1024}
    # 4096 * 10^6 / (10^6 + 1) = 4095.99..: floor 4095, the rare symbol's 0 becomes 1
    assert q({0: 10 ** 6, 1: 1}) == {0: 4095, 1: 1}
    # three equal shares of 1365.33: one unit left, smallest symbol first
    assert q({5: 1, 7: 1, 9: 1}) == {5: 1366, 7: 1365, 9: 1365}
    # 255 rare symbols raised to 1 overshoot by 254, taken from the large share
    big = {0: 10 ** 9}
    big.update({s: 1 for s in range(1, 256)})
    got = q(big)
    assert got[0] == 4095 - 254 and all(got[s] == 1 for s in range(1, 256))
    assert q({200: 12345}) == {200: 4096}
    assert not ans.quantize_freqs(np.zeros(256, dtype=np.uint64)).any()


def take_back_tie_histogram():
    """Two equal large symbols (10 and 20, 10^6 each) and 101 rare ones
    (100..200, one each): n = 2,000,101; 4096 * 10^6 / n = 2047.90, so both
    large shares floor to 2047 and the rare ones are raised to 1, summing to
    4094 + 101 = 4195.  The 99 units of excess are taken one at a time from
    the largest share, the smaller symbol first on ties: symbol 10 gives on
    the 1st, 3rd, ... 99th take (50 units), symbol 20 on the others (49)."""
    h = np.zeros(256, dtype=np.uint64)
    h[10] = h[20] = 10 ** 6
    h[100:201] = 1
    return h


def test_quantize_take_back_ties_go_to_the_smaller_symbol():
    f = ans.quantize_freqs(take_back_tie_histogram())
    assert int(f[10]) == 2047 - 50 and int(f[20]) == 2047 - 49
    assert all(int(f[s]) == 1 for s in range(100, 201))
    assert int(f.sum()) == 4096


def test_quantize_is_largest_remainder_when_no_share_rounds_to_zero():
    rng = np.random.default_rng(90)
    for _ in range(200):
        k = int(rng.integers(2, 40))
        h = np.zeros(256, dtype=np.uint64)
        syms = rng.choice(256, size=k, replace=False)
        h[syms] = rng.integers(10 ** 5, 10 ** 6, size=k)   # every share at least 10
        n = int(h.sum())
        f = ans.quantize_freqs(h)
        assert int(f.sum()) == ans.M
        floor = [int(h[s]) * ans.M // n for s in range(256)]
        assert all(floor[s] >= 1 for s in syms)
        extra = [s for s in range(256) if f[s] == floor[s] + 1]
        assert all(f[s] in (floor[s], floor[s] + 1) for s in range(256))
        d = ans.M - sum(floor)
        rem = sorted(syms.tolist(), key=lambda s: (-(int(h[s]) * ans.M % n), s))
        assert sorted(extra) == sorted(rem[:d])


def test_quantize_properties():
    rng = np.random.default_rng(91)
    for p in (0.01, 0.1, 0.5, 1.0):
        for _ in range(30):
            h = (rng.integers(0, 10 ** rng.integers(1, 9), 256) * (rng.random(256) < p)).astype(np.uint64)
            f = ans.quantize_freqs(h)
            if h.sum() == 0:
                assert not f.any()
                continue
            assert int(f.sum()) == ans.M
            assert ((f > 0) == (h > 0)).all()


def inputs():
    yield "outliers", synth.gaussian_with_outliers((37, 611), 0.02, (93,))
    yield "uniform", synth.uniform_bits((37, 611), (94,))
    yield "ladder", synth.exponent_ladder((37, 611), (95,))
    yield "t", synth.student_t((37, 611), 3.0, 0.02, (96,))
    yield "constant", np.full((37, 611), 0x3F80, dtype=np.uint16)


@pytest.mark.parametrize("steps", [8, 16, 64])
def test_numpy_coder_matches_plain_coder(steps):
    """The per-step numpy coder and decoder against the one-symbol-at-a-time
    definitions, block by block (partial last steps included)."""
    for name, x in inputs():
        enc = ans.encode_ans(x, steps)
        e = ((np.asarray(x, dtype=np.uint16).ravel() >> 7) & 0xFF).astype(np.uint8)
        per = 64 * steps
        for b in range(enc["n_blocks"]):
            seg = e[b * per: (b + 1) * per]
            xs, ws = ans.encode_block_plain(seg, enc["freqs"])
            assert list(enc["states"][b]) == xs, name
            o0, o1 = enc["offsets"][b], enc["offsets"][b + 1]
            assert enc["words"][o0:o1].tolist() == ws, name
            d, end = ans.decode_block_plain(xs, ws, seg.size, enc["freqs"])
            assert np.array_equal(d, seg) and end == [ans.L] * 64, name
        assert np.array_equal(ans.decode_ans(enc), e), name


def test_information_matches_ideal_code_length():
    """Stream bits plus the information held in the final states equal the
    ideal cost sum log2(M / f(s)) up to the coder's rounding."""
    for name, x in inputs():
        for steps in (8, 64, 512):
            enc = ans.encode_ans(x, steps)
            e = ((np.asarray(x, dtype=np.uint16).ravel() >> 7) & 0xFF)
            f = enc["freqs"].astype(np.float64)
            ideal = float(np.sum(np.log2(ans.M / f[e])))
            held = 16 * enc["words"].size + float(np.sum(np.log2(enc["states"].astype(np.float64) / ans.L)))
            assert abs(held - ideal) <= 1e-3 * ideal + 64 * enc["n_blocks"], (name, steps)


def test_states_in_range_and_words_per_step():
    x = synth.gaussian_with_outliers((128, 1024), 0.02, (97,))
    enc = ans.encode_ans(x, 64)
    assert (enc["states"] >= ans.L).all()
    # at most one word per element
    assert (np.diff(enc["offsets"].astype(np.int64)) <= 64 * 64).all()


@pytest.mark.parametrize("n", [0, 1, 2, 63, 64, 65, 511, 512, 513, 5000])
def test_container_round_trip_edge_sizes(n):
    x = synth.gaussian((n,), 0.02, (98, n))
    enc = ans.encode_ans(x, 8)
    blob = ans.write_ans_blob(enc)
    p = bl.parse_blob(blob)
    assert p["layout"] == ans.LAYOUT_ANS and p["tile_k"] == 8 and p["lanes"] == 64
    assert np.array_equal(ans.decode_ans_blob(blob), x.ravel())
    q = ans.parse_ans_blob(blob)
    assert np.array_equal(q["freqs"], enc["freqs"])
    # the frequencies are the only model the container carries
    assert p["sections"]["tables"][1] == 512


def test_size_near_entropy_bound():
    x = synth.gaussian_with_outliers((1024, 4096), 0.02, (99,))
    e = ((x.ravel() >> 7) & 0xFF).astype(np.uint8)
    bound = bl.entropy_bound_bytes(cb.histogram(e))
    for steps, lim in ((256, 1.012), (512, 1.006), (1024, 1.004)):
        assert 1.0 < ans.coded_bytes(ans.encode_ans(x, steps)) / bound < lim, steps


def test_specials_and_foreign_frequencies():
    specials = np.array([0x7FC1, 0xFF81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16)
    x = np.tile(specials, 1001)
    assert np.array_equal(ans.decode_ans_blob(ans.write_ans_blob(ans.encode_ans(x, 16))), x)
    f = ans.quantize_freqs(np.arange(256, dtype=np.uint64) + 1)
    y = synth.uniform_bits((50, 300), (100,))
    enc = ans.encode_ans(y, 32, freqs=f)
    assert np.array_equal(ans.decode_ans_blob(ans.write_ans_blob(enc)), y.ravel())
    with pytest.raises(ValueError):
        ans.encode_ans(y, 32, freqs=ans.quantize_freqs(np.eye(256, dtype=np.uint64)[3]))
