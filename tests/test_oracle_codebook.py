"""Pins for the oracle's field split, histogram, length-limited code lengths and
canonical codes.  Each test checks the oracle against something other than
itself: exhaustive enumeration, brute-force optima, a textbook heap Huffman,
closed forms, and RFC 1951's worked example."""
import itertools
import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import fields


# ------------------------------------------------------------------ fields

def test_split_merge_identity_on_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    e, r = fields.split(bits)
    assert np.array_equal(fields.merge(e, r), bits)
    # every (exponent, raw) pair occurs exactly once: the split is a bijection
    assert np.unique(e.astype(np.int64) * 256 + r).size == 1 << 16


def test_split_known_values(golden):
    g = golden("dyadic8.json")
    bits = np.array([int(h, 16) for h in g["bf16_hex"]], dtype=np.uint16)
    e, r = fields.split(bits)
    assert e.tolist() == g["exponent"]
    assert r.tolist() == g["raw"]


@pytest.mark.parametrize("value,exp,raw", [
    (1.0, 127, 0x00), (-2.0, 128, 0x80), (0.0, 0, 0x00), (-0.0, 0, 0x80),
    (float("inf"), 255, 0x00), (float("-inf"), 255, 0x80),
])
def test_split_float_semantics(value, exp, raw):
    # float32 -> bf16 by truncation is exact for these values
    b = np.array([value], dtype=np.float32).view(np.uint32) >> 16
    e, r = fields.split(b.astype(np.uint16))
    assert (int(e[0]), int(r[0])) == (exp, raw)


def test_nan_payload_and_subnormal_survive():
    pats = np.array([0x7FC1, 0xFF81, 0x0001, 0x807F, 0x7F80], dtype=np.uint16)
    e, r = fields.split(pats)
    assert e.tolist() == [255, 255, 0, 0, 255]
    assert np.array_equal(fields.merge(e, r), pats)


# ------------------------------------------------------------- histogram

def test_histogram_and_entropy_closed_forms():
    e = np.array([3] * 8 + [7] * 4 + [9] * 2 + [11] * 2, dtype=np.uint8)
    h = cb.histogram(e)
    assert int(h.sum()) == e.size and h[3] == 8 and h[7] == 4
    assert cb.entropy_bits(h) == pytest.approx(1.75)
    uniform = np.ones(256, dtype=np.uint64)
    assert cb.entropy_bits(uniform) == pytest.approx(8.0)
    assert cb.entropy_bits(np.zeros(256, dtype=np.uint64)) == 0.0


# --------------------------------------------------------- optimal lengths

def brute_force_cost(weights, max_len):
    """Minimum sum(w*l) over all length vectors with Kraft sum <= 1."""
    best = None
    m = len(weights)
    for ls in itertools.product(range(1, max_len + 1), repeat=m):
        if sum(2.0 ** -l for l in ls) <= 1.0 + 1e-12:
            c = sum(w * l for w, l in zip(weights, ls))
            best = c if best is None else min(best, c)
    return best


def hist_from(weights, symbols=None):
    h = np.zeros(256, dtype=np.uint64)
    symbols = symbols if symbols is not None else list(range(len(weights)))
    for s, w in zip(symbols, weights):
        h[s] = w
    return h


@pytest.mark.parametrize("m", [2, 3, 4, 5, 6])
def test_package_merge_matches_brute_force(m):
    rng = np.random.default_rng((101, m))
    for trial in range(12):
        w = [int(x) for x in rng.integers(1, 60, size=m)]
        if trial % 3 == 0:
            w = [int(x) for x in rng.geometric(0.3, size=m)]  # skewed
        syms = sorted(rng.choice(256, size=m, replace=False).tolist())
        h = hist_from(w, syms)
        for L in range(max(1, math.ceil(math.log2(m))), 7):
            lens = cb.package_merge_lengths(h, L)
            assert lens[[s for s in range(256) if s not in syms]].sum() == 0
            assert int(lens.max()) <= L
            assert cb.kraft_numerator(lens, L) <= 1 << L
            assert cb.code_cost(h, lens) == brute_force_cost(w, L), (w, L)


def test_slack_limit_equals_textbook_huffman():
    rng = np.random.default_rng(7)
    for _ in range(40):
        m = int(rng.integers(2, 40))
        h = hist_from([int(x) for x in rng.integers(1, 10 ** 6, size=m)],
                      sorted(rng.choice(256, size=m, replace=False).tolist()))
        lens = cb.package_merge_lengths(h, 24)
        assert cb.code_cost(h, lens) == cb.huffman_cost(h)


def test_gaussian_weights_code_is_huffman_and_within_one_bit():
    from lossless_entropy_coded_dfc_amd import synth
    x = synth.gaussian((512, 1024), 0.02, (0,))
    e, _ = fields.split(x)
    h = cb.histogram(e)
    lens = cb.package_merge_lengths(h, 24)
    assert cb.code_cost(h, lens) == cb.huffman_cost(h)
    H = cb.entropy_bits(h)
    Lbar = cb.mean_code_length(h, lens)
    assert H <= Lbar < H + 1
    assert 2.4 < H < 2.7  # the low-entropy exponent of N(0, 0.02^2) weights


def test_kraft_equality_for_every_build():
    rng = np.random.default_rng(11)
    for trial in range(60):
        m = int(rng.integers(2, 257))
        syms = rng.choice(256, size=m, replace=False)
        w = rng.integers(1, 1 << int(rng.integers(1, 30)), size=m)
        h = hist_from([int(x) for x in w], syms.tolist())
        L = 24 if trial % 2 else max(8, math.ceil(math.log2(m)))
        lens = cb.package_merge_lengths(h, L)
        assert cb.kraft_numerator(lens, 24) == 1 << 24
        H, Lbar = cb.entropy_bits(h), cb.mean_code_length(h, lens)
        assert H <= Lbar + 1e-12
        if cb.huffman_depth(h) <= L:
            assert Lbar < H + 1


def test_dyadic_lengths_closed_form():
    # p_k = 2^-k (last two share 2^-(K-1)) -> optimal lengths are exactly -log2 p
    K = 12
    w = [1 << (K - k) for k in range(1, K)] + [2]   # sums to 2^K
    h = hist_from(w, list(range(100, 100 + len(w))))
    lens = cb.package_merge_lengths(h, 24)
    expect = [int(-math.log2(x / sum(w))) for x in w]
    assert [int(lens[100 + i]) for i in range(len(w))] == expect
    assert cb.mean_code_length(h, lens) == pytest.approx(cb.entropy_bits(h))


@pytest.mark.parametrize("counts,depth", [
    ([5], 1),                      # one symbol: one bit under the single-symbol reading
    ([1, 1], 1),
    ([1, 1, 1, 1], 2),             # balanced: 2 bits each
    ([1, 1, 1, 1, 1], 3),          # lengths 2, 2, 2, 3, 3
    ([4, 2, 1, 1], 3),             # dyadic: lengths 1, 2, 3, 3
    ([1, 1, 2, 4, 8], 4),          # doubling: 8 -> 1, 4 -> 2, 2 -> 3, 1 and 1 -> 4
    ([1] * 256, 8),
    ([1] * 257 + [0] * 3, 9),      # (counts past 256 symbols only for the tree)
])
def test_huffman_depth_hand_worked(counts, depth):
    """Depths of textbook Huffman trees worked by hand: the longest code of an
    optimal unconstrained code for these counts."""
    assert cb.huffman_depth(np.array(counts, dtype=np.uint64)) == depth


def test_huffman_depth_fibonacci_and_empty():
    # Fibonacci counts make the textbook tree a chain: each merge joins the
    # next leaf and the running package (fib[i + 1] < fib[i + 2] - 1 <
    # fib[i + 2]), so 40 leaves sit at depths 1 .. 39 (the two lightest at 39)
    fib = [1, 1]
    while len(fib) < 40:
        fib.append(fib[-1] + fib[-2])
    assert cb.huffman_depth(np.array(fib, dtype=np.uint64)) == 39
    assert cb.huffman_depth(np.array(fib[:25], dtype=np.uint64)) == 24
    assert cb.huffman_depth(np.zeros(256, dtype=np.uint64)) == 0
    # the depth equals the longest of the package-merge lengths whenever the
    # limit does not bind
    rng = np.random.default_rng(12)
    for _ in range(30):
        h = hist_from([int(x) for x in rng.integers(1, 1 << 12, 40)], list(range(40)))
        assert cb.huffman_depth(h) == int(cb.package_merge_lengths(h, 24).max())


def test_limit_binds_on_deep_ladder():
    # Fibonacci-like counts force an unconstrained depth > 24
    fib = [1, 1]
    while len(fib) < 40:
        fib.append(fib[-1] + fib[-2])
    h = hist_from(fib, list(range(40)))
    assert cb.huffman_depth(h) > 24
    lens = cb.package_merge_lengths(h, 24)
    assert int(lens.max()) == 24
    assert cb.kraft_numerator(lens, 24) == 1 << 24
    assert cb.code_cost(h, lens) >= cb.huffman_cost(h)
    # tighter limits never help
    assert cb.code_cost(h, cb.package_merge_lengths(h, 23)) >= cb.code_cost(h, lens)


def test_single_and_empty_alphabets():
    h = np.zeros(256, dtype=np.uint64)
    assert cb.package_merge_lengths(h, 24).sum() == 0
    h[255] = 1000
    lens = cb.package_merge_lengths(h, 24)
    assert lens[255] == 1 and lens[0] == 1 and lens.sum() == 2  # phantom wraps to 0
    assert cb.kraft_numerator(lens) == 1 << 24


# ------------------------------------------------------------- canonical

def test_rfc1951_worked_example(golden):
    g = golden("rfc1951_canonical.json")
    lens = np.zeros(256, dtype=np.uint8)
    lens[:8] = g["lengths"]
    codes = cb.canonical_codes(lens)
    got = [format(int(codes[i]), "0%db" % g["lengths"][i]) for i in range(8)]
    assert got == g["codes"]


def test_canonical_invariants():
    rng = np.random.default_rng(3)
    for _ in range(30):
        m = int(rng.integers(2, 200))
        h = hist_from([int(x) for x in rng.integers(1, 10 ** 5, size=m)],
                      sorted(rng.choice(256, size=m, replace=False).tolist()))
        lens = cb.package_merge_lengths(h, int(rng.integers(max(8, math.ceil(math.log2(m))), 25)))
        codes = cb.canonical_codes(lens)
        used = [s for s in range(256) if lens[s]]
        strs = {s: format(int(codes[s]), "0%db" % int(lens[s])) for s in used}
        # prefix-free
        vals = sorted(strs.values())
        for a, b in zip(vals, vals[1:]):
            assert not b.startswith(a)
        # left-justified order: sorted by (length, symbol) == sorted by code value
        lj = sorted(used, key=lambda s: int(codes[s]) << (24 - int(lens[s])))
        assert lj == sorted(used, key=lambda s: (int(lens[s]), s))
        # codes of equal length are consecutive integers
        for l in set(int(lens[s]) for s in used):
            cs = [int(codes[s]) for s in used if lens[s] == l]
            assert cs == list(range(cs[0], cs[0] + len(cs)))


def test_canonical_tables_decode_every_code():
    rng = np.random.default_rng(5)
    fib = [1, 1]
    while len(fib) < 30:
        fib.append(fib[-1] + fib[-2])
    for h in (hist_from(fib, list(range(60, 90))),
              hist_from([int(x) for x in rng.integers(1, 1000, size=200)], list(range(200)))):
        lens = cb.package_merge_lengths(h, 24)
        codes = cb.canonical_codes(lens)
        t = cb.canonical_tables(lens)
        for s in range(256):
            if lens[s]:
                l = int(lens[s])
                for tail in (0, (1 << (24 - l)) - 1):
                    w = (int(codes[s]) << (24 - l)) | tail
                    assert cb.decode_window(w, t) == (s, l)


def test_tie_rule_leaves_in_symbol_order():
    """Ties between optimal length assignments follow the stated reading
    (the pages are silent): leaves of equal count are ordered by symbol, so
    package-merge pairs the smaller symbols first and they end up deeper.
    Worked by hand for counts 1, 1, 1 on symbols 5, 9, 200: the kept items
    are the three leaves and the package (5, 9), giving 5 and 9 length 2 and
    200 length 1 (the mirror choice, 200 deeper, costs the same)."""
    hist = np.zeros(256, dtype=np.int64)
    hist[[5, 9, 200]] = 1
    lengths = cb.package_merge_lengths(hist, 24)
    assert {s: int(lengths[s]) for s in (5, 9, 200)} == {5: 2, 9: 2, 200: 1}
    assert int(np.count_nonzero(lengths)) == 3


def test_tie_rule_leaves_before_packages():
    """Same reading, second half: of items with equal weight, leaves come
    before packages.  Counts 1, 1, 2, 2 on symbols 1..4, worked by hand: the
    package (1, 2) of weight 2 ties the leaves 3 and 4; leaves first keeps
    1, 2, 3, 4, (1, 2) and (3, 4), so every symbol has length 2.  Packages
    first would keep (1, 2) ahead of 3 and give lengths 3, 3, 2, 1 at the
    same cost 12."""
    hist = np.zeros(256, dtype=np.int64)
    hist[[1, 2, 3, 4]] = [1, 1, 2, 2]
    lengths = cb.package_merge_lengths(hist, 24)
    assert [int(lengths[s]) for s in (1, 2, 3, 4)] == [2, 2, 2, 2]
    assert int((hist * lengths).sum()) == 12
