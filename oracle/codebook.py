"""Exponent histogram, entropy, length-limited optimal code lengths and the
canonical code (oracle).

Method (DFloat11 blog, section 02): values that occur often receive short
codes and rare values long ones, approaching the information-optimal size
(the introduction calls the compression near information-optimal).  Readings:

* the code is an optimal prefix code under a maximum length of 24 bits,
  computed with the package-merge algorithm (Larmore and Hirschberg, "A fast
  algorithm for optimal length-limited Huffman codes", J. ACM 37(3), 1990);
* ties between equally good assignments are broken deterministically: items
  of equal weight are ordered leaves first (by symbol value), then packages
  (in the order they were formed);
* codes are assigned canonically as in RFC 1951 section 3.2.2: shorter codes
  take numerically smaller values, and codes of one length are consecutive in
  increasing symbol order;
* a histogram with a single used symbol gets that symbol length 1 plus a
  phantom symbol ((s + 1) mod 256, count 0) of length 1, so that the code is
  complete and every coded exponent consumes at least one bit.
"""
from __future__ import annotations

import heapq
import math

import numpy as np

MAX_LEN = 24


def histogram(exponent: np.ndarray) -> np.ndarray:
    """256-bin count of exponent bytes (uint64)."""
    e = np.asarray(exponent, dtype=np.uint8).ravel()
    return np.bincount(e, minlength=256).astype(np.uint64)


def entropy_bits(hist) -> float:
    """Plug-in Shannon entropy -sum p log2 p of a histogram, in bits/symbol."""
    h = np.asarray(hist, dtype=np.float64)
    n = h.sum()
    if n == 0:
        return 0.0
    p = h[h > 0] / n
    return float(-(p * np.log2(p)).sum())


def package_merge_lengths(hist, max_len: int = MAX_LEN) -> np.ndarray:
    """Optimal code lengths under ``max_len`` (uint8[256], 0 = unused).

    Package-merge in its coin-collector form: every used symbol is a coin of
    face value 2^-l for each l in 1..max_len and numismatic value equal to its
    count.  Starting from the list for the smallest denomination, ``max_len-1``
    rounds each pair up neighbouring items into packages and merge the packages
    with a fresh copy of the symbols.  The cheapest 2m-2 items of the final
    list are selected; the length of a symbol is the number of times it occurs
    inside them.
    """
    hist = np.asarray(hist, dtype=np.uint64)
    if hist.shape != (256,):
        raise ValueError("histogram must have 256 bins")
    if not 1 <= max_len <= MAX_LEN:
        raise ValueError("max_len out of range")
    used = [s for s in range(256) if hist[s] > 0]
    m = len(used)
    lengths = np.zeros(256, dtype=np.uint8)
    if m == 0:
        return lengths
    if m == 1:
        s = used[0]
        lengths[s] = 1
        lengths[(s + 1) % 256] = 1
        return lengths
    if m > (1 << max_len):
        raise ValueError("alphabet does not fit under the length limit")

    # An item is (weight, kind, order, multiplicity vector over the used
    # symbols); kind 0 = leaf, 1 = package.  Sorting by (weight, kind, order)
    # realises the tie-break rule stated in the module docstring.
    def leaves():
        order = sorted(range(m), key=lambda i: (int(hist[used[i]]), used[i]))
        items = []
        for rank, i in enumerate(order):
            v = np.zeros(m, dtype=np.int64)
            v[i] = 1
            items.append((int(hist[used[i]]), 0, rank, v))
        return items

    current = leaves()
    for _ in range(max_len - 1):
        packages = []
        for j in range(len(current) // 2):
            a, b = current[2 * j], current[2 * j + 1]
            packages.append((a[0] + b[0], 1, j, a[3] + b[3]))
        current = sorted(leaves() + packages, key=lambda it: (it[0], it[1], it[2]))
    chosen = current[: 2 * m - 2]
    total = np.zeros(m, dtype=np.int64)
    for it in chosen:
        total += it[3]
    for i, s in enumerate(used):
        lengths[s] = int(total[i])
    return lengths


def huffman_cost(hist) -> int:
    """Cost sum(f * l) of an unconstrained Huffman code, computed the textbook
    way (repeatedly merge the two lightest subtrees; the cost is the sum of all
    merged weights)."""
    w = [int(x) for x in np.asarray(hist).ravel() if x > 0]
    if len(w) <= 1:
        return sum(w)  # one symbol of length 1 under the single-symbol reading
    heapq.heapify(w)
    cost = 0
    while len(w) > 1:
        a = heapq.heappop(w)
        b = heapq.heappop(w)
        cost += a + b
        heapq.heappush(w, a + b)
    return cost


def huffman_depth(hist) -> int:
    """Depth of the textbook Huffman tree (lightest-first merging, leaves on
    ties); used to tell whether a length limit binds."""
    items = [(int(x), 0, i, 0) for i, x in enumerate(np.asarray(hist).ravel()) if x > 0]
    if len(items) <= 1:
        return 1 if items else 0
    heapq.heapify(items)
    serial = 1 << 20
    while len(items) > 1:
        a = heapq.heappop(items)
        b = heapq.heappop(items)
        heapq.heappush(items, (a[0] + b[0], 1, serial, max(a[3], b[3]) + 1))
        serial += 1
    return items[0][3]


def code_cost(hist, lengths) -> int:
    """sum over symbols of count * length."""
    return int(sum(int(h) * int(l) for h, l in zip(np.asarray(hist), np.asarray(lengths))))


def kraft_numerator(lengths, max_len: int = MAX_LEN) -> int:
    """sum 2^(max_len - l) over used symbols; equals 2^max_len for a complete code."""
    return sum(1 << (max_len - int(l)) for l in np.asarray(lengths) if l > 0)


def canonical_codes(lengths) -> np.ndarray:
    """Canonical code values (uint32[256]) for the given lengths.

    RFC 1951 section 3.2.2: count the codes of each length; the first code of
    length l is (first code of length l-1 + number of codes of length l-1)
    shifted left by one; codes of one length are handed out in increasing
    symbol order.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    max_len = int(lengths.max()) if lengths.size else 0
    count = [0] * (max_len + 2)
    for l in lengths:
        if l > 0:
            count[int(l)] += 1
    next_code = [0] * (max_len + 2)
    code = 0
    for l in range(1, max_len + 1):
        code = (code + count[l - 1]) << 1 if l > 1 else 0
        next_code[l] = code
    codes = np.zeros(256, dtype=np.uint32)
    for s in range(256):
        l = int(lengths[s])
        if l > 0:
            codes[s] = next_code[l]
            next_code[l] += 1
    return codes


def canonical_tables(lengths):
    """Per-length canonical decoding tables, indexed by length 1..24.

    Returns a dict with
      count[l]  number of codes of length l,
      first[l]  first (smallest) code value of length l,
      limit[l]  (first[l] + count[l]) << (24 - l): a left-justified 24-bit
                window w holds a code of length <= l exactly when w < limit[l],
      base[l]   number of used symbols whose length is < l,
      order     used symbols sorted by (length, symbol).
    A window decodes to the smallest l with w < limit[l]; its symbol is
    order[base[l] + (w >> (24 - l)) - first[l]].
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    count = [0] * (MAX_LEN + 1)
    for l in lengths:
        if l > 0:
            count[int(l)] += 1
    first = [0] * (MAX_LEN + 1)
    limit = [0] * (MAX_LEN + 1)
    base = [0] * (MAX_LEN + 1)
    code = 0
    seen = 0
    for l in range(1, MAX_LEN + 1):
        if l > 1:
            code = (first[l - 1] + count[l - 1]) << 1
        first[l] = code
        limit[l] = (first[l] + count[l]) << (MAX_LEN - l)
        base[l] = seen
        seen += count[l]
    order = sorted((int(lengths[s]), s) for s in range(256) if lengths[s] > 0)
    return {
        "count": count,
        "first": first,
        "limit": limit,
        "base": base,
        "order": [s for _, s in order],
    }


def decode_window(window24: int, tables) -> tuple[int, int]:
    """(symbol, length) of the code at the start of a 24-bit window."""
    for l in range(1, MAX_LEN + 1):
        if window24 < tables["limit"][l]:
            idx = tables["base"][l] + (window24 >> (MAX_LEN - l)) - tables["first"][l]
            return tables["order"][idx], l
    raise ValueError("window matches no code (incomplete code table)")


def build_codebook(hist, max_len: int = MAX_LEN):
    """lengths, codes and summary numbers for a histogram."""
    lengths = package_merge_lengths(hist, max_len)
    codes = canonical_codes(lengths)
    used = lengths > 0
    return {
        "lengths": lengths,
        "codes": codes,
        "n_used": int(used.sum()),
        "max_len": int(lengths.max()) if used.any() else 0,
        "min_len": int(lengths[used].min()) if used.any() else 0,
    }


def mean_code_length(hist, lengths) -> float:
    n = float(np.asarray(hist, dtype=np.float64).sum())
    return code_cost(hist, lengths) / n if n else 0.0


def log2_int(x: int) -> int:
    return int(math.log2(x))
