"""Seeded synthetic bf16 weight tensors.

This module only manufactures inputs: it draws random numbers and rounds them
to bf16 bit patterns.  It contains none of the codec's arithmetic (no field
split, no histogram, no code construction), so both the CPU oracle and the HIP
path may consume what it produces.

Every tensor is returned as a C-contiguous ``numpy.uint16`` array holding the
raw bf16 bit patterns in row-major order.  Random streams are numpy PCG64
generators seeded with a tuple, one tuple per tensor, so any tensor can be
regenerated on its own.

The workloads stand in for trained Llama-class bf16 weights, which the
DFloat11 blog post ("70% Size, 100% Accuracy ... (DFloat11)", section 02)
describes as a low-entropy bf16 distribution; no real checkpoint is used.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_to_bf16_bits",
    "gaussian",
    "gaussian_pieces",
    "gaussian_with_outliers",
    "student_t",
    "bimodal",
    "uniform_bits",
    "exponent_ladder",
    "activations",
    "llama3_8b_block_shapes",
    "llama3_8b_block",
    "llama3_8b_model_plan",
    "model_matrix",
    "single_matrix",
    "gemm_weight",
    "stress",
    "STRESS_KINDS",
]

# Outlier magnitude used by the transformer-block workload: 20 standard
# deviations of N(0, 0.02^2) is 0.4, which rounds to bf16 0x3ECD.
_OUTLIER_POS = np.uint16(0x3ECD)
_OUTLIER_NEG = np.uint16(0xBECD)


def _rng(seed) -> np.random.Generator:
    if isinstance(seed, int):
        seed = (seed,)
    return np.random.default_rng(tuple(int(s) for s in seed))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (round to nearest, ties to even).

    Works on the float32 bit pattern: add 0x7FFF plus the lowest kept bit,
    then keep the high 16 bits.  Inputs here are always finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal_bits(rng: np.random.Generator, n: int, std: float) -> np.ndarray:
    # Draw in float32 and scale in float32 so the stream is cheap at 10^8 scale.
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        z = rng.standard_normal(hi - lo, dtype=np.float32)
        z *= np.float32(std)
        out[lo:hi] = round_to_bf16_bits(z)
    return out


def gaussian(shape, std: float, seed) -> np.ndarray:
    """i.i.d. N(0, std^2) rounded to bf16."""
    n = int(np.prod(shape))
    return _normal_bits(_rng(seed), n, std).reshape(shape)


def gaussian_pieces(n: int, std: float, seed, piece: int = 1 << 26, threads: int = 16) -> np.ndarray:
    """n i.i.d. N(0, std^2) bf16 values drawn in independent pieces of `piece`
    values, piece j from the seed tuple (*seed, j), on up to `threads` host
    threads: for tensors of billions of values, where one generator would take
    minutes.  No two pieces repeat each other."""
    from concurrent.futures import ThreadPoolExecutor
    seed = (seed,) if isinstance(seed, int) else tuple(seed)
    out = np.empty(n, dtype=np.uint16)

    def fill(j):
        lo = j * piece
        out[lo: min(n, lo + piece)] = _normal_bits(_rng(seed + (j,)), min(n, lo + piece) - lo, std)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as pool:
        list(pool.map(fill, range((n + piece - 1) // piece)))
    return out


def gaussian_with_outliers(shape, std: float, seed, frac: float = 1e-3,
                           scale: float = 20.0) -> np.ndarray:
    """N(0, std^2) bf16 with floor(n*frac) distinct positions set to +-scale*std.

    Positions are drawn without replacement; each sign is a fair coin.  With
    std = 0.02 and scale = 20 the outlier is bf16 +-0.4 (0x3ECD / 0xBECD).
    """
    rng = _rng(seed)
    n = int(np.prod(shape))
    w = _normal_bits(rng, n, std)
    k = int(n * frac)
    if k:
        pos = rng.choice(n, size=k, replace=False)
        neg = rng.integers(0, 2, size=k).astype(bool)
        if std == 0.02 and scale == 20.0:
            vals = np.where(neg, _OUTLIER_NEG, _OUTLIER_POS)
        else:
            mag = round_to_bf16_bits(np.float32(scale * std).reshape(1))[0]
            vals = np.where(neg, mag | np.uint16(0x8000), mag)
        w[pos] = vals.astype(np.uint16)
    return w.reshape(shape)


def student_t(shape, df: float, std: float, seed) -> np.ndarray:
    """Student-t(df) scaled so the standard deviation is ``std`` (df > 2)."""
    rng = _rng(seed)
    n = int(np.prod(shape))
    scale = std / np.sqrt(df / (df - 2.0))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        z = (rng.standard_t(df, size=hi - lo) * scale).astype(np.float32)
        out[lo:hi] = round_to_bf16_bits(z)
    return out.reshape(shape)


def bimodal(shape, std: float, seed, ratio: float = 2.0 ** -10) -> np.ndarray:
    """Per element a fair coin picks N(0, std^2) or N(0, (std*ratio)^2).

    The two scales sit ten binades apart, so the exponent histogram has two
    separated bumps.
    """
    rng = _rng(seed)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        z = rng.standard_normal(hi - lo, dtype=np.float32)
        small = rng.integers(0, 2, size=hi - lo).astype(bool)
        z *= np.where(small, np.float32(std * ratio), np.float32(std))
        out[lo:hi] = round_to_bf16_bits(z)
    return out.reshape(shape)


def uniform_bits(shape, seed) -> np.ndarray:
    """Uniformly random 16-bit patterns: every exponent (0..255) equally likely,
    including the Inf/NaN exponent 255 and the zero/subnormal exponent 0."""
    rng = _rng(seed)
    n = int(np.prod(shape))
    return rng.integers(0, 1 << 16, size=n, dtype=np.uint16).reshape(shape)


def exponent_ladder(shape, seed, top: int = 126, steps: int = 40) -> np.ndarray:
    """Exponent top-k drawn with probability proportional to 2^-k (k < steps);
    sign and mantissa bits uniformly random.

    With 40 rungs the unconstrained optimal prefix code is far deeper than 24
    bits, so a 24-bit length limit must bind.
    """
    rng = _rng(seed)
    n = int(np.prod(shape))
    p = 0.5 ** np.arange(steps, dtype=np.float64)
    p /= p.sum()
    k = rng.choice(steps, size=n, p=p)
    e = (top - k).astype(np.uint16)
    low = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    bits = (low & np.uint16(0x807F)) | (e << np.uint16(7))
    return bits.astype(np.uint16).reshape(shape)


def activations(k: int, b: int, seed) -> np.ndarray:
    """GEMM right-hand side: K x B matrix of N(0, 1) values rounded to bf16."""
    return _normal_bits(_rng(seed), k * b, 1.0).reshape(k, b)


# --------------------------------------------------------------------------
# Named workloads (Llama-3-8B shapes; Gaussian stand-ins for trained weights)
# --------------------------------------------------------------------------

def llama3_8b_block_shapes():
    """(name, rows, cols) of one Llama-3-8B transformer block's weight matrices."""
    return [
        ("wq", 4096, 4096),
        ("wk", 1024, 4096),
        ("wv", 1024, 4096),
        ("wo", 4096, 4096),
        ("gate", 14336, 4096),
        ("up", 14336, 4096),
        ("down", 4096, 14336),
    ]


def single_matrix(rows: int = 4096, cols: int = 4096, seed=(0,), std: float = 0.02):
    """One i.i.d. N(0, 0.02^2) bf16 matrix (default 4096 x 4096, seed 0)."""
    return gaussian((rows, cols), std, seed)


def llama3_8b_block(block: int = 0, family: int = 2, scale: float = 1.0):
    """Yield (name, matrix) for one transformer block: N(0, 0.02^2) plus 0.1%
    outliers at 20 sigma, seeds (family, block, j).  ``scale`` < 1 shrinks the
    row count (for quick tests) while keeping the column count."""
    for j, (name, r, c) in enumerate(llama3_8b_block_shapes()):
        rr = max(1, int(r * scale))
        yield name, gaussian_with_outliers((rr, c), 0.02, (family, block, j))


def llama3_8b_model_plan(n_blocks: int = 32, vocab: int = 128256, hidden: int = 4096):
    """List of (name, rows, cols, seed) for a full 8B-shaped weight set:
    n_blocks transformer blocks then the embedding and LM head (untied)."""
    plan = []
    for b in range(n_blocks):
        for j, (name, r, c) in enumerate(llama3_8b_block_shapes()):
            plan.append((f"block{b}.{name}", r, c, (3, b, j)))
    plan.append(("embedding", vocab, hidden, (3, n_blocks, 0)))
    plan.append(("lm_head", vocab, hidden, (3, n_blocks, 1)))
    return plan


def model_matrix(rows: int, cols: int, seed) -> np.ndarray:
    """One matrix of the whole-model workload (same recipe as the block)."""
    return gaussian_with_outliers((rows, cols), 0.02, seed)


def gemm_weight(rows: int = 28672, cols: int = 8192, seed=(4, 0)):
    """Fused-GEMM weight: N(0, 0.015^2) bf16."""
    return gaussian((rows, cols), 0.015, seed)


STRESS_KINDS = ("student_t", "bimodal", "uniform", "ladder")


def stress(kind: str, rows: int = 8192, cols: int = 28672):
    """Stress tensors on the 8192 x 28672 shape (or a smaller one for tests)."""
    shape = (rows, cols)
    if kind == "student_t":
        return student_t(shape, 3.0, 0.02, (5, 0))
    if kind == "bimodal":
        return bimodal(shape, 0.02, (5, 1))
    if kind == "uniform":
        return uniform_bits(shape, (5, 2))
    if kind == "ladder":
        return exponent_ladder(shape, (5, 3))
    raise ValueError(f"unknown stress kind {kind!r}")
