"""Reference product for the fused decode + GEMM path (oracle).

Y = W X with W (M x K) the decoded bf16 weight matrix and X (K x B) bf16
activations.  bf16 -> float64 is exact, and so is every product of two bf16
values; the float64 sum over K = 8192 carries a relative error near 1e-16,
far inside the 1e-3 tolerance the fused path is held to.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def gemm_reference(w_bits: np.ndarray, x_bits: np.ndarray) -> np.ndarray:
    """float64 W @ X from bf16 bit patterns (W: M x K, X: K x B)."""
    w = bf16_bits_to_f64(w_bits)
    x = bf16_bits_to_f64(x_bits)
    return w @ x


def abs_product_bound(w_bits: np.ndarray, x_bits: np.ndarray) -> np.ndarray:
    """|W| @ |X| in float64: the scale of each output element's summands."""
    return np.abs(bf16_bits_to_f64(w_bits)) @ np.abs(bf16_bits_to_f64(x_bits))
