"""bf16 field split (oracle).

A bf16 value is 16 bits: sign (bit 15), exponent (bits 14..7), mantissa
(bits 6..0) (DFloat11 blog, section 01: BFloat16 stores 16 bits per
parameter).  The entropy code is applied to the exponent only; sign and
mantissa travel as one raw byte ``sign << 7 | mantissa`` (reading: the blog's
section 02 does not say which bits are coded; the exponent carries nearly all
of the redundancy of Gaussian-like weights).

All work is on bit patterns; no value is ever converted to a float, so NaN
payloads, infinities, -0 and subnormals pass through unchanged.
"""
from __future__ import annotations

import numpy as np


def split(bits: np.ndarray):
    """Return (exponent bytes, raw bytes) of an array of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).ravel()
    exponent = ((b >> 7) & 0xFF).astype(np.uint8)
    sign = (b >> 15).astype(np.uint8)
    mantissa = (b & 0x7F).astype(np.uint8)
    raw = ((sign << 7) | mantissa).astype(np.uint8)
    return exponent, raw


def merge(exponent: np.ndarray, raw: np.ndarray) -> np.ndarray:
    """Inverse of :func:`split`."""
    e = np.asarray(exponent, dtype=np.uint16)
    r = np.asarray(raw, dtype=np.uint16)
    sign = (r >> 7) & 1
    mantissa = r & 0x7F
    return ((sign << 15) | (e << 7) | mantissa).astype(np.uint16)
