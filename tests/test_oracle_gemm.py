"""Pins for the float64 reference product used by the fused decode + GEMM path."""
import numpy as np

from oracle import gemm
from lossless_entropy_coded_dfc_amd import synth


def test_bf16_conversion_exact_values():
    bits = np.array([0x3F80, 0xC000, 0x3E00, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    v = gemm.bf16_bits_to_f64(bits)
    assert v[:5].tolist() == [1.0, -2.0, 0.125, 0.0, -0.0]
    assert v[5] == 3.140625  # 0x4049 = 1.5703125 * 2


def test_identity_and_integer_products():
    # W = I: Y equals X exactly
    eye = np.where(np.eye(32, dtype=bool), 0x3F80, 0).astype(np.uint16)
    x = synth.activations(32, 5, (1,))
    assert np.array_equal(gemm.gemm_reference(eye, x), gemm.bf16_bits_to_f64(x))
    # small integers are exact in bf16 and their products and sums are exact
    rng = np.random.default_rng(0)
    wi = rng.integers(-8, 9, size=(7, 64)).astype(np.float32)
    xi = rng.integers(-8, 9, size=(64, 3)).astype(np.float32)
    wb = (wi.view(np.uint32) >> 16).astype(np.uint16)
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    ref = (wi.astype(np.int64) @ xi.astype(np.int64)).astype(np.float64)
    assert np.array_equal(gemm.gemm_reference(wb, xb), ref)
    assert np.array_equal(gemm.abs_product_bound(wb, xb), np.abs(wi).astype(np.int64) @ np.abs(xi).astype(np.int64))
