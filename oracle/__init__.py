"""CPU oracle for exponent-Huffman compression of bf16 weights (DFloat11 style).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the HIP decoder is checked against.  Only the test suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product library never imports, links or calls
anything here, and nothing here imports the product library: the two share no
code.  The only module both sides consume is the seeded input generator
``lossless_entropy_coded_dfc_amd.synth``, which holds no codec arithmetic.

What the method computes (DFloat11 blog post, "70% Size, 100% Accuracy:
Lossless LLM Compression for Efficient GPU Inference via Dynamic-Length Float
(DFloat11)"):

* section 02: bf16 weights have a low-entropy distribution; frequent values
  get short codes and rare values long ones (a Huffman-like entropy code), and
  decompression returns the original bits exactly;
* section 03 item 1: decoding uses compact hierarchical lookup tables held in
  on-chip memory;
* section 03 item 2: a two-phase kernel in which threads first agree on read
  and write positions through small auxiliary variables, then rebuild the
  weights.

The oracle fixes what is coded and how the container lays it out.  The
lookup tables of section 03 item 1 are a decoder's own means of finding code
boundaries fast; they are a function of the code lengths, no container
carries them, and nothing here builds them.

Readings taken where the pages leave a step open (each is listed, with its
reason, in the design notes of the repository):

* only the 8 exponent bits are entropy-coded; sign and mantissa stay one raw
  byte ``sign << 7 | mantissa``;
* the code is a length-limited (24 bits) optimal prefix code built by
  package-merge, assigned canonically (RFC 1951, section 3.2.2);
* the bitstream is MSB-first inside little-endian 32-bit words, cut into
  fixed-size chunks with a 5-bit start offset per chunk and a 32-bit output
  offset per block of chunks.

Modules:

* ``fields``   - bf16 <-> (exponent byte, raw byte)
* ``codebook`` - histogram, entropy, package-merge lengths, canonical codes
* ``stream``   - bit packing, chunk/block metadata, sequential and
                 chunk-parallel decoders
* ``blob``     - the serialized container (code lengths and coded data)
* ``gemm``     - float64 reference product and the panel element order
* ``panel``    - the panel layout consumed by the fused decode + product
* ``padded``   - the offset-free padded-chunk layout and its decoders
* ``ans``      - interleaved rANS coding of the exponents (layout 3)

Parity status: every function is pinned by a test in ``tests/`` against
something other than itself (closed forms, brute force, RFC 1951's worked
example, hand-worked fixtures in ``tests/golden/``, or exact round trips).
"""

from . import fields, codebook, stream, blob, gemm, panel, padded, ans  # noqa: F401

__all__ = ["fields", "codebook", "stream", "blob", "gemm", "panel", "padded", "ans"]
