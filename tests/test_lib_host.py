"""Host half of libdfc on the CPU: the library loads and exports every symbol
the header declares, its encoder writes containers byte-identical to the
oracle's, its codebooks are optimal, and validation rejects corrupt
containers with the documented status codes."""
import os
import re
import struct

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import blob as bl
from oracle import codebook as cb
from oracle import fields
from oracle import stream as st

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dfc.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:dfc_status|void|const char \*)\s*\*?\s*(dfc_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = dfc.library()
    names = declared_functions()
    assert {"dfc_build_codebook", "dfc_encode", "dfc_decode", "dfc_decode_batch", "dfc_blob_info"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert dfc.status_str(-3) == "corrupt container"


def oracle_blob(x, C, T=64, k=11):
    shape = x.shape if x.ndim == 2 else (1, x.size)
    if x.size == 0:
        shape = (1, 0)
    return bl.write_blob(st.encode(x, C, T), k, *shape)


@pytest.mark.parametrize("C", [4, 8, 16, 32])
@pytest.mark.parametrize("kind", ["gauss", "outliers", "uniform", "ladder", "bimodal", "t", "const"])
def test_encoder_matches_oracle_bytes(C, kind):
    shape = (37, 1001)
    x = {"gauss": lambda: synth.gaussian(shape, 0.02, (20, C)),
         "outliers": lambda: synth.gaussian_with_outliers(shape, 0.02, (21, C)),
         "uniform": lambda: synth.uniform_bits(shape, (22, C)),
         "ladder": lambda: synth.exponent_ladder(shape, (23, C)),
         "bimodal": lambda: synth.bimodal(shape, 0.02, (24, C)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (25, C)),
         "const": lambda: np.full(shape, 0x3C00, dtype=np.uint16)}[kind]()
    for k in (8, 12):
        lib_blob = dfc.encode(x, chunk_bytes=C, lut_bits=k)
        assert bytes(lib_blob) == oracle_blob(x, C, 64, k)


def test_encoder_threads():
    x = synth.gaussian((3000, 1000), 0.02, (26,))  # 3M elements -> several encoder threads
    for threads in (1, 3, 8):
        b = dfc.encode(x, chunk_bytes=8, threads=threads)
        assert bytes(b) == oracle_blob(x, 8, 64), threads


@pytest.mark.parametrize("layout", [0, 1, 2, 3])
@pytest.mark.parametrize("T", [32, 128, 256])
def test_encoder_refuses_blocks_wider_than_a_wavefront(T, layout):
    """One wavefront (64 lanes) decodes one block, so 64 chunks per block is
    the only width the encoder writes: a container no decoder could take is
    refused before anything is written."""
    x = synth.gaussian((64, 256), 0.02, (27,))
    with pytest.raises(dfc.DfcError) as e:
        dfc.encode(x, lanes=T, layout=layout)
    assert e.value.status == dfc.EINVAL
    with pytest.raises(dfc.DfcError):
        dfc.encode_bound(x.size, dfc.default_params(lanes_per_block=T, layout=layout))


def test_launch_knob_rejects_out_of_range_values():
    """dfc_set_launch validates every field before it changes anything; no
    GPU call is made."""
    for bad in ((17, 0, 0, 0), (0, 65, 0, 0), (0, 0, 3, 0), (0, 0, 0, 65)):
        with pytest.raises(dfc.DfcError) as e:
            dfc.set_launch(*bad)
        assert e.value.status == dfc.EINVAL, bad
    for mode in (dfc.STORES_DEFERRED, dfc.STORES_IMMEDIATE, dfc.STORES_AUTO):
        dfc.set_launch(0, 0, mode)


def test_edge_sizes_match_oracle():
    for n in (0, 1, 2, 15, 16, 17, 63, 64, 65, 1000):
        x = synth.uniform_bits((n,), (27, n))
        b = dfc.encode(x, chunk_bytes=4)
        assert bytes(b) == oracle_blob(x, 4), n
        info = dfc.blob_info(b)
        assert info.n == n


def test_codebook_optimal_and_canonical():
    rng = np.random.default_rng(9)
    for trial in range(30):
        m = int(rng.integers(1, 257))
        h = np.zeros(256, dtype=np.uint64)
        h[rng.choice(256, size=m, replace=False)] = rng.integers(1, 1 << int(rng.integers(1, 34)), size=m)
        L = int(rng.integers(max(1, int(np.ceil(np.log2(max(m, 2))))), 25))
        book = dfc.build_codebook(h, L)
        lens = book.lengths
        assert np.array_equal(lens, cb.package_merge_lengths(h, L))
        assert np.array_equal(book.codes, cb.canonical_codes(lens))
        assert book.n_used == int((lens > 0).sum())
        assert cb.kraft_numerator(lens) == 1 << 24
        if m > 1:
            assert cb.code_cost(h, lens) <= cb.code_cost(h, cb.package_merge_lengths(h, L))


def test_histogram_matches_oracle():
    x = synth.uniform_bits((5_000_000,), (28,))
    assert np.array_equal(dfc.histogram(x), cb.histogram(fields.split(x)[0]))


def test_external_codebook_and_missing_symbol():
    x = synth.gaussian((64, 512), 0.02, (29,))
    h = cb.histogram(fields.split(x)[0]) + 1  # smoothed: every exponent has a code
    book = dfc.build_codebook(h, 24)
    b = dfc.encode(x, codebook=book)
    C = bl.choose_chunk_bytes(cb.histogram(fields.split(x)[0]), book.lengths)
    assert bytes(b) == bl.write_blob(st.encode(x, C, 64, lengths=book.lengths), 11, 64, 512)
    e = fields.split(x)[0]
    h2 = cb.histogram(e)
    h2[int(e[0])] = 0  # a present exponent without a code
    with pytest.raises(dfc.DfcError) as ei:
        dfc.encode(x, codebook=dfc.build_codebook(h2, 24))
    assert ei.value.status == dfc.EINVAL


def test_bad_params_rejected():
    x = synth.gaussian((4, 64), 0.02, (30,))
    for kw in ({"chunk_bytes": 12}, {"lanes": 32}, {"max_code_len": 25}, {"lut_bits": 13}, {"lut_bits": 7}):
        with pytest.raises(dfc.DfcError) as ei:
            dfc.encode(x, **kw)
        assert ei.value.status == dfc.EINVAL


def corrupt(blob: np.ndarray, offset: int, value: bytes) -> np.ndarray:
    b = blob.copy()
    b[offset: offset + len(value)] = np.frombuffer(value, dtype=np.uint8)
    return b


def test_validation_rejects_corruption():
    x = synth.gaussian((128, 1024), 0.02, (31,))
    b = dfc.encode(x)
    info = dfc.blob_info(b)
    cases = {
        "magic": (corrupt(b, 0, b"XXXX"), dfc.ECORRUPT),
        "version": (corrupt(b, 4, struct.pack("<I", 2)), dfc.EUNSUPPORTED),
        "n": (corrupt(b, 8, struct.pack("<Q", info.n + 1)), dfc.ECORRUPT),
        "chunk": (corrupt(b, 40, struct.pack("<I", 12)), dfc.ECORRUPT),
        # (a change that keeps the block count is caught on the GPU by the block count check)
        "total_bits": (corrupt(b, 16, struct.pack("<Q", info.total_bits + 8 * 16 * 64)), dfc.ECORRUPT),
        "length>24": (corrupt(b, 256 + 120, bytes([25])), dfc.ECORRUPT),
        "kraft": (corrupt(b, 256 + int(np.argmax(b[256:512])), bytes([int(b[256:512].max()) + 1])), dfc.ECORRUPT),
        # a tables section where the Huffman layouts have none
        "tables section": (corrupt(b, 88, struct.pack("<QQ", 512, 256)), dfc.ECORRUPT),
        "section": (corrupt(b, 88 + 16, struct.pack("<Q", info.off_words + 256)), dfc.ECORRUPT),
        "blockout_end": (corrupt(b, info.off_blockout + 4 * info.n_blocks, struct.pack("<I", info.n - 1)), dfc.ECORRUPT),
        "blockout_order": (corrupt(b, info.off_blockout + 4, struct.pack("<I", 0xFFFFFF)), dfc.ECORRUPT),
        "offset>max": (corrupt(b, info.off_offsets, bytes([0x1F])), dfc.ECORRUPT),
    }
    for name, (blob, want) in cases.items():
        with pytest.raises(dfc.DfcError) as ei:
            dfc.blob_info(blob)
        assert ei.value.status == want, name
    with pytest.raises(dfc.DfcError) as ei:
        dfc.blob_info(b[: len(b) - 256])
    assert ei.value.status == dfc.ESIZE


def test_encode_bound_and_small_capacity():
    x = synth.uniform_bits((10_000,), (32,))
    p = dfc.default_params()
    bound = dfc.encode_bound(x.size, p)
    b = dfc.encode(x)
    assert len(b) <= bound
    lib = dfc.library()
    import ctypes
    dst = np.empty(len(b) - 1, dtype=np.uint8)
    w = ctypes.c_uint64()
    s = lib.dfc_encode(x.ctypes.data_as(ctypes.c_void_p), x.size, ctypes.byref(p), None,
                       dst.ctypes.data_as(ctypes.c_void_p), dst.size, ctypes.byref(w))
    assert s == dfc.ESIZE


def test_size_accounting_gaussian():
    x = synth.gaussian((1024, 4096), 0.02, (0,))
    e = fields.split(x)[0]
    bound = bl.entropy_bound_bytes(cb.histogram(e))
    for C, lim in ((16, 1.02), (32, 1.02), (8, 1.03)):
        info = dfc.blob_info(dfc.encode(x, chunk_bytes=C))
        assert 1.0 < info.coded_bytes / bound < lim, C
        assert 1.45 < 2 * x.size / info.coded_bytes < 1.55  # ~1.5:1


# ------------------------------------------------------------- panel layout

from oracle import panel as pn  # noqa: E402


@pytest.mark.parametrize("C", [4, 8, 16, 32])
@pytest.mark.parametrize("shape,panel_k", [((64, 96), 32), ((96, 1040), 1024), ((128, 512), 128)])
def test_panel_encoder_matches_oracle_bytes(C, shape, panel_k):
    x = synth.gaussian_with_outliers(shape, 0.02, (64, C, shape[1]))
    got = dfc.encode(x, chunk_bytes=C, layout=dfc.LAYOUT_PANEL, panel_k=panel_k)
    want = pn.write_panel_blob(pn.encode_panel(x, panel_k=panel_k, chunk_bytes=C), 11)
    assert bytes(got) == want
    info = dfc.blob_info(got)
    assert info.layout == dfc.LAYOUT_PANEL and info.panel_rows == 32 and info.panel_k == panel_k
    assert info.n_items == len(pn.panel_items(*shape, panel_k))
    assert info.panels_bytes == 16 * (info.n_items + 1)
    width = 1 if C <= 16 else 2
    assert info.counts_bytes == 16 * -(-width * info.n_chunks // 16) and info.off_counts % 256 == 0
    assert info.coded_bytes == 512 + (info.words_bytes + info.offsets_bytes + info.blockout_bytes + info.raw_bytes
                                      + info.panels_bytes + info.counts_bytes)


def test_panel_stress_kinds_and_threads():
    for kind in synth.STRESS_KINDS:
        x = {"student_t": lambda: synth.student_t((96, 272), 3.0, 0.02, (65,)),
             "bimodal": lambda: synth.bimodal((96, 272), 0.02, (66,)),
             "uniform": lambda: synth.uniform_bits((96, 272), (67,)),
             "ladder": lambda: synth.exponent_ladder((96, 272), (68,))}[kind]()
        want = pn.write_panel_blob(pn.encode_panel(x, panel_k=64, chunk_bytes=8), 10)
        for threads in (1, 3, 16):
            got = dfc.encode(x, chunk_bytes=8, lut_bits=10, layout=dfc.LAYOUT_PANEL, panel_k=64, threads=threads)
            assert bytes(got) == want, (kind, threads)


def test_panel_bad_shapes_rejected():
    for shape, panel_k in (((48, 64), 16), ((64, 72), 16), ((64, 64), 24)):
        x = synth.gaussian(shape, 0.02, (69,))
        with pytest.raises(dfc.DfcError) as ei:
            dfc.encode(x, layout=dfc.LAYOUT_PANEL, panel_k=panel_k)
        assert ei.value.status == dfc.EINVAL


def test_panel_validation_rejects_corruption():
    x = synth.gaussian((96, 2048), 0.02, (70,))
    b = dfc.encode(x, chunk_bytes=16, layout=dfc.LAYOUT_PANEL, panel_k=512)
    info = dfc.blob_info(b)
    pt = info.off_panels
    first_block1 = struct.unpack_from("<I", bytes(b), pt + 16 + 4)[0]
    cases = {
        "panel_rows": corrupt(b, 60, struct.pack("<I", 16)),
        "panel_k": corrupt(b, 80, struct.pack("<I", 24)),
        "bits": corrupt(b, pt + 8, struct.pack("<I", 7)),
        "first_chunk": corrupt(b, pt + 16, struct.pack("<I", 1)),
        "first_block": corrupt(b, pt + 16 + 4, struct.pack("<I", first_block1 + 1)),
        "reserved": corrupt(b, pt + 12, struct.pack("<I", 1)),
        "sentinel": corrupt(b, pt + 16 * info.n_items + 8, struct.pack("<I", 1)),
        "item_start": corrupt(b, info.off_blockout + 4 * first_block1, struct.pack("<I", 32 * 512 + 1)),
        # a chunk count one higher: its block's counts no longer add up to
        # the block's offsets
        "count_sum": corrupt(b, info.off_counts + 3, struct.pack("<B", struct.unpack_from(
            "<B", bytes(b), info.off_counts + 3)[0] + 1)),
        # more codes than a chunk can start (8C codes of at least min_len bits)
        "count_max": corrupt(b, info.off_counts, struct.pack("<BB", 8 * 16 + 1, 0)),
        "count_padding": corrupt(b, info.off_counts + info.counts_bytes - 1, b"\x01")
        if info.counts_bytes > info.n_chunks else corrupt(b, 208, b"\x01"),
        "counts_slot": corrupt(b, 200, struct.pack("<Q", info.counts_bytes + 16)),
    }
    for name, bad in cases.items():
        with pytest.raises(dfc.DfcError) as ei:
            dfc.blob_info(bad)
        assert ei.value.status == dfc.ECORRUPT, name
    # moving one count to the next chunk of the same block keeps every sum:
    # the container still validates (only the decoder, which checks every
    # chunk's codes, can tell)
    c = bytearray(b)
    v0, v1 = struct.unpack_from("<BB", c, info.off_counts + 2)
    struct.pack_into("<BB", c, info.off_counts + 2, v0 - 1, v1 + 1)
    assert dfc.blob_info(np.frombuffer(bytes(c), dtype=np.uint8)).n == info.n


def test_flat_layouts_have_no_counts_section():
    x = synth.gaussian((64, 96), 0.02, (71,))
    for layout in (dfc.LAYOUT_FLAT, dfc.LAYOUT_PADDED, dfc.LAYOUT_ANS):
        info = dfc.blob_info(dfc.encode(x, chunk_bytes=8, layout=layout))
        assert (info.off_counts, info.counts_bytes) == (0, 0), layout


# ------------------------------------------------------------ padded layout

from oracle import padded as pdl  # noqa: E402


def oracle_padded_blob(x, C, T=64, k=11, lengths=None):
    shape = x.shape if x.ndim == 2 else (1, x.size)
    if x.size == 0:
        shape = (1, 0)
    return pdl.write_padded_blob(pdl.encode_padded(x, C, T, lengths=lengths), k, *shape)


@pytest.mark.parametrize("C", [4, 8, 16, 32])
@pytest.mark.parametrize("kind", ["outliers", "uniform", "ladder", "t", "const"])
def test_padded_encoder_matches_oracle_bytes(C, kind):
    shape = (41, 997)
    x = {"outliers": lambda: synth.gaussian_with_outliers(shape, 0.02, (60, C)),
         "uniform": lambda: synth.uniform_bits(shape, (61, C)),
         "ladder": lambda: synth.exponent_ladder(shape, (62, C)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (63, C)),
         "const": lambda: np.full(shape, 0x3C00, dtype=np.uint16)}[kind]()
    for k in (8, 12):
        lib_blob = dfc.encode(x, chunk_bytes=C, lut_bits=k, layout=dfc.LAYOUT_PADDED)
        assert bytes(lib_blob) == oracle_padded_blob(x, C, 64, k)
        info = dfc.blob_info(lib_blob)
        assert info.layout == dfc.LAYOUT_PADDED and info.offsets_bytes == 0 and info.off_offsets == 0


def test_padded_lanes_threads_and_edge_sizes():
    x = synth.gaussian_with_outliers((2500, 1000), 0.02, (64,))
    for threads in (1, 5, 16):
        b = dfc.encode(x, chunk_bytes=8, threads=threads, layout=dfc.LAYOUT_PADDED)
        assert bytes(b) == oracle_padded_blob(x, 8, 64), threads
    for n in (0, 1, 2, 15, 16, 17, 63, 64, 65, 1000):
        y = synth.uniform_bits((n,), (65, n))
        for C in (4, 32):
            b = dfc.encode(y, chunk_bytes=C, layout=dfc.LAYOUT_PADDED)
            assert bytes(b) == oracle_padded_blob(y, C), (n, C)
            dfc.blob_info(b)


def test_padded_external_codebook_bound_and_size():
    g = synth.gaussian((256, 256), 0.02, (66,))
    book = dfc.build_codebook(cb.histogram(fields.split(g)[0]) + 1, 24)
    x = synth.uniform_bits((100, 999), (67,))
    b = dfc.encode(x, chunk_bytes=4, codebook=book, layout=dfc.LAYOUT_PADDED)
    assert bytes(b) == oracle_padded_blob(x, 4, lengths=np.frombuffer(bytes(book.len), dtype=np.uint8))
    # the bound holds for the worst case: every code 24 bits long
    for C in (4, 8, 16, 32):
        p = dfc.default_params(chunk_bytes=C, layout=dfc.LAYOUT_PADDED)
        assert len(dfc.encode(x, chunk_bytes=C, codebook=book, layout=dfc.LAYOUT_PADDED)) <= dfc.encode_bound(x.size, p)
    # offsets gone: smaller than the flat container, within 2% of the
    # entropy bound at every chunk size and within 1% from C = 16 on
    y = synth.gaussian((1024, 4096), 0.02, (0,))
    bound = bl.entropy_bound_bytes(cb.histogram(fields.split(y)[0]))
    for C in (4, 8, 16, 32):
        flat = dfc.blob_info(dfc.encode(y, chunk_bytes=C)).coded_bytes
        pad = dfc.blob_info(dfc.encode(y, chunk_bytes=C, layout=dfc.LAYOUT_PADDED)).coded_bytes
        assert pad < flat, C
        assert pad / bound < (1.01 if C >= 16 else 1.02), C


def test_padded_validation_rejects_corruption():
    x = synth.gaussian((128, 1024), 0.02, (68,))
    b = dfc.encode(x, layout=dfc.LAYOUT_PADDED)
    info = dfc.blob_info(b)
    flat = dfc.encode(x)
    cases = {
        "layout=4": (corrupt(b, 56, struct.pack("<I", 4)), dfc.EUNSUPPORTED),
        "layout=ans": (corrupt(b, 56, struct.pack("<I", 3)), dfc.ECORRUPT),
        # a flat header on a padded body: the section table no longer fits
        "layout=flat": (corrupt(b, 56, struct.pack("<I", 0)), dfc.ECORRUPT),
        "padded header on flat body": (corrupt(flat, 56, struct.pack("<I", 2)), dfc.ECORRUPT),
        "total_bits": (corrupt(b, 16, struct.pack("<Q", info.total_bits + 8 * 16 * 64)), dfc.ECORRUPT),
        "blockout_end": (corrupt(b, info.off_blockout + 4 * info.n_blocks, struct.pack("<I", info.n - 1)),
                         dfc.ECORRUPT),
    }
    for name, (blob, want) in cases.items():
        with pytest.raises(dfc.DfcError) as ei:
            dfc.blob_info(blob)
        assert ei.value.status == want, name


# --------------------------------------------------------------- ANS layout

from oracle import ans as oans  # noqa: E402


def oracle_ans_blob(x, steps):
    shape = x.shape if x.ndim == 2 else (1, x.size)
    if x.size == 0:
        shape = (1, 0)
    return oans.write_ans_blob(oans.encode_ans(x, steps), *shape)


@pytest.mark.parametrize("steps", [8, 64, 512])
@pytest.mark.parametrize("kind", ["outliers", "uniform", "ladder", "t", "const"])
def test_ans_encoder_matches_oracle_bytes(steps, kind):
    shape = (41, 997)
    x = {"outliers": lambda: synth.gaussian_with_outliers(shape, 0.02, (120, steps)),
         "uniform": lambda: synth.uniform_bits(shape, (121, steps)),
         "ladder": lambda: synth.exponent_ladder(shape, (122, steps)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (123, steps)),
         "const": lambda: np.full(shape, 0x3C00, dtype=np.uint16)}[kind]()
    b = dfc.encode(x, layout=dfc.LAYOUT_ANS, ans_steps=steps)
    assert bytes(b) == oracle_ans_blob(x, steps)
    info = dfc.blob_info(b)
    assert info.layout == dfc.LAYOUT_ANS and info.ans_steps == steps and info.ans_prob_bits == 12
    assert info.coded_bytes == oans.coded_bytes(oans.encode_ans(x, steps))


def test_ans_threads_edge_sizes_and_bound():
    x = synth.gaussian_with_outliers((1500, 1000), 0.02, (124,))
    for threads in (1, 3, 16):
        b = dfc.encode(x, layout=dfc.LAYOUT_ANS, ans_steps=64, threads=threads)
        assert bytes(b) == oracle_ans_blob(x, 64), threads
    for n in (0, 1, 2, 63, 64, 65, 511, 512, 513, 5000):
        y = synth.uniform_bits((n,), (125, n))
        b = dfc.encode(y, layout=dfc.LAYOUT_ANS, ans_steps=8)
        assert bytes(b) == oracle_ans_blob(y, 8), n
        dfc.blob_info(b)
        assert len(b) <= dfc.encode_bound(n, dfc.default_params(layout=dfc.LAYOUT_ANS, ans_steps=8))
    assert dfc.blob_info(dfc.encode(x, layout=dfc.LAYOUT_ANS)).ans_steps == 512   # default


def test_ans_bad_params_rejected():
    x = synth.gaussian((4, 64), 0.02, (126,))
    for kw in ({"ans_steps": 12}, {"ans_steps": 4}, {"ans_steps": 65544}, {"lanes": 128}):
        with pytest.raises(dfc.DfcError) as ei:
            dfc.encode(x, layout=dfc.LAYOUT_ANS, **kw)
        assert ei.value.status == dfc.EINVAL, kw
    with pytest.raises(dfc.DfcError):
        dfc.encode(x, ans_steps=64)   # only the ANS layout takes steps
    book = dfc.build_codebook(cb.histogram(fields.split(x)[0]), 24)
    with pytest.raises(dfc.DfcError):
        dfc.encode(x, layout=dfc.LAYOUT_ANS, codebook=book)


def test_ans_size_near_entropy_bound():
    y = synth.gaussian((1024, 4096), 0.02, (0,))
    bound = bl.entropy_bound_bytes(cb.histogram(fields.split(y)[0]))
    pad = dfc.blob_info(dfc.encode(y, layout=dfc.LAYOUT_PADDED)).coded_bytes
    for steps, lim in ((256, 1.012), (512, 1.006), (1024, 1.004)):
        c = dfc.blob_info(dfc.encode(y, layout=dfc.LAYOUT_ANS, ans_steps=steps)).coded_bytes
        assert c / bound < lim, steps
        if steps >= 512:
            assert c < pad, steps


def test_ans_validation_rejects_corruption():
    x = synth.gaussian((128, 1024), 0.02, (127,))
    b = dfc.encode(x, layout=dfc.LAYOUT_ANS, ans_steps=64)
    info = dfc.blob_info(b)
    t = info.off_tables
    cases = {
        "steps": corrupt(b, 80, struct.pack("<I", 60)),
        "chunk_bytes": corrupt(b, 40, struct.pack("<I", 16)),
        "prob_bits": corrupt(b, 52, struct.pack("<I", 11)),
        "lengths area": corrupt(b, 300, b"\x01"),
        "freq sum": corrupt(b, t + 2 * int(np.argmax(np.frombuffer(bytes(b[t: t + 512]), dtype="<u2"))),
                            struct.pack("<H", 1)),
        "frequency table size": corrupt(b, 96, struct.pack("<Q", 512 + 4 * 4096)),
        "offsets end": corrupt(b, info.off_offsets + 4 * info.n_blocks, struct.pack("<I", 1)),
        "offsets order": corrupt(b, info.off_offsets + 4, struct.pack("<I", 0xFFFFFF)),
        "state below 2^16": corrupt(b, info.off_blockout + 8, struct.pack("<I", 5)),
        "total_bits": corrupt(b, 16, struct.pack("<Q", info.total_bits + 8)),
    }
    for name, blob in cases.items():
        with pytest.raises(dfc.DfcError) as ei:
            dfc.blob_info(blob)
        assert ei.value.status == dfc.ECORRUPT, name


def test_header_is_c99_and_host_abi_links_from_c(tmp_path):
    """include/dfc.h compiles as strict C99 and a C program linked to
    libdfc.so encodes and inspects a container through the host entry
    points (tests/c_abi_host.c)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    libdir = os.path.dirname(dfc.library_path())
    dfc.library()
    exe = str(tmp_path / "c_abi_host")
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                        "-I", os.path.join(root, "include"), os.path.join(here, "c_abi_host.c"),
                        "-L", libdir, "-ldfc", "-Wl,-rpath," + libdir, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-2000:]
    assert "c abi ok" in r.stdout


def test_ans_frequencies_take_back_tie():
    """The host encoder's frequencies for the hand-worked take-back tie (two
    equal largest shares, an odd number of units to take back: the smaller
    symbol gives one more), read from the container it writes."""
    from oracle import ans as oans
    h = np.zeros(256, dtype=np.uint64)
    h[10] = h[20] = 10 ** 6
    h[100:201] = 1
    e = np.repeat(np.arange(256, dtype=np.uint16), h.astype(np.int64))
    x = (e << 7) | np.uint16(0x0011)
    np.random.default_rng(11).shuffle(x)
    blob = dfc.encode(x, layout=dfc.LAYOUT_ANS, ans_steps=64)
    f = oans.parse_ans_blob(bytes(blob))["freqs"]
    assert int(f[10]) == 1997 and int(f[20]) == 1998
    assert all(int(f[s]) == 1 for s in range(100, 201)) and int(np.asarray(f).sum()) == 4096


@pytest.mark.parametrize("kind", ["gauss", "outliers", "student_t", "bimodal", "uniform", "ladder", "tiny"])
def test_automatic_chunk_size_matches_oracle(kind):
    """The default chunk size is automatic: the library's choice and its
    container equal the oracle's (flat layout), and the result is within 2%
    of the exponent-entropy bound whenever some chunk size is."""
    x = {"gauss": lambda: synth.gaussian((512, 1024), 0.02, (150,)),
         "outliers": lambda: synth.gaussian_with_outliers((512, 1024), 0.02, (151,)),
         "student_t": lambda: synth.stress("student_t", 512, 1024),
         "bimodal": lambda: synth.stress("bimodal", 512, 1024),
         "uniform": lambda: synth.stress("uniform", 512, 1024),
         "ladder": lambda: synth.stress("ladder", 512, 1024),
         "tiny": lambda: synth.gaussian((3, 37), 0.02, (152,))}[kind]()
    e = fields.split(x)[0]
    h = cb.histogram(e)
    lengths = cb.package_merge_lengths(h, 24)
    C = bl.choose_chunk_bytes(h, lengths)
    b = dfc.encode(x)
    info = dfc.blob_info(b)
    assert info.chunk_bytes == C, kind
    assert bytes(b) == bl.write_blob(st.encode(x, C, 64), 11, *x.shape), kind
    bound = bl.entropy_bound_bytes(h)
    sizes = [dfc.blob_info(dfc.encode(x, chunk_bytes=c)).coded_bytes for c in (4, 8, 16, 32)]
    if min(sizes) <= 1.02 * bound:
        assert info.coded_bytes <= 1.02 * bound, kind
    if kind == "uniform":
        assert C == 32
    if kind in ("gauss", "outliers"):
        assert C == 16
