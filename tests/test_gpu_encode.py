"""GPU encoder (dfc_encode_device) through the C ABI, in the flat, panel and
rANS layouts: its containers must be byte-identical to the host encoder's
(which the oracle pins byte for byte), and decode back to the input."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import blob as bl
from oracle import codebook as cb
from oracle import fields

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.int16)).cuda()


def same_as_host(x, C=16, k=11, T=64, codebook=None, label=""):
    say("case", label, np.shape(x), "C", C, "k", k, "T", T)
    x = np.asarray(x, dtype=np.uint16)
    shape = x.shape if x.ndim == 2 else None
    host = dfc.encode(x, chunk_bytes=C, lut_bits=k, lanes=T, codebook=codebook, shape=shape)
    d, size = dfc.encode_device(dev16(x), chunk_bytes=C, lut_bits=k, lanes=T, codebook=codebook, shape=shape)
    got = d[:size].cpu().numpy()
    assert size == host.size, label
    assert np.array_equal(got, host), label
    return got


@pytest.mark.parametrize("C", [4, 8, 16, 32])
def test_matches_host_all_chunk_sizes(C):
    x = synth.gaussian_with_outliers((300, 1000), 0.02, (100, C))
    for k in (8, 11, 12):
        same_as_host(x, C, k, label=f"outliers C{C}")


@pytest.mark.parametrize("kind", ["uniform", "ladder", "bimodal", "t"])
def test_matches_host_distributions(kind):
    shape = (257, 1031)
    x = {"uniform": lambda: synth.uniform_bits(shape, (101,)),
         "ladder": lambda: synth.exponent_ladder(shape, (102,)),
         "bimodal": lambda: synth.bimodal(shape, 0.02, (103,)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (104,))}[kind]()
    for C in (4, 16, 32):
        same_as_host(x, C, label=kind)


def test_edge_sizes_and_lanes():
    for n in (1, 2, 15, 16, 17, 4095, 4096, 4097, 65537):
        same_as_host(synth.gaussian((n,), 0.02, (105, n)), 4, label=f"n={n}")
    x = synth.gaussian((64, 4099), 0.02, (106,))
    same_as_host(x, 8, T=64, label="T=64")
    with pytest.raises(dfc.DfcError):
        dfc.encode_device(dev16(x), chunk_bytes=8, lanes=128)


def test_special_values_and_constant():
    specials = np.array([0x7FC1, 0xFF81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16)
    same_as_host(np.tile(specials, 3001), 8, label="specials")
    same_as_host(np.full((100, 100), 0x3F80, dtype=np.uint16), 4, label="constant")


def test_external_codebook_and_decode():
    g = synth.gaussian((512, 512), 0.02, (107,))
    book = dfc.build_codebook(cb.histogram(fields.split(g)[0]) + 1, 24)
    x = synth.uniform_bits((200, 999), (108,))
    blob = same_as_host(x, 16, codebook=book, label="foreign codebook")
    assert np.array_equal(bl.decode_blob(bytes(blob)), x.ravel())


def test_errors():
    x = synth.gaussian((64, 64), 0.02, (109,))
    book = dfc.build_codebook(cb.histogram(fields.split(x)[0]), 24)
    y = synth.uniform_bits((64, 64), (110,))   # exponents the book does not cover
    with pytest.raises(dfc.DfcError) as ei:
        dfc.encode_device(dev16(y), codebook=book, shape=(64, 64))
    assert ei.value.status == dfc.EINVAL


@pytest.mark.parametrize("name_shape", [("gate", (14336, 4096)), ("wk", (1024, 4096))])
def test_full_size_block_matrices(name_shape):
    name, shape = name_shape
    x = dict(synth.llama3_8b_block())[name]
    assert x.shape == shape
    d, size = dfc.encode_device(dev16(x), shape=shape)
    host = dfc.encode(x)
    say("case full", name)
    assert size == host.size
    assert torch.equal(d[:size], torch.from_numpy(host).cuda())
    info = dfc.blob_info(host)
    out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
    dfc.decode(d, info, out)
    torch.cuda.synchronize()
    assert torch.equal(out, dev16(x))


# ---------------------------------------------------------------- rANS layout

ANS = dfc.LAYOUT_ANS


def ans_same_as_host(x, steps, label=""):
    say("case ans", label, np.shape(x), "steps", steps)
    x = np.asarray(x, dtype=np.uint16)
    shape = x.shape if x.ndim == 2 else None
    host = dfc.encode(x, shape=shape, layout=ANS, ans_steps=steps)
    d, size = dfc.encode_device(dev16(x), shape=shape, layout=ANS, ans_steps=steps)
    got = d[:size].cpu().numpy()
    assert size == host.size, label
    assert np.array_equal(got, host), label
    return got


@pytest.mark.parametrize("steps", [8, 64, 512, 1024])
def test_ans_matches_host_block_sizes(steps):
    x = synth.gaussian_with_outliers((300, 1000), 0.02, (120, steps))
    ans_same_as_host(x, steps, label="outliers")


@pytest.mark.parametrize("kind", ["uniform", "ladder", "bimodal", "t"])
def test_ans_matches_host_distributions(kind):
    shape = (257, 1031)
    x = {"uniform": lambda: synth.uniform_bits(shape, (121,)),
         "ladder": lambda: synth.exponent_ladder(shape, (122,)),
         "bimodal": lambda: synth.bimodal(shape, 0.02, (123,)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (124,))}[kind]()
    for steps in (16, 256):
        ans_same_as_host(x, steps, label=kind)


def test_ans_edge_sizes_specials_and_one_symbol():
    for n in (0, 1, 2, 63, 64, 65, 511, 512, 513, 4097):
        ans_same_as_host(synth.gaussian((n,), 0.02, (125, n)), 8, label=f"n={n}")
    specials = np.array([0x7FC1, 0xFF81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16)
    ans_same_as_host(np.tile(specials, 3001), 64, label="specials")
    ans_same_as_host(np.full((100, 100), 0x3F80, dtype=np.uint16), 16, label="one symbol (f = 4096)")


def test_ans_rejects_external_codebook():
    x = synth.gaussian((64, 64), 0.02, (126,))
    book = dfc.build_codebook(cb.histogram(fields.split(x)[0]), 24)
    with pytest.raises(dfc.DfcError) as ei:
        dfc.encode_device(dev16(x), codebook=book, shape=(64, 64), layout=ANS)
    assert ei.value.status == dfc.EINVAL


def test_ans_full_size_gate_matrix_and_decode():
    x = dict(synth.llama3_8b_block())["gate"]
    say("case ans full gate")
    d, size = dfc.encode_device(dev16(x), shape=x.shape, layout=ANS, ans_steps=512)
    host = dfc.encode(x, layout=ANS, ans_steps=512)
    assert size == host.size
    assert torch.equal(d[:size], torch.from_numpy(host).cuda())
    info = dfc.blob_info(host)
    out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode(d, info, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, dev16(x))


# --------------------------------------------------------------- panel layout

PANEL = dfc.LAYOUT_PANEL


@pytest.mark.parametrize("shape,panel_k,C", [
    ((64, 1040), 1024, 16),     # a narrow last slice (16 columns)
    ((96, 272), 64, 4),         # five slices, the last one 16 wide
    ((128, 512), 512, 8),       # one item per panel
    ((32, 48), 16, 32),         # one-sub-tile items
    ((256, 4096), 256, 16),
])
def test_panel_matches_host(shape, panel_k, C):
    x = synth.gaussian_with_outliers(shape, 0.02, (180, shape[0], panel_k))
    say("case panel", shape, "panel_k", panel_k, "C", C)
    host = dfc.encode(x, chunk_bytes=C, layout=PANEL, panel_k=panel_k)
    d, size = dfc.encode_device(dev16(x), chunk_bytes=C, shape=shape, layout=PANEL, panel_k=panel_k)
    assert size == host.size
    assert np.array_equal(d[:size].cpu().numpy(), host)


@pytest.mark.parametrize("kind", ["uniform", "ladder"])
def test_panel_matches_host_distributions_and_codebook(kind):
    shape = (96, 1024)
    x = {"uniform": lambda: synth.uniform_bits(shape, (181,)),
         "ladder": lambda: synth.exponent_ladder(shape, (182,))}[kind]()
    host = dfc.encode(x, layout=PANEL, panel_k=256)
    d, size = dfc.encode_device(dev16(x), shape=shape, layout=PANEL, panel_k=256)
    assert size == host.size and np.array_equal(d[:size].cpu().numpy(), host), kind
    g = synth.gaussian((512, 512), 0.02, (183,))
    book = dfc.build_codebook(cb.histogram(fields.split(g)[0]) + 1, 24)
    host = dfc.encode(x, layout=PANEL, panel_k=256, codebook=book)
    d, size = dfc.encode_device(dev16(x), shape=shape, layout=PANEL, panel_k=256, codebook=book)
    assert size == host.size and np.array_equal(d[:size].cpu().numpy(), host), kind + " foreign codebook"


def test_panel_full_size_gemm_matrix():
    w = synth.gemm_weight()
    say("case panel full 28672 x 8192")
    d, size = dfc.encode_device(dev16(w), shape=w.shape, layout=PANEL)
    host = dfc.encode(w, layout=PANEL)
    assert size == host.size
    assert torch.equal(d[:size], torch.from_numpy(host).cuda())


@pytest.mark.parametrize("layout", ["flat", "panel", "ans"])
def test_source_not_16_byte_aligned(layout):
    """A source two bytes past a 16-byte boundary takes the encoder's scalar
    load paths (histogram, segment loads, raw bytes, panel octets); the
    container must still equal the host encoder's."""
    shape = (64, 1040) if layout == "panel" else (1, 200003)
    x = synth.gaussian_with_outliers(shape, 0.02, (181, shape[0], shape[1])).astype(np.uint16)
    n = x.size
    base = torch.empty(n + 8, dtype=torch.int16, device="cuda")
    src = base[1: n + 1]
    src.copy_(dev16(x))
    assert src.data_ptr() % 16 == 2 and src.is_contiguous()
    say("case unaligned", layout, shape)
    kw = {"flat": {}, "panel": {"layout": PANEL, "panel_k": 1024}, "ans": {"layout": dfc.LAYOUT_ANS}}[layout]
    host = dfc.encode(x, shape=shape, **kw)
    d, size = dfc.encode_device(src, shape=shape, **kw)
    assert size == host.size
    assert np.array_equal(d[:size].cpu().numpy(), host)


@pytest.mark.parametrize("layout", ["flat", "ans", "panel"])
def test_device_containers_equal_the_oracles(layout):
    """Containers written by the GPU encoder compared byte for byte with the
    oracle's own writers (not only with the host encoder)."""
    from oracle import ans as oans
    from oracle import panel as opanel
    from oracle import stream as ost
    for j, shape in enumerate(((64, 1008), (96, 2048), (1, 4097), (32, 16))):
        if layout == "panel" and shape[0] % 32:
            continue
        x = synth.gaussian_with_outliers(shape, 0.02, (108, j))
        say("oracle vs device", layout, shape)
        if layout == "flat":
            for C in (4, 16):
                d, size = dfc.encode_device(dev16(x), chunk_bytes=C, shape=shape)
                want = bl.write_blob(ost.encode(x, C, 64), 11, *shape)
                assert size == len(want) and bytes(d[:size].cpu().numpy()) == want, (shape, C)
        elif layout == "ans":
            d, size = dfc.encode_device(dev16(x), layout=dfc.LAYOUT_ANS, ans_steps=64, shape=shape)
            want = oans.write_ans_blob(oans.encode_ans(x, 64), *shape)
            assert size == len(want) and bytes(d[:size].cpu().numpy()) == want, shape
        else:
            d, size = dfc.encode_device(dev16(x), layout=dfc.LAYOUT_PANEL, panel_k=256, chunk_bytes=8, shape=shape)
            want = opanel.write_panel_blob(opanel.encode_panel(x, 256, 8, 64), 11)
            assert size == len(want) and bytes(d[:size].cpu().numpy()) == want, shape
