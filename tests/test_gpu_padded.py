"""GPU parity of the HIP decoder on padded-layout containers (no chunk
offsets), called through the C ABI.

Every case compares the kernel's output bit for bit with the original tensor
and, at sizes the oracle decodes in seconds, with the oracle's decode of the
same container.  Full-size workloads run in the benchmark's launch
configuration; there the oracle decodes sampled blocks."""
import struct
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import blob as bl
from oracle import codebook as cb
from oracle import fields
from oracle import padded as pd

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PADDED = dfc.LAYOUT_PADDED


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# Every test runs twice: with each block's first complete rounds stored
# during the next block's decode, and with every round stored at once (the
# decoder picks one by job size; these inputs are small enough that it would
# always pick the second).
MODE = {"stores": dfc.STORES_AUTO}


@pytest.fixture(scope="module", autouse=True, params=[dfc.STORES_DEFERRED, dfc.STORES_IMMEDIATE],
                ids=["deferred", "immediate"])
def _device(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    MODE["stores"] = request.param
    dfc.set_launch(0, 0, MODE["stores"])
    yield
    MODE["stores"] = dfc.STORES_AUTO
    dfc.set_launch(0, 0)


def gpu_decode(blob: np.ndarray, info=None):
    info = info or dfc.blob_info(blob)
    dev = torch.from_numpy(np.array(blob, dtype=np.uint8)).cuda()
    out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode(dev, info, out, status)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), int(status.item())


def check(x, C=16, k=11, oracle=True, label="", codebook=None):
    say("case padded", label, np.shape(x), "C", C, "k", k)
    blob = dfc.encode(x, chunk_bytes=C, lut_bits=k, layout=PADDED, codebook=codebook)
    got, status = gpu_decode(blob)
    assert status == 0, label
    assert np.array_equal(got, np.asarray(x).ravel()), label
    if oracle:
        assert np.array_equal(got, pd.decode_padded_blob(bytes(blob))), label
    return blob


@pytest.mark.parametrize("C", [4, 8, 16, 32])
def test_all_chunk_sizes_and_table_widths(C):
    x = synth.gaussian_with_outliers((300, 1000), 0.02, (70, C))   # many blocks, ragged tail
    for k in (8, 10, 11, 12):
        check(x, C, k, label=f"outliers k{k}")


@pytest.mark.parametrize("kind", ["uniform", "ladder", "bimodal", "t"])
def test_distributions(kind):
    shape = (211, 1013)
    x = {"uniform": lambda: synth.uniform_bits(shape, (71,)),
         "ladder": lambda: synth.exponent_ladder(shape, (72,)),
         "bimodal": lambda: synth.bimodal(shape, 0.02, (73,)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (74,))}[kind]()
    for C in (4, 8, 16, 32):
        for k in (8, 12):
            check(x, C, k, label=kind)


def test_long_codes_at_chunk_ends():
    """A 24-bit-limited code over all 256 exponents with k = 8: codes longer
    than the window fall on chunk ends, where the tail of ones is read as a
    long code and must be dropped."""
    lengths_hist = (np.arange(256, dtype=np.uint64) + 1) ** 4
    book = dfc.build_codebook(lengths_hist, 24)
    assert book.max_len > 16
    x = synth.uniform_bits((97, 1021), (75,))
    for C in (4, 8, 16, 32):
        check(x, C, 8, label="long codes", codebook=book)


def test_edge_sizes():
    for n in (1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 4095, 4096, 4097, 65537):
        x = synth.gaussian((n,), 0.02, (76, n))
        for C in (4, 32):
            check(x, C, label=f"n={n}")


def test_constant_and_special_values():
    specials = np.array([0x7FC1, 0xFF81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16)
    for C in (4, 8, 16, 32):
        check(np.tile(specials, 3001), C, label="specials")
        check(np.full((100, 1000), 0x3F80, dtype=np.uint16), C, label="constant")


def test_oracle_written_container_decodes():
    x = synth.gaussian_with_outliers((128, 777), 0.02, (77,))
    for C in (4, 16):
        blob = np.frombuffer(pd.write_padded_blob(pd.encode_padded(x, C), 11, 128, 777), dtype=np.uint8)
        got, status = gpu_decode(blob)
        assert status == 0 and np.array_equal(got, x.ravel())


def test_mixed_layouts_and_chunk_sizes_in_one_batch():
    mats = [synth.gaussian_with_outliers((64 + 16 * i, 997), 0.02, (78, i)) for i in range(8)]
    cfg = [(C, lay) for C in (4, 8, 16, 32) for lay in (dfc.LAYOUT_FLAT, PADDED)]
    items = []
    for x, (C, lay) in zip(mats, cfg):
        b = dfc.encode(x, chunk_bytes=C, layout=lay)
        items.append((torch.from_numpy(b).cuda(), dfc.blob_info(b),
                      torch.empty(x.size, dtype=torch.int16, device="cuda")))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("case mixed batch")
    dfc.decode_batch(items, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for x, (_, _, out), c in zip(mats, items, cfg):
        assert np.array_equal(out.cpu().numpy().view(np.uint16), x.ravel()), c


@pytest.mark.parametrize("waves,bpw,run", [(4, 1, 0), (8, 3, 0), (16, 2, 0), (4, 16, 3), (2, 32, 2)])
def test_launch_shapes(waves, bpw, run):
    dfc.set_launch(waves, bpw, MODE["stores"], run)
    try:
        check(synth.gaussian((512, 1024), 0.02, (79,)), 8, oracle=False, label=f"launch {waves}x{bpw} run {run}")
    finally:
        dfc.set_launch(0, 0, MODE["stores"])


def test_status_flag_on_count_mismatch():
    x = synth.gaussian((64, 4096), 0.02, (80,))
    blob = dfc.encode(x, layout=PADDED)
    info = dfc.blob_info(blob)
    bad = blob.copy()
    # an output offset moved by one: the host checks only the order
    o = info.off_blockout + 4
    v = struct.unpack_from("<I", bytes(blob[o: o + 4]))[0]
    bad[o: o + 4] = np.frombuffer(struct.pack("<I", v + 1), dtype=np.uint8)
    got, status = gpu_decode(bad, dfc.blob_info(bad))
    assert status == dfc.ECORRUPT


# ---------------------------------------------------------------- full size

def sampled_oracle_check(blob, got, n_samples=4, seed=0):
    """Decode a few whole blocks with the oracle's padded chunk decoder and
    compare the GPU output at those positions."""
    p = bl.parse_blob(bytes(blob))
    rng = np.random.default_rng(seed)
    C = p["chunk_bytes"]
    picks = sorted(set(rng.integers(0, p["n_blocks"], size=n_samples).tolist()) | {p["n_blocks"] - 1})
    for b in picks:
        c0 = 64 * b
        lo, hi = p["out"][b], p["out"][b + 1]
        words = p["words"][c0 * C // 4:]
        e = pd.decode_padded(words, p["total_bits"] - 8 * C * c0, C, 64, p["lengths"])
        assert e.size == hi - lo
        assert np.array_equal(got[lo:hi], fields.merge(e, p["raw"][lo:hi])), b


def test_full_llama_block_batched():
    """The benchmark's workload (one Llama-3-8B block, seven matrices, one
    batched launch) in the padded layout at 8- and 16-byte chunks."""
    mats = list(synth.llama3_8b_block())
    for C in (8, 16):
        items, blobs = [], []
        for name, x in mats:
            b = dfc.encode(x, chunk_bytes=C, layout=PADDED)
            blobs.append(b)
            items.append((torch.from_numpy(b).cuda(), dfc.blob_info(b),
                          torch.empty(x.size, dtype=torch.int16, device="cuda")))
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        say("case full llama block padded C", C)
        dfc.decode_batch(items, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for (name, x), (_, _, out), b in zip(mats, items, blobs):
            got = out.cpu().numpy().view(np.uint16)
            assert np.array_equal(got, x.ravel()), (name, C)
            sampled_oracle_check(b, got, n_samples=2)
        del items


@pytest.mark.parametrize("kind", list(synth.STRESS_KINDS))
def test_full_stress_8192x28672(kind):
    x = synth.stress(kind)
    for C in (8, 16):
        say("case padded stress", kind, "C", C)
        blob = dfc.encode(x, chunk_bytes=C, layout=PADDED)
        got, status = gpu_decode(blob)
        assert status == 0 and np.array_equal(got, x.ravel()), (kind, C)
    sampled_oracle_check(blob, got, n_samples=2)
