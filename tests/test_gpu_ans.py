"""GPU parity of the interleaved rANS decoder (containers in the ANS layout),
called through the C ABI.

Every case compares the kernel's output bit for bit with the original tensor
and, at sizes the oracle decodes in seconds, with the oracle's decode of the
same container.  Full-size workloads run in the benchmark's launch; there the
oracle decodes sampled blocks."""
import struct
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import ans
from oracle import fields

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ANS = dfc.LAYOUT_ANS


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def gpu_decode(blob: np.ndarray, info=None):
    info = info or dfc.blob_info(blob)
    dev = torch.from_numpy(np.array(blob, dtype=np.uint8)).cuda()
    out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode(dev, info, out, status)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), int(status.item())


def check(x, steps=512, oracle=True, label=""):
    say("case ans", label, np.shape(x), "steps", steps)
    blob = dfc.encode(x, layout=ANS, ans_steps=steps)
    got, status = gpu_decode(blob)
    assert status == 0, label
    assert np.array_equal(got, np.asarray(x).ravel()), label
    if oracle:
        assert np.array_equal(got, ans.decode_ans_blob(bytes(blob))), label
    return blob


@pytest.mark.parametrize("steps", [8, 16, 64, 512, 1024])
def test_block_sizes(steps):
    x = synth.gaussian_with_outliers((300, 1000), 0.02, (130, steps))   # many blocks, ragged tail
    check(x, steps, label="outliers")


@pytest.mark.parametrize("kind", ["uniform", "ladder", "bimodal", "t"])
def test_distributions(kind):
    shape = (211, 1013)
    x = {"uniform": lambda: synth.uniform_bits(shape, (131,)),
         "ladder": lambda: synth.exponent_ladder(shape, (132,)),
         "bimodal": lambda: synth.bimodal(shape, 0.02, (133,)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (134,))}[kind]()
    for steps in (8, 256):
        check(x, steps, label=kind)


def test_edge_sizes():
    for n in (1, 2, 7, 8, 9, 63, 64, 65, 511, 512, 513, 4095, 4097, 65537):
        x = synth.gaussian((n,), 0.02, (135, n))
        for steps in (8, 64):
            check(x, steps, label=f"n={n}")


def test_constant_and_special_values():
    specials = np.array([0x7FC1, 0xFF81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16)
    check(np.tile(specials, 3001), 16, label="specials")
    check(np.full((100, 1000), 0x3F80, dtype=np.uint16), 64, label="constant (one symbol: no words)")


def test_oracle_written_container_decodes():
    x = synth.gaussian_with_outliers((128, 777), 0.02, (136,))
    blob = np.frombuffer(ans.write_ans_blob(ans.encode_ans(x, 32), 128, 777), dtype=np.uint8)
    got, status = gpu_decode(blob)
    assert status == 0 and np.array_equal(got, x.ravel())


def test_mixed_layouts_in_one_batch():
    mats = [synth.gaussian_with_outliers((64 + 16 * i, 997), 0.02, (137, i)) for i in range(6)]
    cfg = [(dfc.LAYOUT_FLAT, {}), (ANS, {"ans_steps": 8}), (dfc.LAYOUT_PADDED, {}),
           (ANS, {"ans_steps": 512}), (ANS, {"ans_steps": 64}), (dfc.LAYOUT_FLAT, {"chunk_bytes": 4})]
    items = []
    for x, (lay, kw) in zip(mats, cfg):
        b = dfc.encode(x, layout=lay, **kw)
        items.append((torch.from_numpy(b).cuda(), dfc.blob_info(b),
                      torch.empty(x.size, dtype=torch.int16, device="cuda")))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("case mixed layouts batch")
    dfc.decode_batch(items, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for x, (_, _, out), c in zip(mats, items, cfg):
        assert np.array_equal(out.cpu().numpy().view(np.uint16), x.ravel()), c


def test_status_flag_on_corrupt_stream():
    x = synth.gaussian((64, 4096), 0.02, (138,))
    blob = dfc.encode(x, layout=ANS, ans_steps=64)
    info = dfc.blob_info(blob)
    # a changed initial state passes the host check but does not return to 2^16
    bad = blob.copy()
    o = info.off_blockout + 4 * 5
    v = struct.unpack_from("<I", bytes(blob[o: o + 4]))[0]
    bad[o: o + 4] = np.frombuffer(struct.pack("<I", v ^ 0x100), dtype=np.uint8)
    got, status = gpu_decode(bad, dfc.blob_info(bad))
    assert status == dfc.ECORRUPT
    # a flipped stream bit either trips the check or changes a value
    flip = blob.copy()
    flip[info.off_words + 1000] ^= 0x10
    got, status = gpu_decode(flip, info)
    assert status == dfc.ECORRUPT or (status == 0 and not np.array_equal(got, x.ravel()))


# ---------------------------------------------------------------- full size

def sampled_oracle_check(blob, got, n_samples=3, seed=0):
    p = ans.parse_ans_blob(bytes(blob))
    rng = np.random.default_rng(seed)
    per = 64 * p["steps"]
    picks = sorted(set(rng.integers(0, p["n_blocks"], size=n_samples).tolist()) | {p["n_blocks"] - 1})
    for b in picks:
        lo, hi = b * per, min(p["n"], (b + 1) * per)
        one = {"n": hi - lo, "lanes": 64, "steps": p["steps"], "freqs": p["freqs"], "n_blocks": 1,
               "states": p["states"][b: b + 1],
               "offsets": p["offsets"][b: b + 2] - p["offsets"][b],
               "words": p["words"][p["offsets"][b]: p["offsets"][b + 1]]}
        e = ans.decode_ans(one)
        assert np.array_equal(got[lo:hi], fields.merge(e, p["raw"][lo:hi])), b


def test_full_llama_block_batched():
    mats = list(synth.llama3_8b_block())
    for steps in (512, 1024):
        items, blobs = [], []
        for name, x in mats:
            b = dfc.encode(x, layout=ANS, ans_steps=steps)
            blobs.append(b)
            items.append((torch.from_numpy(b).cuda(), dfc.blob_info(b),
                          torch.empty(x.size, dtype=torch.int16, device="cuda")))
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        say("case full llama block ans steps", steps)
        dfc.decode_batch(items, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for (name, x), (_, _, out), b in zip(mats, items, blobs):
            got = out.cpu().numpy().view(np.uint16)
            assert np.array_equal(got, x.ravel()), (name, steps)
            sampled_oracle_check(b, got, n_samples=1)
        del items


@pytest.mark.parametrize("kind", list(synth.STRESS_KINDS))
def test_full_stress_8192x28672(kind):
    x = synth.stress(kind)
    say("case ans stress", kind)
    blob = dfc.encode(x, layout=ANS, ans_steps=512)
    got, status = gpu_decode(blob)
    assert status == 0 and np.array_equal(got, x.ravel()), kind
    sampled_oracle_check(blob, got, n_samples=1)
