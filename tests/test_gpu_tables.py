"""GPU: the decode tables every decoding workgroup derives in LDS from the
container's code (DFloat11 blog, section 03 item 1: compact lookup tables in
on-chip memory), read back through ``dfc_derive_tables``.

The tables are the library's own data, not part of the container or of the
oracle.  They are pinned here by hand-worked entries (``tests/golden/
dyadic8.json``), by closed-form cases (one-bit codes fill a window; a
24-bit code escapes), by the slot table's definition for rANS, and by a
test-side decoder (``lut_walk.table_walk_decode``) that decodes oracle-written
containers using nothing but the library's tables and must return the
original exponents.  Every workgroup size must derive the same bytes."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import ans
from oracle import blob as bl
from oracle import codebook as cb
from oracle import fields
from oracle import stream as st
from lut_walk import ESC, parse_lut, rotate, table_walk_decode

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

THREADS = (64, 256, 512, 1024)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def derived(blob, threads=256):
    blob = np.ascontiguousarray(np.frombuffer(bytes(blob), dtype=np.uint8))
    info = dfc.blob_info(blob)
    dev = torch.from_numpy(blob.copy()).cuda()
    t = dfc.derive_tables(dev, info, threads)
    torch.cuda.synchronize()
    return t.cpu().numpy().tobytes()


def container_with_lengths(lens, k, n=4096, seed=0):
    """An oracle-written flat container whose code has exactly these lengths
    (its data draws every used exponent, evenly)."""
    lens = np.asarray(lens, dtype=np.uint8)
    used = np.flatnonzero(lens)
    rng = np.random.default_rng(seed)
    e = used[rng.integers(0, used.size, n)].astype(np.uint16)
    x = (e << 7) | rng.integers(0, 2, n).astype(np.uint16) << 15 | rng.integers(0, 128, n).astype(np.uint16)
    enc = st.encode(x, 16, 64, lengths=lens)
    return bl.write_blob(enc, k), x


@pytest.mark.parametrize("threads", THREADS)
def test_golden_entries(golden, threads):
    g = golden("dyadic8.json")
    x = np.array([int(h, 16) for h in g["bf16_hex"]], dtype=np.uint16)
    k = g["lut_bits"]
    say("dyadic8 threads", threads)
    blob = bl.write_blob(st.encode(x, g["chunk_bytes"], g["lanes"]), k)
    step, wsym, mask, limit, first, base, order = parse_lut(derived(blob, threads), k)
    for ent in g["lut_entries"]:
        w = int(ent["window"], 2)
        assert int(step[w]) == int(ent["step_hex"], 16)
        assert int(step[w]) == ((ent["codes"] << 16) - ent["bits"]) & 0xFFFFFFFF
        assert int(wsym[w]) == int(ent["wsym_hex"], 16)
        assert int(mask[w]) == sum(1 << j for j in ent["mask_bits"])
    # canonical tables of the same code: 127:0, 126:10, 124:110, 125:111
    assert order[:4].tolist() == [127, 126, 124, 125] and not order[4:].any()
    assert [int(first[l]) for l in (1, 2, 3)] == [0, 2, 6]
    assert [int(base[l]) for l in (1, 2, 3)] == [0, 1, 2]
    assert int(limit[3]) == 1 << 24 and int(limit[1]) == 1 << 23 and int(limit[2]) == 3 << 22
    # lengths past the longest code: the canonical recurrence run on (no codes)
    assert all(int(limit[l]) == 1 << 24 and int(first[l]) == 1 << l and int(base[l]) == 4 for l in range(4, 25))
    assert int(limit[0]) == int(first[0]) == int(base[0]) == 0 and not limit[25:].any()
    assert [rotate(e) for e in (127, 126, 125, 124)] == [0xBF, 0x3F, 0xBE, 0x3E]


def test_one_bit_codes_fill_a_window():
    # one used symbol (plus the phantom) has 1-bit codes: a 12-bit window holds
    # 12 whole codes; the symbol entry keeps the first 4
    lens = np.zeros(256, dtype=np.uint8)
    lens[3] = lens[4] = 1
    blob, _ = container_with_lengths(lens, 12)
    step, wsym, mask, *_ = parse_lut(derived(blob), 12)
    assert int(step[0]) == ((12 << 16) - 12) and int(mask[0]) == 0xFFF
    assert int(wsym[0]) == (((4 << 16) - 4) << 32) | 0x81818181   # rotate(3) = 0x81
    assert int(step[0xFFF]) == ((12 << 16) - 12) and int(wsym[0xFFF]) & 0xFFFFFFFF == 0x02020202


def test_long_codes_escape():
    fib = [1, 1]
    while len(fib) < 40:
        fib.append(fib[-1] + fib[-2])
    h = np.zeros(256, dtype=np.uint64)
    h[:40] = fib
    lens = cb.package_merge_lengths(h, 24)
    assert lens.max() == 24
    blob, x = container_with_lengths(lens, 8)
    tabs = derived(blob)
    step, wsym, mask, *_ = parse_lut(tabs, 8)
    # the all-ones window starts with the longest code (24 bits) -> escape
    assert int(step[255]) == ESC and int(wsym[255]) == ESC << 32 and int(mask[255]) == 0
    # the all-zeros window starts with the shortest code
    assert int(step[0]) != ESC and int(mask[0]) != 0
    e, _ = fields.split(x)
    assert np.array_equal(table_walk_decode(bl.parse_blob(blob), tabs), e)


@pytest.mark.parametrize("kind", ["gauss", "ladder", "uniform", "constant"])
@pytest.mark.parametrize("k", [8, 10, 11, 12])
def test_table_walk_reproduces_data(kind, k):
    n = 3000
    x = {"gauss": lambda: synth.gaussian((n,), 0.02, (12,)),
         "ladder": lambda: synth.exponent_ladder((n,), (13,)),
         "uniform": lambda: synth.uniform_bits((n,), (14,)),
         "constant": lambda: np.full(n, 0xBC00, dtype=np.uint16)}[kind]()
    e, _ = fields.split(x)
    say("table walk", kind, k)
    for C in (4, 16, 32):
        blob = bl.write_blob(st.encode(x, C, 64), k)
        tabs = derived(blob, THREADS[C % 4])
        assert np.array_equal(table_walk_decode(bl.parse_blob(blob), tabs), e), C


@pytest.mark.parametrize("kind", ["gauss", "ladder", "uniform", "student_t"])
def test_every_workgroup_size_derives_the_same_tables(kind):
    x = {"gauss": lambda: synth.gaussian((256, 256), 0.02, (15,)),
         "ladder": lambda: synth.exponent_ladder((256, 256), (16,)),
         "uniform": lambda: synth.uniform_bits((256, 256), (17,)),
         "student_t": lambda: synth.student_t((256, 256), 3, 0.02, (18,))}[kind]()
    for k in (8, 11, 12):
        blob = dfc.encode(x, lut_bits=k)
        ref = derived(blob, 64)
        for threads in THREADS[1:]:
            assert derived(blob, threads) == ref, (k, threads)


def slot_table_definition(f):
    """Per slot: rotated exponent | (f - 1) << 8 | (slot - cum) << 20, for the
    symbol whose range [cum, cum + f) holds the slot."""
    t = np.zeros(4096, dtype=np.uint32)
    cum = 0
    for s in range(256):
        for slot in range(cum, cum + int(f[s])):
            t[slot] = rotate(s) | ((int(f[s]) - 1) << 8) | ((slot - cum) << 20)
        cum += int(f[s])
    assert cum == 4096
    return t


@pytest.mark.parametrize("kind", ["gauss", "uniform", "one_symbol", "sparse"])
def test_rans_slot_table(kind):
    rng = np.random.default_rng(92)
    if kind == "sparse":
        # symbols 0 and 255 present, large gaps of absent symbols
        e = rng.choice(np.array([0, 3, 77, 200, 255], dtype=np.uint16), 5000, p=[0.5, 0.1, 0.2, 0.15, 0.05])
        x = (e << 7) | rng.integers(0, 128, e.size).astype(np.uint16)
    else:
        x = {"gauss": lambda: synth.gaussian((64, 1000), 0.02, (93,)),
             "uniform": lambda: synth.uniform_bits((64, 1000), (94,)),
             "one_symbol": lambda: np.full(3000, 0x3F80, dtype=np.uint16)}[kind]()
    blob = ans.write_ans_blob(ans.encode_ans(x, 64))
    f = ans.parse_ans_blob(blob)["freqs"]
    want = slot_table_definition(f)
    for threads in THREADS:
        got = np.frombuffer(derived(blob, threads), dtype="<u4")
        assert np.array_equal(got, want), threads


def test_derive_tables_rejects_bad_arguments():
    blob = dfc.encode(synth.gaussian((64, 64), 0.02, (19,)))
    info = dfc.blob_info(blob)
    dev = torch.from_numpy(blob.copy()).cuda()
    lib = dfc.library()
    out = torch.empty(dfc.derived_tables_bytes(info) + 16, dtype=torch.uint8, device="cuda")
    assert lib.dfc_derive_tables(dev.data_ptr(), info, 96, out.data_ptr(), out.numel(), None) == dfc.EINVAL
    assert lib.dfc_derive_tables(dev.data_ptr(), info, 2048, out.data_ptr(), out.numel(), None) == dfc.EINVAL
    assert lib.dfc_derive_tables(dev.data_ptr(), info, 256, out.data_ptr() + 8, out.numel(), None) == dfc.EINVAL
    assert lib.dfc_derive_tables(dev.data_ptr(), info, 256, out.data_ptr(), 100, None) == dfc.ESIZE
    empty = dfc.encode(np.zeros(0, dtype=np.uint16))
    einfo = dfc.blob_info(empty)
    edev = torch.from_numpy(empty.copy()).cuda()
    assert lib.dfc_derive_tables(edev.data_ptr(), einfo, 256, out.data_ptr(), out.numel(), None) == dfc.EINVAL
