"""GPU: decoding with decode tables prepared once by dfc_derive_tables
(passed as tables_dev) instead of derived by every workgroup.  Both paths
must give the original bits in every layout, chunk size and table width, in
one batch together, and in the fused product; tables of another container
must not pass as correct output; misaligned or short tables are refused."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import ans
from oracle import blob as bl
from oracle import gemm as og
from oracle import stream as st

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dfc.set_launch(0, 0)


def dev(blob):
    if isinstance(blob, (bytes, bytearray)):
        blob = np.frombuffer(bytes(blob), dtype=np.uint8)
    return torch.from_numpy(np.array(blob, dtype=np.uint8)).cuda()


def decode(blob, tables="prepared"):
    info = dfc.blob_info(blob)
    d = dev(blob)
    t = dfc.derive_tables(d, info) if tables == "prepared" else tables
    out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode(d, info, out, status, tables=t)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), int(status.item())


@pytest.mark.parametrize("layout", [dfc.LAYOUT_FLAT, dfc.LAYOUT_PADDED])
@pytest.mark.parametrize("k", [8, 10, 11, 12])
def test_every_chunk_size_and_table_width(layout, k):
    x = synth.gaussian_with_outliers((333, 1001), 0.02, (40, k))
    for C in (4, 8, 16, 32):
        got, status = decode(dfc.encode(x, chunk_bytes=C, lut_bits=k, layout=layout))
        assert status == 0 and np.array_equal(got, x.ravel()), (C, k)


@pytest.mark.parametrize("kind", ["student_t", "bimodal", "uniform", "ladder"])
def test_distributions_and_oracle_containers(kind):
    x = synth.stress(kind, 257, 999)
    for C in (8, 32):
        got, status = decode(bl.write_blob(st.encode(x, C, 64), 11))
        assert status == 0 and np.array_equal(got, x.ravel()), C
    got, status = decode(ans.write_ans_blob(ans.encode_ans(x, 64)))
    assert status == 0 and np.array_equal(got, x.ravel())


def test_edge_sizes():
    for n in (1, 2, 7, 8, 9, 511, 512, 513, 4095, 4097, 20000):
        x = synth.gaussian((n,), 0.02, (41, n))
        for layout, kw in ((dfc.LAYOUT_FLAT, {}), (dfc.LAYOUT_PADDED, {"chunk_bytes": 4}),
                           (dfc.LAYOUT_ANS, {"ans_steps": 8})):
            got, status = decode(dfc.encode(x, layout=layout, **kw))
            assert status == 0 and np.array_equal(got, x), (n, layout)


def test_batch_mixes_prepared_and_derived_tables():
    xs = [synth.gaussian_with_outliers((128 + 37 * j, 512), 0.02, (42, j)) for j in range(12)]
    cfg = [(dfc.LAYOUT_FLAT, 16, 11), (dfc.LAYOUT_PADDED, 8, 10), (dfc.LAYOUT_ANS, 16, 11),
           (dfc.LAYOUT_FLAT, 32, 12)] * 3
    items, refs = [], []
    for j, (x, (layout, C, k)) in enumerate(zip(xs, cfg)):
        b = dfc.encode(x, chunk_bytes=C, lut_bits=k, layout=layout, ans_steps=64 if layout == dfc.LAYOUT_ANS else 0)
        info = dfc.blob_info(b)
        d = dev(b)
        out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
        if j % 2:
            items.append((d, info, out, dfc.derive_tables(d, info, threads=64 * (1 + j % 16))))
        else:
            items.append((d, info, out))
        refs.append(x)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode_batch(items, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for (_, _, out, *_), x in zip(items, refs):
        assert np.array_equal(out.cpu().numpy().view(np.uint16), x.ravel())


def test_fused_product_with_prepared_tables():
    w = synth.gaussian((256, 1024), 0.02, (43,))
    xb = synth.gaussian((16, 1024), 1.0, (44,))
    blob = dfc.encode(w, layout=dfc.LAYOUT_PANEL, panel_k=256)
    info = dfc.blob_info(blob)
    d = dev(blob)
    tabs = dfc.derive_tables(d, info)
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    ys = []
    for t in (tabs, None):
        y = torch.empty((16, 256), dtype=torch.float32, device="cuda")
        dfc.decode_gemm(d, info, x, y, tables=t)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    ref = og.gemm_reference(w, xb.T).T
    err = np.abs(ys[0].cpu().numpy().astype(np.float64) - ref)
    assert err.max() <= 1e-3 * np.abs(ref).max()


def test_tables_of_another_container_do_not_pass():
    a = synth.gaussian((200, 512), 0.02, (45,))
    b = synth.exponent_ladder((200, 512), (46,))
    ba, bb = dfc.encode(a), dfc.encode(b)
    ia, ib = dfc.blob_info(ba), dfc.blob_info(bb)
    tb = dfc.derive_tables(dev(bb), ib)
    got, status = decode(ba, tables=tb)
    assert status == dfc.ECORRUPT or not np.array_equal(got, a.ravel())


def test_bad_tables_refused():
    x = synth.gaussian((64, 64), 0.02, (47,))
    blob = dfc.encode(x)
    info = dfc.blob_info(blob)
    d = dev(blob)
    t = dfc.derive_tables(d, info)
    out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
    lib = dfc.library()
    assert lib.dfc_decode(d.data_ptr(), info, t.data_ptr() + 8, out.data_ptr(), info.n, None, None) == dfc.EINVAL
    with pytest.raises(ValueError):
        dfc.decode(d, info, out, tables=t[:100])
    with pytest.raises(TypeError):
        dfc.decode(d, info, out, tables=t.cpu())
