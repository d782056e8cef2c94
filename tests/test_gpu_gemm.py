"""GPU parity of the fused decode + matrix product (dfc_decode_gemm), called
through the C ABI.

Y starts as NaN in every case, so an element the kernel leaves unwritten
fails.  Two checks that do not depend on the summation order:

* exactness of the decode inside the fused path: with X made of unit
  vectors e_k, every product has one non-zero term, so Y's columns are W's
  columns exactly (bf16 -> fp32 is exact);
* the product for seeded random X against the oracle's float64 W X, within
  the tolerance of the fp32 accumulation: |Y - Y_ref| <= 1e-3 max|Y_ref|
  overall and <= 1e-3 (|W| |X|) per element.
"""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import gemm as og
from oracle import panel as pn

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def upload(w, C=16, k=11, panel_k=1024):
    blob = dfc.encode(w, chunk_bytes=C, lut_bits=k, layout=dfc.LAYOUT_PANEL, panel_k=panel_k)
    info = dfc.blob_info(blob)
    return torch.from_numpy(blob).cuda(), info, blob


def run(dev, info, x_bits):
    """x_bits: (B, K) uint16 host array -> Y (B, M) float32 host array."""
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
    # every element must be written
    y = torch.full((x_bits.shape[0], info.rows), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode_gemm(dev, info, x, y, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return y.cpu().numpy()


def unit_vectors(K, cols):
    x = np.zeros((len(cols), K), dtype=np.uint16)
    x[np.arange(len(cols)), cols] = 0x3F80  # bf16 1.0
    return x


def normal_finite(w):
    """Uniform bit patterns with every exponent moved into 1..254: the
    product path is held to finite normal weights (the decode of zero,
    subnormal, Inf and NaN patterns is checked bit-exactly by the flat
    decoder's tests)."""
    e = (w >> 7) & 0xFF
    e = np.clip(e, 1, 254).astype(np.uint16)
    return (w & np.uint16(0x807F)) | (e << 7)


def w_as_f32(w):
    return (w.astype(np.uint32) << 16).view(np.float32)


def check_product(w, x_rows, y):
    """y (B, M) against the oracle's float64 W X for X = x_rows^T."""
    ref = og.gemm_reference(w, x_rows.T).T
    bound = og.abs_product_bound(w, x_rows.T).T
    err = np.abs(y.astype(np.float64) - ref)
    assert err.max() <= TOL * np.abs(ref).max() + 1e-30
    assert (err <= TOL * bound + 1e-30).all()


@pytest.mark.parametrize("C", [4, 8, 16, 32])
def test_unit_vectors_recover_w_exactly(C):
    M, K = 96, 272
    w = synth.gaussian_with_outliers((M, K), 0.02, (80, C))
    dev, info, _ = upload(w, C=C, panel_k=64)
    wf = w_as_f32(w)
    for c0 in range(0, K, 64):
        cols = list(range(c0, min(K, c0 + 64)))
        say("case unit vectors C", C, "cols", cols[0], "..", cols[-1])
        y = run(dev, info, unit_vectors(K, cols))
        assert np.array_equal(y, wf[:, cols].T)


@pytest.mark.parametrize("B", [1, 2, 16, 31, 32, 33, 64])
def test_product_against_oracle(B):
    M, K = 128, 1040     # two column slices of 1024 and 16
    w = synth.gaussian_with_outliers((M, K), 0.02, (81, B))
    x = synth.gaussian((B, K), 1.0, (82, B))
    dev, info, _ = upload(w, C=16, panel_k=1024)
    say("case product B", B)
    check_product(w, x, run(dev, info, x))


@pytest.mark.parametrize("M,K,panel_k", [
    (160, 1040, 1024),   # 2 slices, 5 panels: four panels per workgroup, ragged last round
    (96, 1040, 64),      # 17 slices (last one 16 wide): wavefronts take 3, 2, 2, ... slices
    (64, 2048, 2048),    # 1 slice: eight panels per workgroup, six of them idle
    (288, 512, 32),      # 16 slices of one sub-tile width, 9 panels
    (32, 48, 16),        # one panel of 3 one-sub-tile slices
])
@pytest.mark.parametrize("B", [5, 33])
def test_slices_and_panel_groups(M, K, panel_k, B):
    """Panels of 1 to 17 column slices, split over a workgroup's wavefronts
    (and, past 8 slices, over several workgroups added with atomics) and
    summed in LDS: against the oracle, and, with at most 8 slices (one
    workgroup per panel, fixed summation order), the same bits on a second
    run."""
    w = synth.gaussian_with_outliers((M, K), 0.02, (90, M, K))
    x = synth.gaussian((B, K), 1.0, (91, B))
    dev, info, _ = upload(w, C=8, panel_k=panel_k)
    say("case slices M", M, "K", K, "panel_k", panel_k, "B", B)
    y = run(dev, info, x)
    check_product(w, x, y)
    if -(-K // panel_k) <= 8:
        assert np.array_equal(y.view(np.uint32), run(dev, info, x).view(np.uint32))
    cols = list(range(K - min(K, 64), K))
    assert np.array_equal(run(dev, info, unit_vectors(K, cols)), w_as_f32(w)[:, cols].T)


@pytest.mark.parametrize("M,K", [(1024, 4096), (4096, 14336)])
def test_transformer_block_shapes(M, K):
    """Wk/Wv- and down-shaped matrices of a Llama-3-8B block with 256-column
    items: 16 or 56 slices per panel and too few panels to fill the GPU, so
    each panel is shared by several workgroups whose sums are added with
    atomics.  Sampled rows against the oracle at B = 1 and 16; one 64-column
    window bit-exact with unit vectors."""
    w = synth.gaussian_with_outliers((M, K), 0.02, (92, M, K))
    dev, info, _ = upload(w, C=16, panel_k=256)
    rows = np.random.default_rng(7).choice(M, 256, replace=False)
    for B in (1, 16):
        x = synth.gaussian((B, K), 1.0, (93, B))
        say("case block shape M", M, "K", K, "B", B)
        y = run(dev, info, x)
        check_product(w[rows], x, y[:, rows])
    cols = list(range(K // 2, K // 2 + 64))
    assert np.array_equal(run(dev, info, unit_vectors(K, cols)), w_as_f32(w)[:, cols].T)


@pytest.mark.parametrize("kind", list(synth.STRESS_KINDS))
def test_stress_distributions(kind):
    M, K = 64, 512
    w = {"student_t": lambda: synth.student_t((M, K), 3.0, 0.02, (83,)),
         "bimodal": lambda: synth.bimodal((M, K), 0.02, (84,)),
         "uniform": lambda: normal_finite(synth.uniform_bits((M, K), (85,))),
         "ladder": lambda: synth.exponent_ladder((M, K), (86,))}[kind]()
    dev, info, _ = upload(w, C=8, k=10, panel_k=128)
    say("case stress", kind)
    y = run(dev, info, unit_vectors(K, list(range(0, 64))))
    assert np.array_equal(y, w_as_f32(w)[:, :64].T)


@pytest.mark.parametrize("C", [16, 32])
def test_one_bit_codes_fill_whole_blocks(C):
    """Two equally likely exponents (126 and 127): every code is one bit, so
    a block of 64 chunks holds 512 C values and completes up to C sub-tiles,
    more than the kernel prefetches (7 at C = 16, 10 at C = 32): the rest
    load when used.  At C = 32 the staging areas are large enough that fewer
    than 8 wavefronts fit a workgroup."""
    M, K = 64, 4096
    u = synth.uniform_bits((M, K), (98, C))
    w = (u & np.uint16(0x807F)) | ((np.uint16(126) + ((u >> np.uint16(7)) & np.uint16(1))) << np.uint16(7))
    dev, info, _ = upload(w, C=C)
    assert info.max_block_elems > 512 * (7 if C == 16 else 10)
    say("case one-bit codes C", C)
    for c0 in (0, K - 64):
        cols = list(range(c0, c0 + 64))
        assert np.array_equal(run(dev, info, unit_vectors(K, cols)), w_as_f32(w)[:, cols].T)
    x = synth.gaussian((16, K), 1.0, (99, C))
    check_product(w, x, run(dev, info, x))


def test_oracle_written_container():
    w = synth.gaussian((64, 256), 0.02, (87,))
    blob = pn.write_panel_blob(pn.encode_panel(w, panel_k=128, chunk_bytes=16), 11)
    arr = np.frombuffer(blob, dtype=np.uint8)
    info = dfc.blob_info(arr)
    dev = torch.from_numpy(arr.copy()).cuda()
    y = run(dev, info, unit_vectors(256, list(range(64, 128))))
    assert np.array_equal(y, w_as_f32(w)[:, 64:128].T)


def test_invalid_arguments():
    w = synth.gaussian((64, 128), 0.02, (88,))
    dev, info, _ = upload(w)
    x = torch.zeros((65, 128), dtype=torch.int16, device="cuda")
    y = torch.zeros((65, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(dfc.DfcError) as ei:
        dfc.decode_gemm(dev, info, x, y)
    assert ei.value.status == dfc.EINVAL
    with pytest.raises(ValueError):   # Y must be float32
        dfc.decode_gemm(dev, info, x[:4], torch.zeros((4, 64), dtype=torch.int32, device="cuda"))
    flat = dfc.encode(w)
    finfo = dfc.blob_info(flat)
    with pytest.raises(ValueError):
        dfc.decode_gemm(torch.from_numpy(flat).cuda(), finfo, x[:4], y[:4])


@pytest.mark.parametrize("B", [33, 47, 64])
def test_packed_x_same_bits_as_in_place(B):
    """Batches above 32 read X through the packed copy in the workspace (the
    default) or in place (workspace=False): the same products in the same
    order, so the same bits; both against the oracle."""
    M, K = 160, 1040
    w = synth.gaussian_with_outliers((M, K), 0.02, (95, B))
    x = synth.gaussian((B, K), 1.0, (96, B))
    dev, info, _ = upload(w, C=16, panel_k=256)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    ys = []
    for ws in (None, False, torch.empty(dfc.gemm_workspace_bytes(B, K) + 64, dtype=torch.uint8, device="cuda")):
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        dfc.decode_gemm(dev, info, xd, y, status, workspace=ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        ys.append(y.cpu().numpy())
    say("case packed X B", B)
    check_product(w, x, ys[0])
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    assert np.array_equal(ys[0].view(np.uint32), ys[2].view(np.uint32))


def test_workspace_arguments():
    assert dfc.gemm_workspace_bytes(32, 8192) == 0
    assert dfc.gemm_workspace_bytes(33, 8192) == 2 * 64 * 8192
    assert dfc.gemm_workspace_bytes(64, 1040) == 2 * 64 * 1040
    w = synth.gaussian((64, 128), 0.02, (97,))
    dev, info, _ = upload(w)
    x = torch.zeros((40, 128), dtype=torch.int16, device="cuda")
    y = torch.zeros((40, 64), dtype=torch.float32, device="cuda")
    small = torch.empty(dfc.gemm_workspace_bytes(40, 128) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dfc.DfcError) as ei:
        dfc.decode_gemm(dev, info, x, y, workspace=small)
    assert ei.value.status == dfc.ESIZE
    odd = torch.empty(dfc.gemm_workspace_bytes(40, 128) + 32, dtype=torch.uint8, device="cuda")[8:]
    with pytest.raises(dfc.DfcError) as ei:
        dfc.decode_gemm(dev, info, x, y, workspace=odd)
    assert ei.value.status == dfc.EINVAL
    # batches up to 32 ignore a workspace
    dfc.decode_gemm(dev, info, x[:32], y[:32], workspace=small)
    torch.cuda.synchronize()


def test_status_flag_on_corrupt_block_offsets():
    w = synth.gaussian((64, 2048), 0.02, (89,))
    dev, info, blob = upload(w, panel_k=2048)
    bad = torch.from_numpy(blob.copy()).cuda()
    # second block offset of the first item moved by one
    o = info.off_blockout + 4
    v = int(np.frombuffer(blob[o: o + 4].tobytes(), dtype="<u4")[0])
    bad[o: o + 4] = torch.from_numpy(np.frombuffer(np.uint32(v + 1).tobytes(), dtype=np.uint8).copy())
    x = torch.zeros((1, 2048), dtype=torch.int16, device="cuda")
    y = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode_gemm(bad, info, x, y, status)
    torch.cuda.synchronize()
    assert int(status.item()) == dfc.ECORRUPT


def put_u8(t, offset, values):
    raw = np.asarray(values, dtype=np.uint8)
    t[offset: offset + raw.size] = torch.from_numpy(raw.copy()).cuda()


@pytest.mark.parametrize("case", ["moved", "sum", "huge"])
def test_status_flag_on_wrong_chunk_counts(case):
    """Stored chunk counts (one byte each at C = 16) that the stream
    contradicts: one count moved to the next chunk of the same block (every
    sum still matches, so the container validates and only the kernel's
    per-chunk check can tell), one count raised (the block's sum no longer
    matches its offsets), and a count above what a chunk can hold."""
    w = synth.gaussian((64, 2048), 0.02, (90,))
    dev, info, blob = upload(w, C=16, panel_k=2048)
    bad = torch.from_numpy(blob.copy()).cuda()
    o = info.off_counts + 5
    v0, v1 = (int(v) for v in blob[o: o + 2])
    new = {"moved": [v0 - 1, v1 + 1], "sum": [v0 + 1, v1], "huge": [255, v1]}[case]
    put_u8(bad, o, new)
    if case == "moved":
        assert dfc.blob_info(bad.cpu().numpy()).n == info.n
    say("case wrong chunk counts", case)
    x = torch.zeros((1, 2048), dtype=torch.int16, device="cuda")
    y = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode_gemm(bad, info, x, y, status)
    torch.cuda.synchronize()
    assert int(status.item()) == dfc.ECORRUPT
    # the intact container still decodes cleanly after the failed call
    status.zero_()
    dfc.decode_gemm(dev, info, x, y, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


@pytest.mark.slow
@pytest.mark.parametrize("B", [1, 16, 64])
def test_full_28672x8192(B):
    """The benchmark's matrix: W 28672 x 8192 ~ N(0, 0.015^2), X ~ N(0, 1).
    The product is checked on sampled rows against the oracle; the decode
    is checked exactly on every column with unit vectors (B = 64 only)."""
    w = synth.gemm_weight()
    dev, info, _ = upload(w)
    x = synth.gaussian((B, 8192), 1.0, (4, 1, B))
    say("case full gemm B", B)
    y = run(dev, info, x)
    rows = np.random.default_rng(5).choice(28672, 384, replace=False)
    check_product(w[rows], x, y[:, rows])
    if B == 64:
        wt = torch.from_numpy(w.view(np.int16)).cuda()
        wf = (wt.to(torch.int32) << 16).view(torch.float32)
        xs = torch.zeros((64, 8192), dtype=torch.int16, device="cuda")
        ys = torch.empty((64, 28672), dtype=torch.float32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        for c0 in range(0, 8192, 64):
            xs.zero_()
            xs[torch.arange(64), torch.arange(c0, c0 + 64)] = 0x3F80
            dfc.decode_gemm(dev, info, xs, ys, status)
            assert torch.equal(ys, wf[:, c0: c0 + 64].T.contiguous())
        torch.cuda.synchronize()
        assert int(status.item()) == 0
