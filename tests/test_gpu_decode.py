"""GPU parity of the HIP decoder, called through the C ABI.

Every case compares the kernel's output bit for bit (uint16 views) with the
original tensor and, at sizes the oracle decodes in seconds, with the
oracle's own decode of the same container.  Full-size workloads run in the
launch configuration the benchmark times; there the oracle decodes sampled
blocks one by one."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import blob as bl
from oracle import codebook as cb
from oracle import fields
from oracle import stream as st

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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
    dev = torch.from_numpy(np.ascontiguousarray(blob)).cuda()
    out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode(dev, info, out, status)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), int(status.item())


def check(x, C=16, k=12, oracle=True, label=""):
    say("case", label, x.shape, "C", C, "k", k)
    blob = dfc.encode(x, chunk_bytes=C, lut_bits=k)
    got, status = gpu_decode(blob)
    assert status == 0
    assert np.array_equal(got, np.asarray(x).ravel()), label
    if oracle:
        assert np.array_equal(got, bl.decode_blob(bytes(blob))), label
    return blob


@pytest.mark.parametrize("C", [4, 8, 16, 32])
def test_single_matrix_small_all_chunks(C):
    x = synth.gaussian((300, 1000), 0.02, (40, C))   # many blocks, ragged tail
    for k in (8, 10, 11, 12):
        check(x, C, k, label=f"gauss300x1000 C{C}")


def test_mixed_chunk_sizes_in_one_batch():
    """One batch call with matrices of every chunk size and table width:
    one launch per chunk size, items of different widths share a launch."""
    xs = [synth.gaussian_with_outliers((97 + 13 * j, 1024 + 7 * j), 0.02, (53, j)) for j in range(8)]
    cfg = [(4, 11), (8, 12), (16, 11), (32, 10), (16, 8), (8, 11), (4, 12), (32, 11)]
    blobs = [dfc.encode(x, chunk_bytes=C, lut_bits=k) for x, (C, k) in zip(xs, cfg)]
    infos = [dfc.blob_info(b) for b in blobs]
    devs = [torch.from_numpy(b).cuda() for b in blobs]
    outs = [torch.empty(int(i.n), dtype=torch.int16, device="cuda") for i in infos]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("case mixed batch", cfg)
    dfc.decode_batch(list(zip(devs, infos, outs)), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for x, o, b in zip(xs, outs, blobs):
        got = o.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, x.ravel())
        assert np.array_equal(got, bl.decode_blob(bytes(b)))


@pytest.mark.parametrize("run", [0, 3])
def test_items_of_very_different_sizes_share_a_launch(run):
    """32 matrices of one chunk size in one launch, from 1 weight to 33.5 M:
    each gets its share of the resident wavefronts, and with automatic runs
    the large ones are dealt out in runs of 2 blocks while the small ones
    (fewer blocks than 4 per wavefront) go one block per run; run = 3 forces
    runs longer than the small matrices' whole block count."""
    shapes = [(1,), (2,), (7,), (8,), (9,), (63,), (64,), (65,), (511,), (512,), (513,), (1000,), (4097,),
              (6300,), (3, 3151), (64, 1024), (100, 1037), (257, 1031), (512, 4096), (1024, 4096), (333, 7777),
              (1024, 4096), (2048, 4096), (4096, 1024), (4096, 4096), (8192, 4096), (1, 65537), (17, 64),
              (4096, 14336 // 4), (5, 200003), (128, 128), (4095, 4097)]
    assert len(shapes) == 32
    xs = [synth.gaussian_with_outliers(sh, 0.02, (58, j)) for j, sh in enumerate(shapes)]
    blobs = [dfc.encode(x, chunk_bytes=16, lut_bits=11) for x in xs]
    infos = [dfc.blob_info(b) for b in blobs]
    devs = [torch.from_numpy(b).cuda() for b in blobs]
    outs = [torch.full((int(i.n),), 0x7E7E, dtype=torch.int16, device="cuda") for i in infos]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("case 32 sizes in one launch, run", run, "blocks", [int(i.n_blocks) for i in infos])
    dfc.set_launch(0, 0, MODE["stores"], run)
    try:
        dfc.decode_batch(list(zip(devs, infos, outs)), status)
        torch.cuda.synchronize()
    finally:
        dfc.set_launch(0, 0, MODE["stores"])
    assert int(status.item()) == 0
    for x, o, b, info in zip(xs, outs, blobs, infos):
        got = o.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, x.ravel()), x.shape
        if info.n <= 300_000:
            assert np.array_equal(got, bl.decode_blob(bytes(b))), x.shape


@pytest.mark.parametrize("kind", ["outliers", "uniform", "ladder", "bimodal", "t"])
def test_distributions_small(kind):
    shape = (257, 1031)
    x = {"outliers": lambda: synth.gaussian_with_outliers(shape, 0.02, (41,)),
         "uniform": lambda: synth.uniform_bits(shape, (42,)),
         "ladder": lambda: synth.exponent_ladder(shape, (43,)),
         "bimodal": lambda: synth.bimodal(shape, 0.02, (44,)),
         "t": lambda: synth.student_t(shape, 3.0, 0.02, (45,))}[kind]()
    for C in (4, 16, 32):
        check(x, C, label=kind)


def test_edge_sizes():
    for n in (1, 2, 15, 16, 17, 63, 64, 65, 127, 1000, 4097):
        for C in (4, 32):
            check(synth.uniform_bits((n,), (46, n)), C, label=f"n={n}")
            check(synth.gaussian((n,), 0.02, (47, n)), C, label=f"gauss n={n}")


def test_empty_tensor_is_noop():
    blob = dfc.encode(np.zeros(0, dtype=np.uint16))
    info = dfc.blob_info(blob)
    dev = torch.from_numpy(blob).cuda()
    out = torch.empty(0, dtype=torch.int16, device="cuda")
    dfc.decode(dev, info, out)
    torch.cuda.synchronize()


def test_constant_and_special_values():
    check(np.full((100, 100), 0x3F80, dtype=np.uint16), 4, label="constant")
    specials = np.array([0x7FC1, 0xFF81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16)
    x = np.tile(specials, 5000)
    check(x, 8, label="specials")


@pytest.mark.parametrize("C", [16, 32])
def test_one_bit_codes(C):
    """Two equally likely exponents (126, 127): one-bit codes, the most
    values a block can hold (512 C), so the largest staging areas, store
    runs and raw-byte rounds past the prefetched ones."""
    u = synth.uniform_bits((64, 16384), (41, C))
    x = (u & np.uint16(0x807F)) | ((np.uint16(126) + ((u >> np.uint16(7)) & np.uint16(1))) << np.uint16(7))
    blob = check(x, C, k=11, label=f"one-bit codes C={C}")
    assert dfc.blob_info(blob).max_block_elems == 512 * C


def test_long_codes_everywhere():
    """Uniform data under a codebook trained on Gaussian weights: most codes
    are longer than the first-level table (slow path on every lane)."""
    g = synth.gaussian((512, 512), 0.02, (48,))
    h = cb.histogram(fields.split(g)[0]) + 1
    book = dfc.build_codebook(h, 24)
    assert book.max_len == 24 or book.max_len > 12
    x = synth.uniform_bits((200, 999), (49,))
    for C in (4, 16, 32):
        blob = dfc.encode(x, chunk_bytes=C, codebook=book)
        got, status = gpu_decode(blob)
        assert status == 0 and np.array_equal(got, x.ravel())
        assert np.array_equal(got, bl.decode_blob(bytes(blob)))


def test_oracle_written_container_decodes():
    x = synth.gaussian_with_outliers((123, 4567), 0.02, (50,))
    for C in (8, 16):
        blob = np.frombuffer(bl.write_blob(st.encode(x, C, 64), 12, 123, 4567), dtype=np.uint8)
        got, status = gpu_decode(blob)
        assert status == 0 and np.array_equal(got, x.ravel())


# (waves per workgroup, blocks per wavefront, blocks per run): with fixed
# work per workgroup (bpw > 0) and runs of several blocks, each wavefront
# decodes several runs, and its carry and prefetch cross from one to the next.
@pytest.mark.parametrize("waves,bpw,run", [(4, 1, 0), (8, 1, 0), (8, 3, 0), (16, 2, 0), (4, 16, 0), (4, 16, 3),
                                           (8, 3, 2), (4, 16, 16), (1, 8, 5), (2, 64, 64)])
def test_launch_shapes(waves, bpw, run):
    dfc.set_launch(waves, bpw, MODE["stores"], run)
    try:
        x = synth.gaussian((700, 1024), 0.02, (51,))
        check(x, 16, oracle=False, label=f"launch {waves}x{bpw} run {run}")
    finally:
        dfc.set_launch(0, 0, MODE["stores"])


def test_status_flags_count_mismatch():
    x = synth.gaussian((64, 4096), 0.02, (52,))
    blob = dfc.encode(x)
    info = dfc.blob_info(blob)
    bad = blob.copy()
    # the host accepts this (same block count) but the decoded count changes
    import struct
    bad[16:24] = np.frombuffer(struct.pack("<Q", info.total_bits + 3), dtype=np.uint8)
    binfo = dfc.blob_info(bad)
    got, status = gpu_decode(bad, binfo)
    assert status == dfc.ECORRUPT
    # a flipped stream bit either changes a count or changes a value
    flip = blob.copy()
    flip[info.off_words + 1000] ^= 0x10
    got, status = gpu_decode(flip, info)
    assert status == dfc.ECORRUPT or (status == 0 and not np.array_equal(got, x.ravel()))


def test_invalid_arguments_rejected():
    x = synth.gaussian((16, 64), 0.02, (53,))
    blob = dfc.encode(x)
    info = dfc.blob_info(blob)
    dev = torch.from_numpy(blob).cuda()
    out = torch.empty(info.n + 8, dtype=torch.int16, device="cuda")
    lib = dfc.library()
    s = lib.dfc_decode(dev.data_ptr(), info, None, out.data_ptr() + 2, info.n, None, None)   # misaligned dst
    assert s == dfc.EINVAL
    s = lib.dfc_decode(dev.data_ptr(), info, None, out.data_ptr(), info.n + 1, None, None)
    assert s == dfc.ESIZE
    # a block wider than one wavefront is refused at encode time, and a
    # description claiming one is refused before launch
    with pytest.raises(dfc.DfcError):
        dfc.encode(x, lanes=128)
    wide = dfc.blob_info(blob)
    wide.lanes_per_block = 128
    s = lib.dfc_decode(dev.data_ptr(), wide, None, out.data_ptr(), info.n, None, None)
    assert s == dfc.EUNSUPPORTED
    # the binding refuses a device container shorter than its info, a host
    # container and a status word that is not 32-bit, before any launch
    with pytest.raises(ValueError):
        dfc.decode(dev[: info.blob_bytes - 1], info, out[: info.n])
    with pytest.raises(TypeError):
        dfc.decode(torch.from_numpy(blob), info, out[: info.n])
    with pytest.raises(ValueError):
        dfc.decode(dev, info, out[: info.n], torch.zeros(1, dtype=torch.int16, device="cuda"))
    with pytest.raises(ValueError):
        dfc.decode_batch([(dev[:256], info, out[: info.n])])


# ---------------------------------------------------------------- full size

def sampled_oracle_check(blob, got, n_samples=6, seed=0):
    """Decode a few whole blocks with the oracle's chunk decoder and compare
    the GPU output at those positions."""
    p = bl.parse_blob(bytes(blob))
    rng = np.random.default_rng(seed)
    C = p["chunk_bytes"]
    picks = sorted(set(rng.integers(0, p["n_blocks"], size=n_samples).tolist()) | {p["n_blocks"] - 1})
    for b in picks:
        c0 = 64 * b
        lo = p["out"][b]
        hi = p["out"][b + 1]
        # decode chunks of block b by slicing the stream to that block
        words = p["words"][c0 * C // 4:]
        off = p["off"][c0:]
        e = st.decode_chunked(words, off, p["total_bits"] - 8 * C * c0, C, 64, p["lengths"])
        assert e.size == hi - lo
        want = fields.merge(e, p["raw"][lo:hi])
        assert np.array_equal(got[lo:hi], want), b


def test_full_single_matrix_4096():
    x = synth.single_matrix()
    for C in (16, 32):
        say("full 4096x4096 C", C)
        blob = dfc.encode(x, chunk_bytes=C)
        got, status = gpu_decode(blob)
        assert status == 0 and np.array_equal(got, x.ravel())
        sampled_oracle_check(blob, got)


def test_full_llama_block_batched():
    """The benchmark's workload and launch: one Llama-3-8B block, seven
    matrices, one batched launch."""
    mats = list(synth.llama3_8b_block())
    blobs, infos, devs, outs = [], [], [], []
    for name, x in mats:
        say("encode", name, x.shape)
        b = dfc.encode(x)
        blobs.append(b)
        infos.append(dfc.blob_info(b))
        devs.append(torch.from_numpy(b).cuda())
        outs.append(torch.empty(x.size, dtype=torch.int16, device="cuda"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfc.decode_batch(list(zip(devs, infos, outs)), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for (name, x), out, b in zip(mats, outs, blobs):
        got = out.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, x.ravel()), name
        sampled_oracle_check(b, got, n_samples=3)


@pytest.mark.parametrize("kind", list(synth.STRESS_KINDS))
def test_full_stress_8192x28672(kind):
    """The stress tensors at full size, every chunk size (the persistent
    kernel's next-block path runs at every C here: each wavefront decodes
    several blocks), compared on the device; sampled blocks by the oracle."""
    say("stress", kind)
    x = synth.stress(kind)
    ref = torch.from_numpy(x.ravel().view(np.int16)).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for C in (4, 8, 16, 32):
        blob = dfc.encode(x, chunk_bytes=C)
        info = dfc.blob_info(blob)
        assert info.n_blocks > 2 * 8192, (kind, C)   # several blocks per resident wavefront
        dev = torch.from_numpy(blob).cuda()
        out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
        tables = dfc.derive_tables(dev, info) if C in (8, 32) else None
        status.zero_()
        dfc.decode(dev, info, out, status, tables=tables)
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and torch.equal(out, ref), (kind, C)
        if C == 8:
            sampled_oracle_check(blob, out.cpu().numpy().view(np.uint16), n_samples=2)


@pytest.mark.slow
def test_largest_accepted_matrix():
    """The largest matrix the launcher accepts: every stream is addressed
    with 32-bit byte offsets that stay 64 KiB below the top, so n = 777 under
    (2^32 - 16 - 2^16) / 2, i.e. 2,147,450,095 weights and 4.29 GB of bf16
    output, ragged against blocks and octets.  Drawn in independent pieces
    (no period that a wrapped offset could hide behind), decoded in the
    flat, padded and rANS layouts and compared bit for bit on the device.
    One weight more is refused before any launch."""
    import ctypes
    limit = 0xFFFFFFF0 - (1 << 16)
    n = limit // 2 - 777
    say("case largest matrix: generating", n, "weights")
    x = synth.gaussian_pieces(n, 0.02, (150,))
    ref = torch.from_numpy(x.view(np.int16)).cuda()
    lib = dfc.library()
    for layout, kw in ((dfc.LAYOUT_FLAT, {}), (dfc.LAYOUT_PADDED, {}), (dfc.LAYOUT_ANS, {"ans_steps": 512})):
        blob = dfc.encode(x, layout=layout, **kw)
        info = dfc.blob_info(blob)
        dev = torch.from_numpy(blob).cuda()
        del blob
        out = torch.empty(n, dtype=torch.int16, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        say("case largest matrix layout", layout, "container bytes", info.blob_bytes)
        dfc.decode(dev, info, out, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, layout
        assert torch.equal(out, ref), layout
        over = dfc.Info.from_buffer_copy(info)
        over.n = limit // 2 + 1
        s = lib.dfc_decode(ctypes.c_void_p(dev.data_ptr()), ctypes.byref(over), None,
                           ctypes.c_void_p(out.data_ptr()), over.n, None, None)
        assert s == dfc.EUNSUPPORTED, layout
        del dev, out
        torch.cuda.empty_cache()


def test_concurrent_calls_from_host_threads():
    """Four host threads, each with its own stream and its own containers
    (flat, padded, rANS, and a fused product), call the library at the same
    time, repeatedly; every result is exact (the product against unit
    vectors).  Launch set-up (the per-kernel LDS limit, the launch knob) is
    shared process state."""
    import threading
    xs = [synth.gaussian_with_outliers((512, 1024), 0.02, (160, i)) for i in range(3)]
    cfg = [{}, {"layout": dfc.LAYOUT_PADDED}, {"layout": dfc.LAYOUT_ANS, "ans_steps": 64}]
    jobs = []
    for x, kw in zip(xs, cfg):
        b = dfc.encode(x, **kw)
        jobs.append((torch.from_numpy(b).cuda(), dfc.blob_info(b), torch.from_numpy(x.ravel().view(np.int16)).cuda()))
    w = synth.gaussian((256, 512), 0.02, (161,))
    pb = dfc.encode(w, layout=dfc.LAYOUT_PANEL, panel_k=128)
    pinfo = dfc.blob_info(pb)
    pdev = torch.from_numpy(pb).cuda()
    cols = list(range(100, 132))
    xg = np.zeros((len(cols), 512), dtype=np.uint16)
    xg[np.arange(len(cols)), cols] = 0x3F80
    xdev = torch.from_numpy(xg.view(np.int16)).cuda()
    want = torch.from_numpy(((w[:, cols].T.astype(np.uint32) << 16).view(np.float32)).copy()).cuda()
    errors = []
    barrier = threading.Barrier(4)

    def decoder(k):
        try:
            dev, info, ref = jobs[k]
            s = torch.cuda.Stream()
            out = torch.empty(int(info.n), dtype=torch.int16, device="cuda")
            st_ = torch.zeros(1, dtype=torch.int32, device="cuda")
            barrier.wait()
            for _ in range(20):
                with torch.cuda.stream(s):
                    out.fill_(0)
                    dfc.decode(dev, info, out, st_, stream=s.cuda_stream)
                s.synchronize()
                if not torch.equal(out, ref) or int(st_.item()) != 0:
                    errors.append(f"decoder {k}")
                    return
        except Exception as e:  # reported below
            errors.append(f"decoder {k}: {e!r}")

    def product():
        try:
            s = torch.cuda.Stream()
            y = torch.empty((len(cols), 256), dtype=torch.float32, device="cuda")
            barrier.wait()
            for _ in range(20):
                with torch.cuda.stream(s):
                    dfc.decode_gemm(pdev, pinfo, xdev, y, stream=s.cuda_stream)
                s.synchronize()
                if not torch.equal(y, want):
                    errors.append("product")
                    return
        except Exception as e:
            errors.append(f"product: {e!r}")

    say("case concurrent host threads")
    threads = [threading.Thread(target=decoder, args=(k,)) for k in range(3)] + [threading.Thread(target=product)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors


def test_hip_graph_capture_and_replay():
    """The decode and fused-product launches allocate nothing and never
    synchronize, so they can be captured in a HIP graph (torch.cuda.CUDAGraph
    is a HIP graph on ROCm).  The graph is replayed several times with eager
    work and synchronizations in between, and every replay's outputs are
    checked (outputs cleared by a fill kernel before each replay)."""
    xs = [synth.gaussian_with_outliers((384, 1024), 0.02, (170, i)) for i in range(3)]
    cfg = [{}, {"layout": dfc.LAYOUT_PADDED}, {"layout": dfc.LAYOUT_ANS, "ans_steps": 64}]
    items, refs = [], []
    for x, kw in zip(xs, cfg):
        b = dfc.encode(x, **kw)
        info = dfc.blob_info(b)
        items.append((torch.from_numpy(b).cuda(), info, torch.empty(int(info.n), dtype=torch.int16, device="cuda")))
        refs.append(torch.from_numpy(x.ravel().view(np.int16)).cuda())
    w = synth.gaussian((256, 512), 0.02, (171,))
    pb = dfc.encode(w, layout=dfc.LAYOUT_PANEL, panel_k=128)
    pinfo, pdev = dfc.blob_info(pb), torch.from_numpy(pb).cuda()
    cols = list(range(7, 39))
    xg = np.zeros((len(cols), 512), dtype=np.uint16)
    xg[np.arange(len(cols)), cols] = 0x3F80
    xdev = torch.from_numpy(xg.view(np.int16)).cuda()
    y = torch.empty((len(cols), 256), dtype=torch.float32, device="cuda")
    want = torch.from_numpy(((w[:, cols].T.astype(np.uint32) << 16).view(np.float32)).copy()).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):   # eager warm-up: one-time launch set-up happens outside the capture
        dfc.decode_batch(items, status, stream=s.cuda_stream)
        dfc.decode_gemm(pdev, pinfo, xdev, y, status, stream=s.cuda_stream)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _, _, out in items:
            out.fill_(0)
        y.fill_(0)
        dfc.decode_batch(items, status, stream=torch.cuda.current_stream().cuda_stream)
        dfc.decode_gemm(pdev, pinfo, xdev, y, status, stream=torch.cuda.current_stream().cuda_stream)
    say("case hip graph replays")
    for rep in range(4):
        for _, _, out in items:
            out.fill_(-1)        # eager work between replays
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, rep
        for (_, _, out), ref in zip(items, refs):
            assert torch.equal(out, ref), rep
        assert torch.equal(y, want), rep


@pytest.mark.parametrize("layout", [dfc.LAYOUT_FLAT, dfc.LAYOUT_PADDED])
@pytest.mark.parametrize("waves,bpw,run", [(0, 0, 0), (1, 8, 0), (4, 2, 0), (4, 4, 2), (2, 8, 3)])
def test_corrupt_block_leaves_the_rest_exact(layout, waves, bpw, run):
    """A block offset moved by one makes the two blocks around it fail their
    count check: those two blocks stay unwritten, the status word is set,
    and every other block -- before them in the same run of blocks, and
    after them -- is still decoded exactly."""
    import struct
    x = synth.gaussian((256, 4096), 0.02, (54, layout))
    blob = dfc.encode(x, layout=layout)
    info = dfc.blob_info(blob)
    assert info.n_blocks > 40
    bad = blob.copy()
    b = info.n_blocks // 2 + 1
    o = info.off_blockout + 4 * b
    ob = struct.unpack_from("<III", bytes(blob[o - 4: o + 8]))
    bad[o: o + 4] = np.frombuffer(struct.pack("<I", ob[1] + 1), dtype=np.uint8)
    binfo = dfc.blob_info(bad)
    dfc.set_launch(waves, bpw, MODE["stores"], run)
    try:
        dev = torch.from_numpy(bad).cuda()
        out = torch.full((int(info.n),), 0x7E7E, dtype=torch.int16, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        dfc.decode(dev, binfo, out, status)
        torch.cuda.synchronize()
    finally:
        dfc.set_launch(0, 0, MODE["stores"])
    got = out.cpu().numpy().view(np.uint16)
    assert int(status.item()) == dfc.ECORRUPT
    lo, hi = ob[0], ob[2]   # blocks b - 1 and b
    assert np.array_equal(got[:lo], x.ravel()[:lo])
    assert np.array_equal(got[hi:], x.ravel()[hi:])
    assert (got[lo:hi] == 0x7E7E).all()
