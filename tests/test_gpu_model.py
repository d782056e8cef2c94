"""GPU parity at the scale of the whole-model decode (online decompression
of a full weight set, DFloat11 blog, introduction): the 226 matrices of an
8B-shaped model (32 Llama-3-8B-shaped blocks, the 128256 x 4096 embedding
and LM head; 8,029,995,008 weights, about 16 GB of bf16) decoded through
dfc_decode_batch in the benchmark's launch sequence -- model order, calls of
at most 32 matrices, the last one holding the embedding and the LM head --
with every output compared bit for bit with its original on the device, and
sampled blocks of the embedding and of block 0 decoded by the oracle one by
one.  Groups alternate between tables prepared by dfc_derive_tables (as the
benchmark decodes) and tables derived by every workgroup."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth
from oracle import blob as bl
from oracle import fields
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


def oracle_blocks(blob, got, picks):
    """Whole blocks decoded by the oracle's chunk decoder, compared with the
    GPU output at those positions."""
    p = bl.parse_blob(bytes(blob))
    C = p["chunk_bytes"]
    for b in picks:
        b = int(b) % p["n_blocks"]
        c0 = 64 * b
        lo, hi = int(p["out"][b]), int(p["out"][b + 1])
        e = st.decode_chunked(p["words"][c0 * C // 4:], p["off"][c0:], p["total_bits"] - 8 * C * c0, C, 64,
                              p["lengths"])
        assert e.size == hi - lo
        assert np.array_equal(got[lo:hi], fields.merge(e, p["raw"][lo:hi])), b


@pytest.mark.timeout(1200)
def test_whole_model_decode_in_32_item_batches():
    plan = synth.llama3_8b_model_plan()
    assert len(plan) == 226
    groups = [plan[i: i + dfc.MAX_BATCH] for i in range(0, len(plan), dfc.MAX_BATCH)]
    assert [len(g) for g in groups] == [32] * 7 + [2]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    total = 0
    with ThreadPoolExecutor(max_workers=8) as pool:
        for gi, group in enumerate(groups):
            mats = list(pool.map(lambda e: (e[0], synth.model_matrix(e[1], e[2], e[3])), group))
            blobs = list(pool.map(lambda m: dfc.encode(m[1], threads=2), mats))
            infos = [dfc.blob_info(b) for b in blobs]
            devs = [torch.from_numpy(b).cuda() for b in blobs]
            outs = [torch.empty(int(i.n), dtype=torch.int16, device="cuda") for i in infos]
            prepared = gi % 2 == 0
            if prepared:
                tabs = [dfc.derive_tables(d, i) for d, i in zip(devs, infos)]
                items = list(zip(devs, infos, outs, tabs))
            else:
                items = list(zip(devs, infos, outs))
            say(f"group {gi}: {len(items)} matrices, {sum(int(i.n) for i in infos)} weights, "
                f"{'prepared' if prepared else 'derived'} tables")
            status.zero_()
            dfc.decode_batch(items, status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0, gi
            for (name, x), out in zip(mats, outs):
                assert torch.equal(out, torch.from_numpy(x.ravel().view(np.int16)).cuda()), name
                total += x.size
            for (name, x), out, b in zip(mats, outs, blobs):
                if name in ("block0.wq", "block0.down", "embedding"):
                    got = out.cpu().numpy().view(np.uint16)
                    rng = np.random.default_rng(len(name))
                    oracle_blocks(b, got, list(rng.integers(0, 1 << 30, 3)) + [0, -1])
            del mats, blobs, devs, outs, items
            torch.cuda.empty_cache()
    assert total == 8_029_995_008
