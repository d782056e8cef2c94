"""GPU checks of decode-just-before-use (DecodeAhead): every layer's weights,
decoded on the side stream into the reused scratch sets, equal the originals
bit for bit at the moment the compute stream uses them, and a chained
computation over the layers matches the one with resident weights exactly."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_dfc_amd as dfc
from lossless_entropy_coded_dfc_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def make_layers(n_layers, shapes, C=16):
    layers, originals = [], []
    for i in range(n_layers):
        layer, orig = [], []
        for j, (r, c) in enumerate(shapes):
            x = synth.gaussian_with_outliers((r, c), 0.02, (90, i, j))
            blob = dfc.encode(x, chunk_bytes=C)
            layer.append((torch.from_numpy(blob).cuda(), dfc.blob_info(blob), (r, c)))
            orig.append(x)
        layers.append(layer)
        originals.append(orig)
    return layers, originals


@pytest.mark.parametrize("prepare", [True, False])
def test_weights_equal_originals_when_used(prepare):
    """Tables prepared once per container on the side stream, or derived by
    every decoding workgroup: the same weights either way."""
    from lossless_entropy_coded_dfc_amd.ahead import DecodeAhead
    shapes = [(256, 512), (512, 256), (128, 512)]
    layers, originals = make_layers(5, shapes)
    dec = DecodeAhead(layers, prepare_tables=prepare)
    say("case decode-ahead 5 layers, prepared tables" if prepare else "case decode-ahead 5 layers, derived tables")
    dec.prefetch(0)
    for i in range(5):
        if i + 1 < 5:
            dec.prefetch(i + 1)
        W = dec.weights(i)
        # copies taken on the compute stream, before release
        got = [w.view(torch.int16).clone() for w in W]
        dec.release(i)
        for g, x in zip(got, originals[i]):
            assert torch.equal(g, torch.from_numpy(x.view(np.int16)).cuda())
    assert not dec.corrupt_blocks_seen()


def test_chained_products_match_resident_weights():
    from lossless_entropy_coded_dfc_amd.ahead import DecodeAhead
    d = 256
    shapes = [(d, d), (d, d)]
    layers, originals = make_layers(6, shapes, C=8)
    resident = [[torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for x in orig] for orig in originals]
    h0 = torch.from_numpy(synth.gaussian((64, d), 1.0, (91,)).view(np.int16)).cuda().view(torch.bfloat16)

    def step(h, W):
        h = (h @ W[0].t()) @ W[1].t()
        return (h.float() / (h.float().abs().amax() + 1e-6)).to(torch.bfloat16)

    h = h0
    for W in resident:
        h = step(h, W)
    dec = DecodeAhead(layers)
    g = h0
    dec.prefetch(0)
    for i in range(6):
        if i + 1 < 6:
            dec.prefetch(i + 1)
        g = step(g, dec.weights(i))
        dec.release(i)
    torch.cuda.synchronize()
    say("case decode-ahead chained products")
    assert torch.equal(g, h)
    assert not dec.corrupt_blocks_seen()


def test_out_of_order_use_raises():
    """Prefetching into a scratch set whose layer is still held, asking for
    weights of a layer not in its set, or releasing one twice raises before
    any decode is enqueued."""
    from lossless_entropy_coded_dfc_amd.ahead import DecodeAhead
    layers, originals = make_layers(4, [(64, 256)])
    dec = DecodeAhead(layers)
    dec.prefetch(0)
    dec.prefetch(1)
    with pytest.raises(RuntimeError):
        dec.prefetch(2)          # layer 0 still holds set 0
    with pytest.raises(RuntimeError):
        dec.weights(2)           # never prefetched
    w0 = dec.weights(0)[0].view(torch.int16).clone()
    dec.release(0)
    with pytest.raises(RuntimeError):
        dec.release(0)           # already released
    dec.prefetch(2)              # set 0 is free again
    w2 = dec.weights(2)[0].view(torch.int16).clone()
    dec.release(1)
    dec.release(2)
    assert torch.equal(w0, torch.from_numpy(originals[0][0].view(np.int16)).cuda())
    assert torch.equal(w2, torch.from_numpy(originals[2][0].view(np.int16)).cuda())
    assert not dec.corrupt_blocks_seen()


def test_prefetch_waits_for_the_callers_stream():
    """A container written on the caller's stream right before prefetch (the
    copy queued behind a few large products) is what the side stream
    decodes: prefetch orders the side stream after the caller's work."""
    from lossless_entropy_coded_dfc_amd.ahead import DecodeAhead
    x = synth.gaussian_with_outliers((512, 1024), 0.02, (92,))
    blob = dfc.encode(x, chunk_bytes=16)
    info = dfc.blob_info(blob)
    host = torch.from_numpy(blob).pin_memory()
    dev = torch.zeros(host.numel(), dtype=torch.uint8, device="cuda")
    with DecodeAhead([[(dev, info, (512, 1024))]]) as dec:
        a = torch.ones((4096, 4096), dtype=torch.bfloat16, device="cuda")
        for _ in range(8):
            a = (a @ a) * (1.0 / 4096)
        dev.copy_(host, non_blocking=True)
        say("case decode-ahead after a producer on the caller's stream")
        dec.prefetch(0)
        got = dec.weights(0)[0].view(torch.int16).clone()
        dec.release(0)
        assert torch.equal(got, torch.from_numpy(x.view(np.int16)).cuda())
        assert not dec.corrupt_blocks_seen()
    with pytest.raises(RuntimeError):
        dec.prefetch(0)          # closed
