"""Decode-just-before-use for layer-by-layer consumers.

The DFloat11 blog's introduction describes weights kept compressed in GPU
memory and decompressed online, just before they are used.  ``DecodeAhead``
does that for a stack of layers: while the caller's stream computes with layer
i, the matrices of layer i + 1 decode on a side stream into the other of two
reused scratch sets, so at most two layers are ever held decompressed.

Ordering uses HIP stream waits and events only: every ``prefetch(i)`` first
makes the side stream wait for the caller's stream as it stands (so a
container written, or memory freed and reused, earlier on the caller's stream
is settled before the decode reads or writes it), ``weights(i)`` makes the
caller's stream wait for layer i's decode, and ``release(i)`` marks the point
after which its scratch set may be overwritten by the decode of layer i + 2.
The calls must come in that order for every layer (prefetch, weights,
release); a prefetch into a set whose layer has not been released, or weights
of a layer that is not in its set, raises instead of racing.  ``close()``
waits for the side stream and drops the scratch sets; the scratch tensors are
also marked as used by the side stream, so the caching allocator does not
hand their memory out while a decode into them is pending.
"""
from __future__ import annotations

from . import MAX_BATCH, Info, decode_batch, derive_tables


class DecodeAhead:
    """Double-buffered decode of ``layers`` (a list, per layer, of
    ``(blob_dev, info, shape)`` with blob_dev a device uint8 tensor holding a
    container in the flat, padded or rANS layout and shape the matrix
    shape).  With ``prepare_tables`` every container's decode tables are
    derived once, on the side stream before its first decode
    (``derive_tables``), and every decode copies them instead of deriving
    them in each workgroup; a container must therefore not change after its
    layer's first prefetch."""

    def __init__(self, layers, device="cuda", prepare_tables: bool = True):
        import torch

        self.torch = torch
        self.layers = [list(layer) for layer in layers]
        for layer in self.layers:
            for _, info, shape in layer:
                if not isinstance(info, Info) or int(info.n) != int(shape[0]) * int(shape[1]):
                    raise ValueError("every matrix needs its container info and a matching 2-D shape")
        width = max((len(layer) for layer in self.layers), default=0)
        sizes = [max((int(layer[j][1].n) for layer in self.layers if j < len(layer)), default=0)
                 for j in range(width)]
        self.scratch = [[torch.empty(max(1, s), dtype=torch.int16, device=device) for s in sizes]
                        for _ in range(2)]
        self.side = torch.cuda.Stream(device=device)  # default priority
        self.ready = [torch.cuda.Event() for _ in range(2)]
        self.free = [torch.cuda.Event() for _ in range(2)]
        self.free_recorded = [False, False]
        self.held = [None, None]  # layer decoded (or decoding) into each set, until released
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.prepare_tables = prepare_tables
        self.tables = [[None] * len(layer) for layer in self.layers]
        for t in [self.status] + [t for s in self.scratch for t in s]:
            t.record_stream(self.side)
        # the scratch and status allocations (and the zero fill) were ordered
        # on the caller's stream
        self.side.wait_stream(torch.cuda.current_stream())

    def prefetch(self, i: int):
        """Enqueue the decode of layer i on the side stream, after everything
        the caller's stream holds so far."""
        if self.scratch is None:
            raise RuntimeError("DecodeAhead is closed")
        slot = i % 2
        if self.held[slot] is not None:
            raise RuntimeError(f"layer {self.held[slot]} still holds scratch set {slot}: release it before "
                               f"prefetching layer {i}")
        self.held[slot] = i
        self.side.wait_stream(self.torch.cuda.current_stream())
        with self.torch.cuda.stream(self.side):
            if self.free_recorded[slot]:
                self.side.wait_event(self.free[slot])
            if self.prepare_tables:
                for j, (blob, info, _) in enumerate(self.layers[i]):
                    if self.tables[i][j] is None:
                        self.tables[i][j] = derive_tables(blob, info, stream=self.side.cuda_stream)
            items = [(blob, info, self.scratch[slot][j][: int(info.n)], self.tables[i][j])
                     for j, (blob, info, _) in enumerate(self.layers[i])]
            for k in range(0, len(items), MAX_BATCH):
                decode_batch(items[k: k + MAX_BATCH], self.status, stream=self.side.cuda_stream)
            self.ready[slot].record(self.side)

    def weights(self, i: int):
        """bf16 views of layer i's matrices; the current stream waits for
        their decode."""
        slot = i % 2
        if self.scratch is None:
            raise RuntimeError("DecodeAhead is closed")
        if self.held[slot] != i:
            raise RuntimeError(f"layer {i} is not in scratch set {slot} (prefetch it first)")
        self.torch.cuda.current_stream().wait_event(self.ready[slot])
        return [self.scratch[slot][j][: int(info.n)].view(self.torch.bfloat16).view(*shape)
                for j, (_, info, shape) in enumerate(self.layers[i])]

    def release(self, i: int):
        """The current stream is done with layer i's matrices."""
        slot = i % 2
        if self.held[slot] != i:
            raise RuntimeError(f"layer {i} is not in scratch set {slot}")
        self.free[slot].record(self.torch.cuda.current_stream())
        self.free_recorded[slot] = True
        self.held[slot] = None

    def close(self):
        """Waits for the side stream's decodes and drops the scratch sets."""
        if self.scratch is not None:
            self.side.synchronize()
            self.scratch = None
            self.tables = None
            self.held = [None, None]

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def corrupt_blocks_seen(self) -> bool:
        """True if any decode so far met a block that failed its check (the
        status word then holds DFC_ECORRUPT; synchronizes the side stream)."""
        self.side.synchronize()
        return int(self.status.item()) != 0
