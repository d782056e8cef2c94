"""Python binding of libdfc: lossless exponent-Huffman compression of bf16
weights with a gfx950 (MI355X) GPU decoder.

This module only marshals arguments into the C ABI declared in
``include/dfc.h``: every step of encoding runs in the host library and every
step of decoding runs in its HIP kernels.  torch supplies device memory
(``data_ptr()``) and the current HIP stream.  If ``libdfc.so`` has not been
built, every entry point raises ``DfcLibraryMissing``; there is no fallback.

Importing the package does not load the library; ``synth`` (seeded input
generators) is usable without it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "DfcError", "DfcLibraryMissing", "Params", "Codebook", "Info", "BatchItem",
    "library", "library_path", "default_params", "histogram", "build_codebook",
    "encode_bound", "encode", "blob_info", "decode", "decode_batch", "set_launch",
    "STORES_AUTO", "STORES_DEFERRED", "STORES_IMMEDIATE",
    "status_str", "MAX_BATCH", "derived_tables_bytes", "derive_tables",
]

MAX_BATCH = 32
LAYOUT_FLAT = 0
LAYOUT_PANEL = 1
LAYOUT_PADDED = 2
LAYOUT_ANS = 3
PANEL_ROWS = 32
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdfc.so")
_LIB = None

OK, EINVAL, ESIZE, ECORRUPT, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5


class DfcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class DfcLibraryMissing(ImportError):
    pass


class Params(ctypes.Structure):
    _fields_ = [("chunk_bytes", ctypes.c_uint32), ("lanes_per_block", ctypes.c_uint32),
                ("max_code_len", ctypes.c_uint32), ("lut_bits", ctypes.c_uint32),
                ("layout", ctypes.c_uint32), ("threads", ctypes.c_uint32),
                ("panel_k", ctypes.c_uint32), ("ans_steps", ctypes.c_uint32),
                ("rows", ctypes.c_uint64), ("cols", ctypes.c_uint64)]


class Codebook(ctypes.Structure):
    _fields_ = [("len", ctypes.c_uint8 * 256), ("code", ctypes.c_uint32 * 256),
                ("n_used", ctypes.c_uint32), ("min_len", ctypes.c_uint32), ("max_len", ctypes.c_uint32)]

    @property
    def lengths(self) -> np.ndarray:
        return np.frombuffer(bytes(self.len), dtype=np.uint8).copy()

    @property
    def codes(self) -> np.ndarray:
        return np.array(list(self.code), dtype=np.uint32)


class Info(ctypes.Structure):
    _fields_ = [(name, ctypes.c_uint64) for name in (
        "n", "rows", "cols", "blob_bytes", "coded_bytes", "total_bits", "n_chunks", "n_blocks",
        "off_tables", "tables_bytes", "off_words", "words_bytes", "off_offsets", "offsets_bytes",
        "off_blockout", "blockout_bytes", "off_raw", "raw_bytes")] + \
        [(name, ctypes.c_uint32) for name in (
            "chunk_bytes", "lanes_per_block", "max_code_len", "lut_bits", "layout",
            "n_used", "min_len", "max_len", "max_block_elems", "panel_rows", "panel_k")] + \
        [(name, ctypes.c_uint64) for name in ("n_items", "off_panels", "panels_bytes")] + \
        [(name, ctypes.c_uint32) for name in ("ans_steps", "ans_prob_bits")] + \
        [(name, ctypes.c_uint64) for name in ("off_counts", "counts_bytes")]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class BatchItem(ctypes.Structure):
    _fields_ = [("blob_dev", ctypes.c_void_p), ("info", ctypes.POINTER(Info)),
                ("dst_dev", ctypes.c_void_p), ("n", ctypes.c_uint64), ("tables_dev", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libdfc.so (once).  Raises DfcLibraryMissing if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise DfcLibraryMissing(
            f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python -m lossless_entropy_coded_dfc_amd.csrc.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    st = ctypes.c_int
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.dfc_default_params.argtypes = [ctypes.POINTER(Params)]
    lib.dfc_default_params.restype = None
    lib.dfc_histogram.argtypes = [ctypes.c_void_p, ctypes.c_uint64, u64p]
    lib.dfc_histogram.restype = st
    lib.dfc_build_codebook.argtypes = [u64p, ctypes.c_uint32, ctypes.POINTER(Codebook)]
    lib.dfc_build_codebook.restype = st
    lib.dfc_encode_bound.argtypes = [ctypes.c_uint64, ctypes.POINTER(Params), u64p]
    lib.dfc_encode_bound.restype = st
    lib.dfc_encode.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(Params),
                               ctypes.POINTER(Codebook), ctypes.c_void_p, ctypes.c_uint64, u64p]
    lib.dfc_encode.restype = st
    lib.dfc_blob_info.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(Info)]
    lib.dfc_blob_info.restype = st
    lib.dfc_decode.argtypes = [ctypes.c_void_p, ctypes.POINTER(Info), ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.dfc_decode.restype = st
    lib.dfc_decode_batch.argtypes = [ctypes.POINTER(BatchItem), ctypes.c_uint32, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.dfc_decode_batch.restype = st
    lib.dfc_decode_gemm.argtypes = [ctypes.c_void_p, ctypes.POINTER(Info), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.dfc_decode_gemm.restype = st
    lib.dfc_gemm_workspace_bytes.argtypes = [ctypes.c_uint32, ctypes.c_uint64]
    lib.dfc_gemm_workspace_bytes.restype = ctypes.c_uint64
    lib.dfc_encode_device_workspace.argtypes = [ctypes.c_uint64, u64p]
    lib.dfc_encode_device_workspace.restype = st
    lib.dfc_histogram_device.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.dfc_histogram_device.restype = st
    lib.dfc_encode_device.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(Params),
                                      ctypes.POINTER(Codebook), ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_uint64, u64p, ctypes.c_void_p]
    lib.dfc_encode_device.restype = st
    lib.dfc_encode_device_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(Params),
                                              ctypes.POINTER(Codebook), ctypes.c_void_p, ctypes.c_uint64, u64p,
                                              ctypes.c_void_p]
    lib.dfc_encode_device_noalloc.restype = st
    lib.dfc_derived_tables_bytes.argtypes = [ctypes.POINTER(Info), u64p]
    lib.dfc_derived_tables_bytes.restype = st
    lib.dfc_derive_tables.argtypes = [ctypes.c_void_p, ctypes.POINTER(Info), ctypes.c_uint32, ctypes.c_void_p,
                                      ctypes.c_uint64, ctypes.c_void_p]
    lib.dfc_derive_tables.restype = st
    lib.dfc_set_launch.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    lib.dfc_set_launch.restype = st
    lib.dfc_status_str.argtypes = [ctypes.c_int]
    lib.dfc_status_str.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_str(status: int) -> str:
    try:
        return library().dfc_status_str(int(status)).decode()
    except DfcLibraryMissing:
        return "libdfc not built"


def _check(status: int, where: str):
    if status != OK:
        raise DfcError(status, where)


def _u16(bits) -> np.ndarray:
    a = np.asarray(bits)
    if a.dtype != np.uint16:
        if a.dtype.itemsize != 2:
            raise TypeError("expected 16-bit bf16 bit patterns")
        a = a.view(np.uint16)
    return np.ascontiguousarray(a).ravel()


# ------------------------------------------------------------------ host

def default_params(**overrides) -> Params:
    p = Params()
    library().dfc_default_params(ctypes.byref(p))
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


def histogram(bits) -> np.ndarray:
    src = _u16(bits)
    h = np.zeros(256, dtype=np.uint64)
    _check(library().dfc_histogram(src.ctypes.data_as(ctypes.c_void_p), src.size,
                                   h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))), "dfc_histogram")
    return h


def build_codebook(hist, max_code_len: int = 24) -> Codebook:
    h = np.ascontiguousarray(np.asarray(hist, dtype=np.uint64))
    if h.shape != (256,):
        raise ValueError("histogram must have 256 bins")
    cb = Codebook()
    _check(library().dfc_build_codebook(h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), max_code_len,
                                        ctypes.byref(cb)), "dfc_build_codebook")
    return cb


def encode_bound(n: int, params: Params | None = None) -> int:
    out = ctypes.c_uint64()
    _check(library().dfc_encode_bound(n, ctypes.byref(params) if params else None, ctypes.byref(out)),
           "dfc_encode_bound")
    return out.value


def encode(bits, chunk_bytes: int = 0, lanes: int = 64, max_code_len: int = 24, lut_bits: int = 11,
           codebook: Codebook | None = None, threads: int = 0, shape=None, layout: int = LAYOUT_FLAT,
           panel_k: int = 0, ans_steps: int = 0) -> np.ndarray:
    """Encode bf16 bit patterns (any shape, row-major) into a DFC1 container
    (numpy uint8 array).  ``layout=LAYOUT_PANEL`` writes the order the fused
    decode + GEMM consumes (2-D input, rows % 32 == 0, cols % 16 == 0);
    ``layout=LAYOUT_PADDED`` keeps codes inside their chunks and drops the
    chunk offsets; ``layout=LAYOUT_ANS`` codes the exponents with interleaved
    rANS (``ans_steps`` steps of 64 elements per block, 0 = 512)."""
    arr = np.asarray(bits)
    src = _u16(arr)
    if shape is None:
        shape = arr.shape if arr.ndim == 2 else (1, src.size)
    p = default_params(chunk_bytes=chunk_bytes, lanes_per_block=lanes, max_code_len=max_code_len,
                       lut_bits=lut_bits, threads=threads, rows=int(shape[0]), cols=int(shape[1]),
                       layout=layout, panel_k=panel_k, ans_steps=ans_steps)
    if src.size == 0:
        p.rows, p.cols = 0, 0
    cap = encode_bound(src.size, p)
    dst = np.empty(cap, dtype=np.uint8)
    written = ctypes.c_uint64()
    _check(library().dfc_encode(src.ctypes.data_as(ctypes.c_void_p), src.size, ctypes.byref(p),
                                ctypes.byref(codebook) if codebook is not None else None,
                                dst.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(written)),
           "dfc_encode")
    return dst[: written.value]


def blob_info(blob) -> Info:
    b = np.ascontiguousarray(np.frombuffer(blob, dtype=np.uint8) if isinstance(blob, (bytes, bytearray))
                             else np.asarray(blob, dtype=np.uint8))
    info = Info()
    _check(library().dfc_blob_info(b.ctypes.data_as(ctypes.c_void_p), b.size, ctypes.byref(info)),
           "dfc_blob_info")
    return info


# ---------------------------------------------------------------- device

def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_ptr(t) -> int:
    if t is None:
        return 0
    if not getattr(t, "is_cuda", False):
        raise TypeError("expected a device (cuda) tensor")
    return t.data_ptr()


def _blob_ptr(blob_dev, info: Info) -> int:
    """Device address of a container tensor that holds info.blob_bytes:
    the kernels read the sections at the offsets the info records, so a
    shorter buffer would be read past its end."""
    if not getattr(blob_dev, "is_cuda", False) or not blob_dev.is_contiguous():
        raise TypeError("the container must be a contiguous device (cuda) tensor")
    if blob_dev.numel() * blob_dev.element_size() < info.blob_bytes:
        raise ValueError(f"the device container holds {blob_dev.numel() * blob_dev.element_size()} bytes, "
                         f"fewer than the {info.blob_bytes} its info describes")
    return blob_dev.data_ptr()


def _status_ptr(status) -> int:
    if status is None:
        return 0
    if status.element_size() != 4 or status.numel() < 1:
        raise ValueError("status must be a device tensor of at least one 32-bit element")
    return _dev_ptr(status)


def _tables_ptr(tables, info: Info) -> int:
    """Device address of prepared decode tables (from ``derive_tables``), or 0."""
    if tables is None:
        return 0
    if not getattr(tables, "is_cuda", False) or not tables.is_contiguous():
        raise TypeError("tables must be a contiguous device tensor from derive_tables")
    if tables.numel() * tables.element_size() < derived_tables_bytes(info):
        raise ValueError("tables are shorter than the container's decode tables")
    return tables.data_ptr()


def decode(blob_dev, info: Info, out, status=None, stream=None, tables=None):
    """Decode a container held in device memory (torch uint8 tensor) into
    ``out`` (torch tensor of info.n 16-bit elements).  ``tables``: the
    container's decode tables from ``derive_tables`` (else every workgroup
    derives them).  Asynchronous."""
    if not out.is_contiguous() or out.element_size() != 2 or out.numel() != info.n:
        raise ValueError("out must be a contiguous 16-bit tensor with info.n elements")
    _check(library().dfc_decode(ctypes.c_void_p(_blob_ptr(blob_dev, info)), ctypes.byref(info),
                                ctypes.c_void_p(_tables_ptr(tables, info)), ctypes.c_void_p(_dev_ptr(out)), info.n,
                                ctypes.c_void_p(_status_ptr(status)), _stream(stream)), "dfc_decode")
    return out


def decode_batch(items, status=None, stream=None):
    """Decode up to MAX_BATCH (blob_dev, info, out) or (blob_dev, info, out,
    tables) tuples with one launch."""
    items = list(items)
    if len(items) > MAX_BATCH:
        raise ValueError(f"at most {MAX_BATCH} items per batch")
    arr = (BatchItem * max(1, len(items)))()
    keep = []
    for k, item in enumerate(items):
        blob_dev, info, out = item[:3]
        tables = item[3] if len(item) > 3 else None
        if not out.is_contiguous() or out.element_size() != 2 or out.numel() != info.n:
            raise ValueError("out must be a contiguous 16-bit tensor with info.n elements")
        keep.append(info)
        arr[k].blob_dev = _blob_ptr(blob_dev, info)
        arr[k].info = ctypes.pointer(info)
        arr[k].dst_dev = _dev_ptr(out)
        arr[k].n = info.n
        arr[k].tables_dev = _tables_ptr(tables, info)
    _check(library().dfc_decode_batch(arr, len(items), ctypes.c_void_p(_status_ptr(status)), _stream(stream)),
           "dfc_decode_batch")


def encode_device(src, chunk_bytes: int = 0, lanes: int = 64, max_code_len: int = 24, lut_bits: int = 11,
                  codebook: Codebook | None = None, shape=None, stream=None, layout: int = LAYOUT_FLAT,
                  ans_steps: int = 0, panel_k: int = 0):
    """Encode a contiguous 16-bit device tensor (bf16 bits) on the GPU, in the
    flat, panel or rANS layout.  Returns (container as a device uint8 tensor,
    its size in bytes); the container is byte-identical to ``encode``'s."""
    import torch
    n = src.numel()
    if src.element_size() != 2 or not src.is_contiguous():
        raise ValueError("src must be a contiguous 16-bit device tensor")
    if shape is None:
        shape = tuple(src.shape) if src.dim() == 2 else (1, n)
    p = default_params(chunk_bytes=chunk_bytes, lanes_per_block=lanes, max_code_len=max_code_len,
                       lut_bits=lut_bits, rows=int(shape[0]), cols=int(shape[1]), layout=layout,
                       ans_steps=ans_steps, panel_k=panel_k)
    if n == 0:
        p.rows, p.cols = 0, 0
    cap = encode_bound(n, p)
    wb = ctypes.c_uint64()
    _check(library().dfc_encode_device_workspace(n, ctypes.byref(wb)), "dfc_encode_device_workspace")
    dst = torch.empty(cap, dtype=torch.uint8, device=src.device)
    work = torch.empty(max(256, wb.value), dtype=torch.uint8, device=src.device)
    written = ctypes.c_uint64()
    _check(library().dfc_encode_device(ctypes.c_void_p(src.data_ptr() if n else 0), n, ctypes.byref(p),
                                       ctypes.byref(codebook) if codebook is not None else None,
                                       ctypes.c_void_p(dst.data_ptr()), cap, ctypes.c_void_p(work.data_ptr()),
                                       wb.value, ctypes.byref(written), _stream(stream)), "dfc_encode_device")
    if stream is not None:
        # the packing kernels may still run on that stream: keep torch's
        # allocator from handing the workspace to other streams' work first
        work.record_stream(torch.cuda.ExternalStream(int(stream), device=src.device))
    return dst, written.value


GEMM_MAX_BATCH = 64


def gemm_workspace_bytes(batch: int, cols: int) -> int:
    """Device bytes of the workspace decode_gemm uses for B vectors of K values
    (0 for B <= 32)."""
    return int(library().dfc_gemm_workspace_bytes(batch, cols))


def decode_gemm(blob_dev, info: Info, x, y, status=None, stream=None, tables=None, workspace=None):
    """Fused decode + product: y[b, :] = W @ x[b, :] for a panel-layout
    container of W (M x K).  x: contiguous 16-bit device tensor of shape
    (B, K) (bf16 bits); y: contiguous float32 device tensor of shape (B, M);
    tables: as in ``decode``; workspace: None or a device uint8 tensor of at
    least gemm_workspace_bytes(B, K) bytes that nothing else uses until the
    call's work has run (for B > 32 one is allocated on the device of x when
    none is given; pass False to read X in place)."""
    if info.layout != LAYOUT_PANEL:
        raise ValueError("decode_gemm needs a panel-layout container")
    if x.dim() != 2 or y.dim() != 2 or not x.is_contiguous() or not y.is_contiguous():
        raise ValueError("x and y must be contiguous 2-D tensors")
    B, K = x.shape
    import torch
    if x.element_size() != 2 or K != info.cols or tuple(y.shape) != (B, info.rows) or y.dtype != torch.float32:
        raise ValueError("x must be (B, K) 16-bit and y (B, M) float32 for the container's M x K")
    need = gemm_workspace_bytes(B, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        if stream is not None:
            # the caching allocator must not hand this memory out before the
            # call's work on that stream has run
            workspace.record_stream(torch.cuda.ExternalStream(int(stream), device=x.device))
    if workspace is False or workspace is None:
        ws_ptr, ws_bytes = 0, 0
    else:
        ws_ptr, ws_bytes = _dev_ptr(workspace), workspace.numel() * workspace.element_size()
    _check(library().dfc_decode_gemm(ctypes.c_void_p(_blob_ptr(blob_dev, info)), ctypes.byref(info),
                                     ctypes.c_void_p(_tables_ptr(tables, info)), ctypes.c_void_p(_dev_ptr(x)), B,
                                     ctypes.c_void_p(_dev_ptr(y)), ctypes.c_void_p(ws_ptr), ws_bytes,
                                     ctypes.c_void_p(_status_ptr(status)), _stream(stream)), "dfc_decode_gemm")


def derived_tables_bytes(info: Info) -> int:
    out = ctypes.c_uint64()
    _check(library().dfc_derived_tables_bytes(ctypes.byref(info), ctypes.byref(out)), "dfc_derived_tables_bytes")
    return out.value


def derive_tables(blob_dev, info: Info, threads: int = 0, stream=None):
    """The decode tables of a container, derived from its code on the GPU by
    one workgroup of ``threads`` threads (0 = 1024) exactly as a decoding
    workgroup builds them in LDS: a device uint8 tensor (the byte layout is
    the library's own) to pass as ``tables`` to the decoders.  Asynchronous."""
    import torch
    nbytes = derived_tables_bytes(info)
    out = torch.empty(nbytes, dtype=torch.uint8, device=blob_dev.device)
    _check(library().dfc_derive_tables(ctypes.c_void_p(_blob_ptr(blob_dev, info)), ctypes.byref(info), threads,
                                       ctypes.c_void_p(out.data_ptr()), nbytes, _stream(stream)), "dfc_derive_tables")
    return out


STORES_AUTO, STORES_DEFERRED, STORES_IMMEDIATE = 0, 1, 2


def set_launch(waves_per_group: int = 0, blocks_per_wave: int = 0, stores: int = STORES_AUTO, run_blocks: int = 0):
    """dfc_set_launch: the Huffman decoder's process-wide launch shape
    (wavefronts per workgroup, blocks per wavefront, store build, blocks per
    run; 0 = automatic for each).  Changes launch shapes, never results."""
    _check(library().dfc_set_launch(waves_per_group, blocks_per_wave, stores, run_blocks), "dfc_set_launch")
