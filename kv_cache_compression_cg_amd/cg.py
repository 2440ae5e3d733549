"""Python binding of libcg (include/cg.h): argument marshalling only.

Every step of the codec runs in the library's HIP kernels; this module checks tensor
shapes, passes device pointers and the current HIP stream, and wraps the handles.
Torch tensors provide device memory and streams.  If libcg.so is not built the import
fails: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

from .build import LIB

CG_OK = 0
ERRORS = {-1: "CG_E_INVAL", -2: "CG_E_NOMEM", -3: "CG_E_HIP", -4: "CG_E_NONFINITE",
          -5: "CG_E_CORRUPT"}
MAX_BINS = 32
LANES = 64


class CgError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


class Params(ctypes.Structure):
    _fields_ = [("L", ctypes.c_uint32), ("H_kv", ctypes.c_uint32), ("d", ctypes.c_uint32),
                ("S", ctypes.c_uint32), ("group", ctypes.c_uint32), ("chunk", ctypes.c_uint32),
                ("bins", ctypes.POINTER(ctypes.c_uint8)), ("bins_v", ctypes.POINTER(ctypes.c_uint8)),
                ("n_sink", ctypes.c_uint32), ("anchor_bits", ctypes.c_uint32),
                ("outlier_ppm", ctypes.c_uint32)]


class ContainerHeader(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("magic", "version", "L", "H_kv", "d", "S", "group", "chunk", "chunk_begin",
                 "chunk_end", "n_blocks", "anchor_bits", "n_sink", "outlier_ppm")] + \
               [(n, ctypes.c_uint64) for n in
                ("n_groups", "offsets_offset", "anchors_offset", "anchors_bytes", "sinks_offset",
                 "outliers_offset", "outlier_keys_offset", "outlier_values_offset",
                 "n_outliers", "clamped", "payload_offset", "payload_words", "total_bytes")]


class TablesHeader(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("magic", "version", "L", "H_kv", "d", "S", "group", "chunk", "n_sink",
                 "anchor_bits", "outlier_ppm", "reserved")] + [("total_bytes", ctypes.c_uint64)]


class BlobInfo(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("header", ContainerHeader)]


class TablesInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in ("L", "H_kv", "d", "S", "group", "chunk")] + \
               [("stored_bytes", ctypes.c_uint64)]


class StreamItem(ctypes.Structure):
    _fields_ = [("tables", ctypes.c_void_p), ("blob", ctypes.c_void_p),
                ("host_container", ctypes.c_void_p)]


class StreamStats(ctypes.Structure):
    _fields_ = [("total_ms", ctypes.c_float), ("copy_ms", ctypes.c_float),
                ("decode_ms", ctypes.c_float), ("copied_bytes", ctypes.c_uint64)]


EXPORTED = ["cg_build_cdf", "cg_encode", "cg_decode", "cg_free", "cg_last_error",
            "cg_tables_export", "cg_tables_get_info", "cg_blob_get_info", "cg_blob_read",
            "cg_quantize", "cg_decode_symbols", "cg_dequantize", "cg_stream_decode",
            "cg_decode_paged", "cg_tables_serialize", "cg_tables_check", "cg_tables_import",
            "cg_container_check", "cg_blob_import", "cg_encode_noalloc"]

_lib = None


def load() -> ctypes.CDLL:
    """Loads the in-tree libcg.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise ImportError("libcg.so is not built (%s); run `python -m "
                          "kv_cache_compression_cg_amd.build`" % LIB)
    L = ctypes.CDLL(LIB)
    vp, u32, u64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "cg_build_cdf": [ctypes.POINTER(Params), vp, vp, pp],
        "cg_encode": [vp, vp, u32, u32, vp, pp],
        "cg_decode": [vp, vp, vp, vp, vp],
        "cg_decode_paged": [vp, vp, vp, vp, vp, u32, u32, vp],
        "cg_tables_export": [vp, vp, vp, vp, vp],
        "cg_tables_get_info": [vp, ctypes.POINTER(TablesInfo)],
        "cg_blob_get_info": [vp, ctypes.POINTER(BlobInfo)],
        "cg_blob_read": [vp, u64, u64, vp],
        "cg_quantize": [vp, vp, u32, u32, vp, vp],
        "cg_decode_symbols": [vp, vp, vp, vp, vp],
        "cg_dequantize": [vp, vp, vp, vp, vp, vp],
        "cg_stream_decode": [ctypes.POINTER(StreamItem), u32, vp, u64, u32, vp, vp, vp,
                             ctypes.POINTER(StreamStats)],
        "cg_tables_serialize": [vp, vp, u64, ctypes.POINTER(ctypes.c_uint64)],
        "cg_tables_check": [vp, u64, ctypes.POINTER(TablesHeader)],
        "cg_tables_import": [vp, u64, pp],
        "cg_container_check": [vp, u64, ctypes.POINTER(ContainerHeader)],
        "cg_blob_import": [vp, vp, u64, vp, pp],
        "cg_encode_noalloc": [vp, vp, u32, u32, vp, u64, vp, ctypes.POINTER(ContainerHeader)],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.cg_free.argtypes = [vp]
    L.cg_free.restype = None
    L.cg_last_error.argtypes = []
    L.cg_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != CG_OK:
        raise CgError(rc, load().cg_last_error().decode(errors="replace"))


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _kv_check(kv: torch.Tensor, shape=None) -> None:
    if not kv.is_cuda or kv.dtype != torch.float16 or not kv.is_contiguous() or kv.dim() != 4 \
            or kv.shape[1] != 2:
        raise ValueError("expected a contiguous fp16 CUDA tensor [L, 2, S, C]")
    if shape is not None and tuple(kv.shape) != tuple(shape):
        raise ValueError("KV shape %s does not match the tables %s" % (tuple(kv.shape), shape))


class Tables:
    """Per-(layer, K/V, channel) ranges and frequency tables, owned by libcg."""

    def __init__(self, handle: ctypes.c_void_p, L, H_kv, d, S, group, chunk, bins, device,
                 bins_v=None, n_sink=0, anchor_bits=16, outlier_ppm=0):
        self.handle = handle
        self.n_sink = min(int(n_sink), S)
        self.anchor_bits = int(anchor_bits)
        self.outlier_ppm = int(outlier_ppm)
        self.L, self.H_kv, self.d, self.S = L, H_kv, d, S
        self.group, self.chunk = group, chunk
        self.bins = tuple(int(b) for b in bins)             # K rows (and V rows without bins_v)
        self.bins_v = self.bins if bins_v is None else tuple(int(b) for b in bins_v)
        self.device = device

    @property
    def row_bins(self):
        """Bin count of every (layer, K/V) row, in row order l * 2 + kv."""
        return tuple(n for kv_pair in zip(self.bins, self.bins_v) for n in kv_pair)

    @property
    def C(self) -> int:
        return self.H_kv * self.d

    @property
    def shape(self):
        return (self.L, 2, self.S, self.C)

    @property
    def n_chunks(self) -> int:
        return -(-self.S // self.chunk)

    @property
    def raw_bytes(self) -> int:
        return 2 * self.L * self.C * self.S * 2

    @property
    def stored_bytes(self) -> int:
        info = TablesInfo()
        _check(load().cg_tables_get_info(self.handle, ctypes.byref(info)))
        return int(info.stored_bytes)

    def export(self) -> dict:
        rows = (self.L, 2, self.C)
        lo, w, r = (np.empty(rows, np.float32) for _ in range(3))
        fr = np.empty(rows + (MAX_BINS,), np.uint16)
        _check(load().cg_tables_export(self.handle, lo.ctypes.data, w.ctypes.data,
                                       r.ctypes.data, fr.ctypes.data))
        return {"lo": lo, "w": w, "r": r, "freqs": fr}

    def serialize(self) -> bytes:
        """The stored tables (include/cg.h layout)."""
        n = ctypes.c_uint64()
        _check(load().cg_tables_serialize(self.handle, None, 0, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(max(n.value, 1))
        _check(load().cg_tables_serialize(self.handle, buf, n.value, ctypes.byref(n)))
        return buf.raw[:n.value]

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.cg_free(self.handle)
            self.handle = None


class Blob:
    """One encoded container (device memory owned by libcg)."""

    def __init__(self, handle: ctypes.c_void_p, tables: Tables):
        self.handle = handle
        self.tables = tables
        info = BlobInfo()
        _check(load().cg_blob_get_info(handle, ctypes.byref(info)))
        self.data_ptr = int(info.data)
        h = info.header
        self.header = {f: getattr(h, f) for f, _ in ContainerHeader._fields_}

    @property
    def nbytes(self) -> int:
        return int(self.header["total_bytes"])

    @property
    def chunk_begin(self) -> int:
        return int(self.header["chunk_begin"])

    @property
    def chunk_end(self) -> int:
        return int(self.header["chunk_end"])

    def read_into(self, dst: torch.Tensor) -> torch.Tensor:
        """Copies the whole container into a contiguous uint8 CPU tensor (e.g. pinned)."""
        if dst.device.type != "cpu" or dst.dtype != torch.uint8 or not dst.is_contiguous() \
                or dst.numel() < self.nbytes:
            raise ValueError("destination must be a contiguous uint8 CPU tensor of the "
                             "container's size")
        _check(load().cg_blob_read(self.handle, 0, self.nbytes, dst.data_ptr()))
        return dst

    def read(self, offset: int = 0, nbytes: Optional[int] = None) -> np.ndarray:
        nbytes = self.nbytes - offset if nbytes is None else nbytes
        buf = np.empty(max(nbytes, 1), np.uint8)
        _check(load().cg_blob_read(self.handle, offset, nbytes, buf.ctypes.data))
        return buf[:nbytes]

    def offsets(self) -> np.ndarray:
        h = self.header
        return self.read(h["offsets_offset"], (h["n_groups"] + 1) * 8).view(np.uint64)

    def anchors(self) -> np.ndarray:
        """fp16 bits [rows, C], or uint8 grid codes [rows, C] with 8-bit anchors."""
        h = self.header
        raw = self.read(h["anchors_offset"], h["anchors_bytes"])
        return (raw if h["anchor_bits"] == 8 else raw.view(np.uint16)).reshape(-1, self.tables.C)

    def outliers(self):
        """(offsets uint64 [n_groups + 1], keys uint32, values uint16), or None without
        the outlier table."""
        h = self.header
        if not h["outlier_ppm"]:
            return None
        n = h["n_outliers"]
        offs = self.read(h["outliers_offset"], (h["n_groups"] + 1) * 8).view(np.uint64)
        keys = self.read(h["outlier_keys_offset"], n * 4).view(np.uint32)
        vals = self.read(h["outlier_values_offset"], n * 2).view(np.uint16)
        return offs, keys, vals

    def payload(self) -> np.ndarray:
        h = self.header
        return self.read(h["payload_offset"], h["payload_words"] * 2).view(np.uint16)

    def raw_bytes(self) -> int:
        t = self.tables
        t0 = self.chunk_begin * t.chunk
        t1 = min(self.chunk_end * t.chunk, t.S)
        return 2 * t.L * t.C * (t1 - t0) * 2

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.cg_free(self.handle)
            self.handle = None


def build_cdf(kv: torch.Tensor, group: int, chunk: int, bins: Sequence[int],
              H_kv: Optional[int] = None, bins_v: Optional[Sequence[int]] = None,
              n_sink: int = 0, anchor_bits: int = 16, outlier_ppm: int = 0) -> Tables:
    """kv: fp16 CUDA [L, 2, S, C].  H_kv only labels the channel split (C = H_kv * d).
    bins: bin count per layer; with bins_v, those of the K rows, and bins_v those of the
    V rows.  n_sink: the first n_sink tokens are kept in fp16 (attention sinks), in every
    container that holds them.
    anchor_bits: 16 (fp16 anchors) or 8 (anchors as codes on a per-channel grid).
    outlier_ppm: 0, or the clip budget (parts per million at each end) of the sparse
    outlier table."""
    _kv_check(kv)
    if n_sink < 0:
        raise ValueError("n_sink must be >= 0")
    if anchor_bits not in (8, 16):
        raise ValueError("anchor_bits must be 8 or 16")
    L, _, S, C = kv.shape
    H = H_kv if H_kv is not None else 1
    if C % H:
        raise ValueError("C must be a multiple of H_kv")
    b = np.ascontiguousarray(np.asarray(bins, dtype=np.uint8))
    if b.shape != (L,):
        raise ValueError("need one bin count per layer")
    bv = None if bins_v is None else np.ascontiguousarray(np.asarray(bins_v, dtype=np.uint8))
    if bv is not None and bv.shape != (L,):
        raise ValueError("need one V bin count per layer")
    u8p = ctypes.POINTER(ctypes.c_uint8)
    p = Params(L, H, C // H, S, group, chunk, b.ctypes.data_as(u8p),
               bv.ctypes.data_as(u8p) if bv is not None else None, int(n_sink),
               int(anchor_bits), int(outlier_ppm))
    h = ctypes.c_void_p()
    with torch.cuda.device(kv.device):
        _check(load().cg_build_cdf(ctypes.byref(p), kv.data_ptr(), _stream(kv.device),
                                   ctypes.byref(h)))
    return Tables(h, L, H, C // H, S, group, chunk, b, kv.device, bins_v=bv, n_sink=n_sink,
                  anchor_bits=anchor_bits, outlier_ppm=outlier_ppm)


def encode(tables: Tables, kv: torch.Tensor, chunk_begin: int = 0,
           chunk_end: Optional[int] = None) -> Blob:
    _kv_check(kv, tables.shape)
    chunk_end = tables.n_chunks if chunk_end is None else chunk_end
    h = ctypes.c_void_p()
    with torch.cuda.device(kv.device):
        _check(load().cg_encode(tables.handle, kv.data_ptr(), chunk_begin, chunk_end,
                                _stream(kv.device), ctypes.byref(h)))
    return Blob(h, tables)


def decode_paged(tables: Tables, blob: Blob, pages: torch.Tensor, block_table: torch.Tensor,
                 container: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decodes into a paged cache: pages fp16 CUDA [L, 2, num_pages, page_tokens, C],
    block_table int32 CUDA [ceil(S / page_tokens)] (logical token block -> page)."""
    L, two, num_pages, P, C = pages.shape
    if (pages.dtype != torch.float16 or not pages.is_cuda or not pages.is_contiguous()
            or (L, two, C) != (tables.L, 2, tables.C)):
        raise ValueError("pages must be contiguous fp16 CUDA [L, 2, num_pages, page_tokens, C]")
    nb = -(-tables.S // P)
    if (block_table.dtype != torch.int32 or not block_table.is_cuda
            or not block_table.is_contiguous() or block_table.numel() < nb):
        raise ValueError("block_table must be contiguous int32 CUDA with ceil(S / page_tokens) entries")
    with torch.cuda.device(pages.device):
        _check(load().cg_decode_paged(tables.handle, blob.handle,
                                      container.data_ptr() if container is not None else None,
                                      pages.data_ptr(), block_table.data_ptr(), P, num_pages,
                                      _stream(pages.device)))
    return pages


def decode(tables: Tables, blob: Blob, out: Optional[torch.Tensor] = None,
           container: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Writes the container's tokens into `out` (fp16 [L, 2, S, C]); asynchronous."""
    if out is None:
        out = torch.empty(tables.shape, dtype=torch.float16, device=tables.device)
    _kv_check(out, tables.shape)
    cptr = None
    if container is not None:
        if not container.is_cuda or container.numel() * container.element_size() < blob.nbytes:
            raise ValueError("container buffer must be a CUDA tensor of at least blob.nbytes")
        cptr = container.data_ptr()
    with torch.cuda.device(out.device):
        _check(load().cg_decode(tables.handle, blob.handle, cptr, out.data_ptr(),
                                _stream(out.device)))
    return out


def quantize(tables: Tables, kv: torch.Tensor, chunk_begin: int = 0,
             chunk_end: Optional[int] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _kv_check(kv, tables.shape)
    chunk_end = tables.n_chunks if chunk_end is None else chunk_end
    if out is None:
        out = torch.zeros(tables.shape, dtype=torch.uint8, device=kv.device)
    if out.dtype != torch.uint8 or tuple(out.shape) != tables.shape or not out.is_contiguous():
        raise ValueError("symbols must be contiguous uint8 [L, 2, S, C]")
    with torch.cuda.device(kv.device):
        _check(load().cg_quantize(tables.handle, kv.data_ptr(), chunk_begin, chunk_end,
                                  out.data_ptr(), _stream(kv.device)))
    return out


def decode_symbols(tables: Tables, blob: Blob, out: Optional[torch.Tensor] = None,
                   container: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.zeros(tables.shape, dtype=torch.uint8, device=tables.device)
    if out.dtype != torch.uint8 or tuple(out.shape) != tables.shape or not out.is_contiguous():
        raise ValueError("symbols must be contiguous uint8 [L, 2, S, C]")
    cptr = container.data_ptr() if container is not None else None
    with torch.cuda.device(out.device):
        _check(load().cg_decode_symbols(tables.handle, blob.handle, cptr, out.data_ptr(),
                                        _stream(out.device)))
    return out


def dequantize(tables: Tables, blob: Blob, sym: torch.Tensor,
               out: Optional[torch.Tensor] = None,
               container: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.zeros(tables.shape, dtype=torch.float16, device=tables.device)
    _kv_check(out, tables.shape)
    if sym.dtype != torch.uint8 or tuple(sym.shape) != tables.shape or not sym.is_contiguous():
        raise ValueError("symbols must be contiguous uint8 [L, 2, S, C]")
    cptr = container.data_ptr() if container is not None else None
    with torch.cuda.device(out.device):
        _check(load().cg_dequantize(tables.handle, blob.handle, cptr, sym.data_ptr(),
                                    out.data_ptr(), _stream(out.device)))
    return out


def compressed_bytes(tables: Tables, blobs: Sequence[Blob]) -> int:
    """Everything needed to decode: the containers plus the stored tables."""
    return sum(b.nbytes for b in blobs) + tables.stored_bytes


def stream_decode(items: Sequence[tuple], staging: torch.Tensor, n_slots: int,
                  out: torch.Tensor, copy_stream: torch.cuda.Stream,
                  decode_stream: torch.cuda.Stream, wait: bool = True) -> Optional[dict]:
    """items: (Tables, Blob, host uint8 tensor holding Blob.read()) per container, decoded
    in order into `out`; `staging` (uint8 CUDA) is split into n_slots equal slots.  With
    wait=True returns the event timings, otherwise returns once the work is queued."""
    if not items:
        return {"total_ms": 0.0, "copy_ms": 0.0, "decode_ms": 0.0, "copied_bytes": 0}
    t0 = items[0][0]
    _kv_check(out, t0.shape)
    if not staging.is_cuda or staging.dtype != torch.uint8 or not staging.is_contiguous():
        raise ValueError("staging must be a contiguous uint8 CUDA tensor")
    slot_bytes = staging.numel() // n_slots if n_slots > 0 else 0
    arr = (StreamItem * len(items))()
    for i, (t, b, host) in enumerate(items):
        if host.device.type != "cpu" or host.dtype != torch.uint8 or host.numel() < b.nbytes \
                or not host.is_contiguous():
            raise ValueError("item %d: host container must be a contiguous uint8 CPU tensor "
                             "of the container's size" % i)
        arr[i] = StreamItem(t.handle.value if isinstance(t.handle, ctypes.c_void_p) else t.handle,
                            b.handle.value if isinstance(b.handle, ctypes.c_void_p) else b.handle,
                            host.data_ptr())
    st = StreamStats()
    with torch.cuda.device(out.device):
        _check(load().cg_stream_decode(arr, len(items), staging.data_ptr(), slot_bytes,
                                       max(n_slots, 0), out.data_ptr(),
                                       ctypes.c_void_p(copy_stream.cuda_stream),
                                       ctypes.c_void_p(decode_stream.cuda_stream),
                                       ctypes.byref(st) if wait else None))
    if not wait:
        return None
    return {"total_ms": st.total_ms, "copy_ms": st.copy_ms, "decode_ms": st.decode_ms,
            "copied_bytes": int(st.copied_bytes)}


# ------------------------------------------------------------------ stored form
def _bytes_arg(data) -> tuple:
    buf = np.frombuffer(bytes(data) if not isinstance(data, (bytes, bytearray)) else data, np.uint8)
    return buf, buf.ctypes.data if buf.size else None


def tables_check(data) -> dict:
    """Checks stored tables on the host (no device); returns the header fields."""
    buf, ptr = _bytes_arg(data)
    h = TablesHeader()
    _check(load().cg_tables_check(ptr, buf.size, ctypes.byref(h)))
    return {f: getattr(h, f) for f, _ in TablesHeader._fields_}


def container_check(data) -> dict:
    """Checks a container on the host (no device); returns the header fields."""
    buf, ptr = _bytes_arg(data)
    h = ContainerHeader()
    _check(load().cg_container_check(ptr, buf.size, ctypes.byref(h)))
    return {f: getattr(h, f) for f, _ in ContainerHeader._fields_}


def tables_import(data, device=None) -> Tables:
    """Tables handle on `device` (default: the current CUDA device) from stored tables."""
    hdr = tables_check(data)
    buf, ptr = _bytes_arg(data)
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    h = ctypes.c_void_p()
    with torch.cuda.device(dev):
        _check(load().cg_tables_import(ptr, buf.size, ctypes.byref(h)))
    L = hdr["L"]
    bins = np.frombuffer(buf[56:56 + 2 * L].tobytes(), np.uint8).reshape(L, 2)
    return Tables(h, L, hdr["H_kv"], hdr["d"], hdr["S"], hdr["group"], hdr["chunk"],
                  bins[:, 0].copy(), dev, bins_v=bins[:, 1].copy(), n_sink=hdr["n_sink"],
                  anchor_bits=hdr["anchor_bits"], outlier_ppm=hdr["outlier_ppm"])


def blob_import(tables: Tables, data) -> Blob:
    """Blob on the tables' device from container bytes (checked first)."""
    buf, ptr = _bytes_arg(data)
    h = ctypes.c_void_p()
    with torch.cuda.device(tables.device):
        _check(load().cg_blob_import(tables.handle, ptr, buf.size, _stream(tables.device),
                                     ctypes.byref(h)))
    return Blob(h, tables)


def encode_noalloc(tables: Tables, kv: torch.Tensor, container: torch.Tensor,
                   chunk_begin: int = 0, chunk_end: Optional[int] = None) -> dict:
    """cg_encode_noalloc: the container of chunks [chunk_begin, chunk_end) written into
    `container` (a CUDA uint8 tensor, 256-byte aligned); returns the header fields."""
    _kv_check(kv, tables.shape)
    chunk_end = tables.n_chunks if chunk_end is None else chunk_end
    if not container.is_cuda or container.dtype != torch.uint8 or not container.is_contiguous():
        raise ValueError("container must be a contiguous uint8 CUDA tensor")
    h = ContainerHeader()
    with torch.cuda.device(kv.device):
        _check(load().cg_encode_noalloc(tables.handle, kv.data_ptr(), chunk_begin, chunk_end,
                                        container.data_ptr(), container.numel(),
                                        _stream(kv.device), ctypes.byref(h)))
    return {f: getattr(h, f) for f, _ in ContainerHeader._fields_}
