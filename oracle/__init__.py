"""CPU oracle of the KV-cache codec: TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  It wraps oracle/cgo.c (plain scalar C, -O2 -ffp-contract=off) with ctypes
and numpy; it shares no code with the GPU library and never imports it.

Parity status of each function is listed in its docstring; every function here is
pinned by the CPU tests in tests/test_oracle_pins.py against properties fixed by the
pages or by mathematics (closed-form sizes, exhaustive round trips, a big-integer
closed form of the coder on uniform tables, exact rational bounds, brute force on tiny tensors).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cgo.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD_DIR, "libcgo.so")

PROB_BITS = 8
PROB_TOTAL = 1 << PROB_BITS
MAX_BINS = 32
LANES = 64

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_u32 = ctypes.c_uint32


def build(force: bool = True) -> str:
    """Compile cgo.c into oracle/_build/libcgo.so with gcc."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                           "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, SRC, "-lm"])
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)          # (re)compiles only when cgo.c is newer than the library
        L = ctypes.CDLL(LIB)
        L.cgo_half_to_float_n.argtypes = [_u16p, _f32p, ctypes.c_size_t]
        L.cgo_float_to_half_n.argtypes = [_f32p, _u16p, ctypes.c_size_t]
        L.cgo_range.argtypes = [_u32] * 6 + [_u8p, _u16p, _f32p, _f32p, _f32p, _u32]
        L.cgo_range.restype = ctypes.c_int
        L.cgo_quantize.argtypes = [_u32] * 6 + [_u8p, _u16p, _f32p, _f32p, _u32, _u32, _u8p]
        L.cgo_histograms.argtypes = [_u32] * 6 + [_u8p, _u8p, _u64p, _u32]
        L.cgo_anchor_grid.argtypes = [_u32] * 6 + [_u16p, _f32p, _f32p, _f32p]
        L.cgo_snap_anchors.argtypes = [_u32] * 6 + [_u16p, _f32p, _f32p, _f32p, _u16p]
        L.cgo_anchor_codes.argtypes = [_u32] * 6 + [_u16p, _f32p, _f32p, _u32, _u32, _u8p]
        L.cgo_anchors_from_codes.argtypes = [_u32] * 5 + [_u8p, _f32p, _f32p, _u32, _u32, _u16p]
        L.cgo_freqs.argtypes = [_u32, _u32, _u8p, _u64p, _u16p]
        L.cgo_freqs_from_counts.argtypes = [_u64p, _u32, _u16p]
        L.cgo_rans_encode.argtypes = [_u8p, _u32, _u16p, _u32, _u16p, _i32p]
        L.cgo_rans_encode.restype = _u32
        L.cgo_rans_decode.argtypes = [_u16p, _u32, _u32, _u16p, _u32, _u8p,
                                      ctypes.POINTER(ctypes.c_uint32)]
        L.cgo_rans_decode.restype = _u32
        L.cgo_num_groups.argtypes = [_u32, _u32, _u32, _u32]
        L.cgo_num_groups.restype = ctypes.c_uint64
        L.cgo_anchor_rows.argtypes = [_u32] * 6
        L.cgo_anchor_rows.restype = ctypes.c_uint64
        L.cgo_anchors.argtypes = [_u32] * 6 + [_u16p, _u32, _u32, _u16p]
        L.cgo_encode_payload.argtypes = ([_u32] * 6 + [_u8p, _u8p, _u16p, _u32, _u32, _u64p,
                                                       _u16p, ctypes.c_uint64])
        L.cgo_encode_payload.restype = ctypes.c_int64
        L.cgo_decode.argtypes = ([_u32] * 6 + [_u8p, _f32p, _f32p, _u16p, _u32, _u32, _u64p,
                                               _u16p, ctypes.c_uint64, _u16p, _u16p])
        L.cgo_decode.restype = ctypes.c_int
        L.cgo_dequantize.argtypes = ([_u32] * 6 + [_f32p, _f32p, _u8p, _u16p, _u32, _u32,
                                                   _u16p])
        for name in ("cgo_num_chunks", "cgo_chunk_len", "cgo_groups_in", "cgo_anchor_of"):
            getattr(L, name).restype = _u32
        L.cgo_num_chunks.argtypes = [_u32, _u32]
        L.cgo_chunk_len.argtypes = [_u32, _u32, _u32]
        L.cgo_groups_in.argtypes = [_u32, _u32]
        L.cgo_is_anchor.argtypes = [_u32, _u32, _u32]
        L.cgo_is_anchor.restype = ctypes.c_int
        L.cgo_anchor_of.argtypes = [_u32, _u32, _u32]
        _lib = L
    return _lib


def _p(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


@dataclass
class Shape:
    L: int
    H: int
    d: int
    S: int
    G: int
    Tc: int
    bins: np.ndarray  # uint8 [L][2] flattened: bin count of (layer l, K/V kv) at l * 2 + kv
    n_sink: int = 0   # first tokens of the sequence kept in fp16 (attention sinks)
    anchor_bits: int = 16  # 16: anchors stored as fp16; 8: as codes on a 256-level grid

    @property
    def C(self) -> int:
        return self.H * self.d

    @property
    def n_chunks(self) -> int:
        return -(-self.S // self.Tc)

    def args(self):
        return (self.L, self.H, self.d, self.S, self.G, self.Tc)

    @staticmethod
    def make(L, H, d, S, G, Tc, bins: Sequence[int], bins_v: Optional[Sequence[int]] = None,
             n_sink: int = 0, anchor_bits: int = 16) -> "Shape":
        """bins: the bin count of each layer (K and V rows alike), or of its K rows when
        bins_v gives those of the V rows (the keys-finer-than-values variant of the
        Guide's Solution pillar 1).  n_sink: the first n_sink tokens of the sequence are
        reproduced exactly from an fp16 copy and left out of the ranges and histograms
        (the Guide's Best Practices: protect the attention sinks).  anchor_bits = 8 stores
        each anchor as a code on a 256-level grid of its channel (the Guide's Solution
        pillar 2: anchors quantized with high precision); the deltas are taken against
        the anchor's grid value."""
        assert anchor_bits in (8, 16)
        k = np.asarray(bins, dtype=np.uint8)
        v = k if bins_v is None else np.asarray(bins_v, dtype=np.uint8)
        assert k.shape == (L,) and v.shape == (L,)
        return Shape(L, H, d, S, G, Tc, np.ascontiguousarray(np.stack([k, v], axis=1).reshape(-1)),
                     int(n_sink), int(anchor_bits))


# ------------------------------------------------------------------ fp16 conversions
def half_to_float(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    f = np.empty(h.shape, dtype=np.float32)
    lib().cgo_half_to_float_n(_p(h, _u16p), _p(f, _f32p), h.size)
    return f


def float_to_half(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    h = np.empty(f.shape, dtype=np.uint16)
    lib().cgo_float_to_half_n(_p(f, _f32p), _p(h, _u16p), f.size)
    return h


# ------------------------------------------------------------------ tables
@dataclass
class Tables:
    lo: np.ndarray      # float32 [L, 2, C]
    w: np.ndarray       # float32 [L, 2, C]
    r: np.ndarray       # float32 [L, 2, C]
    counts: np.ndarray  # uint64 [L, 2, C, 32]
    freqs: np.ndarray   # uint16 [L, 2, C, 32]
    sinks: Optional[np.ndarray] = None  # uint16 [L, 2, min(n_sink, S), C]: fp16 copy
    alo: Optional[np.ndarray] = None    # float32 [L, 2, C]: anchor grid (8-bit anchors)
    aw: Optional[np.ndarray] = None
    ar: Optional[np.ndarray] = None


class NonFinite(ValueError):
    pass


def anchor_grid(shp: Shape, X: np.ndarray):
    """alo, aw, ar (float32 [L, 2, C]) of the 8-bit anchor grid."""
    alo = np.empty((shp.L, 2, shp.C), np.float32)
    aw, ar = np.empty_like(alo), np.empty_like(alo)
    lib().cgo_anchor_grid(*shp.args(), _p(X, _u16p), _p(alo, _f32p), _p(aw, _f32p), _p(ar, _f32p))
    return alo, aw, ar


def snap_anchors(shp: Shape, X: np.ndarray, tab: "Tables") -> np.ndarray:
    """X with its anchor tokens replaced by their 8-bit grid values (X itself for fp16
    anchors): the cache the encoder codes the deltas of."""
    if shp.anchor_bits == 16:
        return X
    Y = np.empty_like(X)
    lib().cgo_snap_anchors(*shp.args(), _p(X, _u16p), _p(tab.alo, _f32p), _p(tab.aw, _f32p),
                           _p(tab.ar, _f32p), _p(Y, _u16p))
    return Y


def build_tables(shp: Shape, X: np.ndarray) -> Tables:
    """X: uint16 view of fp16 [L, 2, S, C].  Range, quantize, histogram, frequencies."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    assert X.shape == (shp.L, 2, shp.S, shp.C)
    grid = anchor_grid(shp, X) if shp.anchor_bits == 8 else (None, None, None)
    X0 = X
    X = snap_anchors(shp, X, Tables(None, None, None, None, None, None, *grid))
    lo = np.empty((shp.L, 2, shp.C), np.float32)
    w = np.empty_like(lo)
    r = np.empty_like(lo)
    rc = lib().cgo_range(*shp.args(), _p(shp.bins, _u8p), _p(X, _u16p), _p(lo, _f32p),
                         _p(w, _f32p), _p(r, _f32p), shp.n_sink)
    if rc == -4:
        raise NonFinite("input holds Inf or NaN")
    sym = quantize(shp, X, lo, r, 0, shp.S)
    counts = np.empty((shp.L, 2, shp.C, MAX_BINS), np.uint64)
    lib().cgo_histograms(*shp.args(), _p(shp.bins, _u8p), _p(sym, _u8p), _p(counts, _u64p),
                         shp.n_sink)
    freqs = np.empty((shp.L, 2, shp.C, MAX_BINS), np.uint16)
    lib().cgo_freqs(shp.L, shp.C, _p(shp.bins, _u8p), _p(counts, _u64p), _p(freqs, _u16p))
    sinks = X0[:, :, :min(shp.n_sink, shp.S)].copy()
    return Tables(lo, w, r, counts, freqs, sinks, *grid)


def freqs_from_counts(counts: Sequence[int], N: int) -> np.ndarray:
    c = np.zeros(MAX_BINS, np.uint64)
    c[:N] = counts
    f = np.zeros(MAX_BINS, np.uint16)
    lib().cgo_freqs_from_counts(_p(c, _u64p), N, _p(f, _u16p))
    return f[:N].copy()


def quantize(shp: Shape, X: np.ndarray, lo: np.ndarray, r: np.ndarray,
             t_begin: int, t_end: int) -> np.ndarray:
    """uint8 symbols [L, 2, S, C]; anchors and tokens outside [t_begin, t_end) are 0."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    sym = np.zeros((shp.L, 2, shp.S, shp.C), np.uint8)
    lib().cgo_quantize(*shp.args(), _p(shp.bins, _u8p), _p(X, _u16p),
                       _p(np.ascontiguousarray(lo, np.float32), _f32p),
                       _p(np.ascontiguousarray(r, np.float32), _f32p), t_begin, t_end,
                       _p(sym, _u8p))
    return sym


# ------------------------------------------------------------------ rANS coder
def rans_encode(x: Sequence[int], f: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Single stream: returns (words uint16 in read order, read step of every word int32)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.uint8))
    f = np.ascontiguousarray(np.asarray(f, dtype=np.uint16))
    words = np.zeros(len(x) + 2, np.uint16)
    steps = np.zeros(len(x) + 2, np.int32)
    n = lib().cgo_rans_encode(_p(x, _u8p), len(x), _p(f, _u16p), len(f), _p(words, _u16p),
                              _p(steps, _i32p))
    return words[:n].copy(), steps[:n].copy()


def rans_decode(words: Sequence[int], m: int, f: Sequence[int]) -> Tuple[np.ndarray, int, int]:
    """Returns (symbols, words consumed, final decoder state)."""
    words = np.ascontiguousarray(np.asarray(words, dtype=np.uint16))
    if words.size == 0:
        words = np.zeros(1, np.uint16)[:0]
    f = np.ascontiguousarray(np.asarray(f, dtype=np.uint16))
    out = np.zeros(max(m, 1), np.uint8)
    buf = np.ascontiguousarray(np.concatenate([words, np.zeros(1, np.uint16)]))
    fin = ctypes.c_uint32(0)
    used = lib().cgo_rans_decode(_p(buf, _u16p), len(words), m, _p(f, _u16p), len(f),
                                 _p(out, _u8p), ctypes.byref(fin))
    return out[:m].copy(), int(used), int(fin.value)


# ------------------------------------------------------------------ container
@dataclass
class Encoded:
    k_begin: int
    k_end: int
    offsets: np.ndarray  # uint64 [n_groups + 1] (word offsets)
    payload: np.ndarray  # uint16 [offsets[-1]]
    anchors: np.ndarray  # uint16 (fp16 bits) [rows, C], or uint8 codes with 8-bit anchors

    @property
    def payload_bytes(self) -> int:
        return int(self.payload.size) * 2


def n_groups(shp: Shape, k_begin: int, k_end: int) -> int:
    return int(lib().cgo_num_groups(shp.L, shp.C, k_begin, k_end))


def anchor_rows(shp: Shape, k_begin: int, k_end: int) -> int:
    return int(lib().cgo_anchor_rows(shp.L, shp.S, shp.G, shp.Tc, k_begin, k_end))


def encode(shp: Shape, X: np.ndarray, tab: Tables, k_begin: int = 0,
           k_end: Optional[int] = None) -> Encoded:
    k_end = shp.n_chunks if k_end is None else k_end
    X = np.ascontiguousarray(X, dtype=np.uint16)
    t0, t1 = k_begin * shp.Tc, min(k_end * shp.Tc, shp.S)
    sym = quantize(shp, snap_anchors(shp, X, tab), tab.lo, tab.r, t0, t1)
    ng = n_groups(shp, k_begin, k_end)
    offsets = np.zeros(ng + 1, np.uint64)
    cap = 0
    for k in range(k_begin, k_end):
        m = int(lib().cgo_chunk_len(shp.S, shp.Tc, k))
        cap += shp.L * 2 * shp.C * (m + 2)
    payload = np.zeros(max(cap, 1), np.uint16)
    n = lib().cgo_encode_payload(*shp.args(), _p(shp.bins, _u8p), _p(sym, _u8p),
                                 _p(np.ascontiguousarray(tab.freqs), _u16p), k_begin, k_end,
                                 _p(offsets, _u64p), _p(payload, _u16p), cap)
    assert n >= 0
    rows = anchor_rows(shp, k_begin, k_end)
    if shp.anchor_bits == 8:
        anchors = np.zeros((max(rows, 1), shp.C), np.uint8)
        lib().cgo_anchor_codes(*shp.args(), _p(X, _u16p), _p(tab.alo, _f32p), _p(tab.ar, _f32p),
                               k_begin, k_end, _p(anchors, _u8p))
    else:
        anchors = np.zeros((max(rows, 1), shp.C), np.uint16)
        lib().cgo_anchors(*shp.args(), _p(X, _u16p), k_begin, k_end, _p(anchors, _u16p))
    return Encoded(k_begin, k_end, offsets, payload[:n].copy(), anchors[:rows].copy())


def anchor_values(shp: Shape, tab: Tables, enc: "Encoded") -> np.ndarray:
    """The fp16 anchor rows a container stands for (its codes mapped back for 8-bit
    anchors)."""
    if shp.anchor_bits == 16:
        return enc.anchors
    out = np.zeros(enc.anchors.shape, np.uint16)
    codes = np.ascontiguousarray(enc.anchors)
    lib().cgo_anchors_from_codes(shp.L, shp.C, shp.S, shp.G, shp.Tc, _p(codes, _u8p),
                                 _p(tab.alo, _f32p), _p(tab.aw, _f32p), enc.k_begin, enc.k_end,
                                 _p(out, _u16p))
    return out


def decode(shp: Shape, tab: Tables, enc: Encoded, out: Optional[np.ndarray] = None,
           payload: Optional[np.ndarray] = None) -> np.ndarray:
    """fp16 bits [L, 2, S, C]; tokens outside the encoded chunks are left as in `out`."""
    if out is None:
        out = np.zeros((shp.L, 2, shp.S, shp.C), np.uint16)
    payload = enc.payload if payload is None else payload
    pl = np.ascontiguousarray(np.concatenate([payload.astype(np.uint16), np.zeros(1, np.uint16)]))
    av = anchor_values(shp, tab, enc)
    anchors = np.ascontiguousarray(av if av.size else np.zeros((1, shp.C), np.uint16))
    rc = lib().cgo_decode(*shp.args(), _p(shp.bins, _u8p),
                          _p(np.ascontiguousarray(tab.lo), _f32p),
                          _p(np.ascontiguousarray(tab.w), _f32p),
                          _p(np.ascontiguousarray(tab.freqs), _u16p), enc.k_begin, enc.k_end,
                          _p(np.ascontiguousarray(enc.offsets), _u64p), _p(pl, _u16p),
                          payload.size, _p(anchors, _u16p), _p(out, _u16p))
    if rc != 0:
        raise ValueError("inconsistent container (code %d)" % rc)
    _put_sinks(shp, tab, out, enc.k_begin * shp.Tc, min(enc.k_end * shp.Tc, shp.S))
    return out


def _put_sinks(shp: Shape, tab: Tables, out: np.ndarray, t_begin: int, t_end: int) -> None:
    """The sink tokens in [t_begin, t_end) take their stored fp16 values."""
    for t in range(t_begin, min(t_end, shp.n_sink, shp.S)):
        out[:, :, t] = tab.sinks[:, :, t]


def dequantize(shp: Shape, tab: Tables, sym: np.ndarray, X_anchor_src: np.ndarray,
               t_begin: int, t_end: int) -> np.ndarray:
    out = np.zeros((shp.L, 2, shp.S, shp.C), np.uint16)
    src = snap_anchors(shp, np.ascontiguousarray(X_anchor_src, np.uint16), tab)
    lib().cgo_dequantize(*shp.args(), _p(np.ascontiguousarray(tab.lo), _f32p),
                         _p(np.ascontiguousarray(tab.w), _f32p),
                         _p(np.ascontiguousarray(sym, np.uint8), _u8p),
                         _p(src, _u16p),
                         t_begin, t_end, _p(out, _u16p))
    _put_sinks(shp, tab, out, t_begin, t_end)
    return out


def table_bytes(shp: Shape) -> int:
    """Stored side information: lo and w (4 B each) per channel row, one 2-byte frequency
    per symbol per channel row, one byte per (layer, K/V) for the bin count, the fp16
    copy of the sink tokens, and alo and aw (4 B each) per channel row with 8-bit anchors."""
    return int(2 * shp.C * shp.L * 8 + sum(int(b) * shp.C * 2 for b in shp.bins) + 2 * shp.L
               + 2 * shp.L * min(shp.n_sink, shp.S) * shp.C * 2
               + (2 * shp.C * shp.L * 8 if shp.anchor_bits == 8 else 0))
