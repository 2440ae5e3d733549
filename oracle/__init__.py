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
_u32p = ctypes.POINTER(ctypes.c_uint32)
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
        L.cgo_range.argtypes = [_u32] * 6 + [_u8p, _u16p, _f32p, _f32p, _f32p, _u32, _u32]
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
        L.cgo_outliers.argtypes = ([_u32] * 6 + [_u8p, _u16p, _u16p, _f32p, _f32p, _f32p, _f32p,
                                               _u32, _u32, _u32, _u64p, _u32p, _u16p])
        L.cgo_outliers.restype = ctypes.c_uint64
        L.cgo_apply_outliers.argtypes = ([_u32] * 5 + [_u32, _u32, _u64p, _u32p, _u16p,
                                                     ctypes.c_uint64, _u16p])
        L.cgo_apply_outliers.restype = ctypes.c_int
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
    outlier_ppm: int = 0   # 0: no outlier table; else the clip budget per end, parts per million

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
             n_sink: int = 0, anchor_bits: int = 16, outlier_ppm: int = 0) -> "Shape":
        """bins: the bin count of each layer (K and V rows alike), or of its K rows when
        bins_v gives those of the V rows (the keys-finer-than-values variant of the
        Guide's Solution pillar 1).  n_sink: the first n_sink tokens of the sequence are
        reproduced exactly from an fp16 copy and left out of the ranges and histograms
        (the Guide's Best Practices: protect the attention sinks).  anchor_bits = 8 stores
        each anchor as a code on a 256-level grid of its channel (the Guide's Solution
        pillar 2: anchors quantized with high precision); the deltas are taken against
        the anchor's grid value.  outlier_ppm > 0 turns on the sparse outlier table (the
        Guide's Solution pillar 3): each channel's grid spans a central range that leaves
        at most outlier_ppm / 10^6 of its deltas out at each end, and every element off
        its grid is stored exactly in fp16 in the container."""
        assert anchor_bits in (8, 16)
        assert 0 <= outlier_ppm <= 250000
        k = np.asarray(bins, dtype=np.uint8)
        v = k if bins_v is None else np.asarray(bins_v, dtype=np.uint8)
        assert k.shape == (L,) and v.shape == (L,)
        return Shape(L, H, d, S, G, Tc, np.ascontiguousarray(np.stack([k, v], axis=1).reshape(-1)),
                     int(n_sink), int(anchor_bits), int(outlier_ppm))


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
    X = snap_anchors(shp, X, Tables(None, None, None, None, None, *grid))
    lo = np.empty((shp.L, 2, shp.C), np.float32)
    w = np.empty_like(lo)
    r = np.empty_like(lo)
    rc = lib().cgo_range(*shp.args(), _p(shp.bins, _u8p), _p(X, _u16p), _p(lo, _f32p),
                         _p(w, _f32p), _p(r, _f32p), shp.n_sink, shp.outlier_ppm)
    if rc == -4:
        raise NonFinite("input holds Inf or NaN")
    sym = quantize(shp, X, lo, r, 0, shp.S)
    counts = np.empty((shp.L, 2, shp.C, MAX_BINS), np.uint64)
    lib().cgo_histograms(*shp.args(), _p(shp.bins, _u8p), _p(sym, _u8p), _p(counts, _u64p),
                         shp.n_sink)
    freqs = np.empty((shp.L, 2, shp.C, MAX_BINS), np.uint16)
    lib().cgo_freqs(shp.L, shp.C, _p(shp.bins, _u8p), _p(counts, _u64p), _p(freqs, _u16p))
    del X0
    return Tables(lo, w, r, counts, freqs, *grid)


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
    sinks: np.ndarray = None        # uint16 [L, 2, n, C]: the sink tokens among the chunks
    out_offsets: np.ndarray = None  # uint64 [n_groups + 1]: outlier entries per group
    out_keys: np.ndarray = None     # uint32 [n_out]: (token within the chunk) << 6 | lane
    out_values: np.ndarray = None   # uint16 [n_out]: fp16 bits
    clamped: int = 0                # off-grid elements coded clamped (no outlier table)

    @property
    def payload_bytes(self) -> int:
        return int(self.payload.size) * 2

    @property
    def n_outliers(self) -> int:
        return 0 if self.out_keys is None else int(self.out_keys.size)


def n_groups(shp: Shape, k_begin: int, k_end: int) -> int:
    return int(lib().cgo_num_groups(shp.L, shp.C, k_begin, k_end))


def anchor_rows(shp: Shape, k_begin: int, k_end: int) -> int:
    return int(lib().cgo_anchor_rows(shp.L, shp.S, shp.G, shp.Tc, k_begin, k_end))


def sink_tokens(shp: Shape, k_begin: int, k_end: int) -> Tuple[int, int]:
    """Token range [a, b) of the sink tokens among chunks [k_begin, k_end)."""
    a = k_begin * shp.Tc
    b = min(k_end * shp.Tc, shp.S, shp.n_sink)
    return a, max(a, b)


def outliers(shp: Shape, X: np.ndarray, tab: Tables, k_begin: int, k_end: int, store: bool):
    """(offsets, keys, values, count) of the outlier table of chunks [k_begin, k_end);
    with store=False only the count of off-grid elements."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    Xs = np.ascontiguousarray(snap_anchors(shp, X, tab))
    ng = n_groups(shp, k_begin, k_end)
    a8 = shp.anchor_bits == 8
    f32 = lambda a: _p(np.ascontiguousarray(a, np.float32), _f32p) if a is not None else None
    args = (*shp.args(), _p(shp.bins, _u8p), _p(X, _u16p), _p(Xs, _u16p), f32(tab.lo), f32(tab.r),
            f32(tab.alo) if a8 else None, f32(tab.ar) if a8 else None, shp.n_sink, k_begin, k_end)
    n = int(lib().cgo_outliers(*args, None, None, None))
    if not store:
        return None, None, None, n
    offsets = np.zeros(ng + 1, np.uint64)
    keys = np.zeros(max(n, 1), np.uint32)
    values = np.zeros(max(n, 1), np.uint16)
    n2 = int(lib().cgo_outliers(*args, _p(offsets, _u64p), _p(keys, _u32p), _p(values, _u16p)))
    assert n2 == n
    return offsets, keys[:n].copy(), values[:n].copy(), n


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
    sa, sb = sink_tokens(shp, k_begin, k_end)
    enc = Encoded(k_begin, k_end, offsets, payload[:n].copy(), anchors[:rows].copy(),
                  sinks=X[:, :, sa:sb].copy())
    if shp.outlier_ppm:
        enc.out_offsets, enc.out_keys, enc.out_values, _ = outliers(shp, X, tab, k_begin, k_end, True)
    else:
        enc.clamped = outliers(shp, X, tab, k_begin, k_end, False)[3]
    return enc


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
    """fp16 bits [L, 2, S, C]; tokens outside the encoded chunks are left as in `out`.
    The decoded rows first, then the container's sink rows and outlier entries."""
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
    _put_extras(shp, enc, out)
    return out


def _put_extras(shp: Shape, enc: Encoded, out: np.ndarray) -> None:
    """The container's sink rows, then its outlier entries, written over `out`."""
    sa, sb = sink_tokens(shp, enc.k_begin, enc.k_end)
    if sb > sa:
        out[:, :, sa:sb] = enc.sinks
    if enc.out_keys is not None and enc.out_keys.size:
        rc = lib().cgo_apply_outliers(shp.L, shp.H, shp.d, shp.S, shp.Tc, enc.k_begin, enc.k_end,
                                      _p(np.ascontiguousarray(enc.out_offsets), _u64p),
                                      _p(np.ascontiguousarray(enc.out_keys), _u32p),
                                      _p(np.ascontiguousarray(enc.out_values), _u16p),
                                      enc.out_keys.size, _p(out, _u16p))
        if rc != 0:
            raise ValueError("inconsistent outlier table (code %d)" % rc)


def dequantize(shp: Shape, tab: Tables, sym: np.ndarray, X_anchor_src: np.ndarray,
               t_begin: int, t_end: int, enc: Optional[Encoded] = None) -> np.ndarray:
    """The unfused path: symbols and anchors to fp16, then (given a container) its sink
    rows and outlier entries."""
    out = np.zeros((shp.L, 2, shp.S, shp.C), np.uint16)
    src = snap_anchors(shp, np.ascontiguousarray(X_anchor_src, np.uint16), tab)
    lib().cgo_dequantize(*shp.args(), _p(np.ascontiguousarray(tab.lo), _f32p),
                         _p(np.ascontiguousarray(tab.w), _f32p),
                         _p(np.ascontiguousarray(sym, np.uint8), _u8p),
                         _p(src, _u16p),
                         t_begin, t_end, _p(out, _u16p))
    if enc is not None:
        _put_extras(shp, enc, out)
    return out


# ------------------------------------------------------------------ stored bytes
# Byte layouts of the two stored objects, written from their specification in
# include/cg.h (cg_tables_header, cg_container_header): little endian, fixed-width.
TABLES_MAGIC = 0x31544743      # "CGT1"
TABLES_VERSION = 1
CONTAINER_MAGIC = 0x31474B43   # "CKG1"
CONTAINER_VERSION = 3
PAYLOAD_PAD = 1024


def _a256(x: int) -> int:
    return (x + 255) & ~255


def table_bytes(shp: Shape) -> int:
    """Size of the stored tables (tables_bytes): a 56-byte header, the bin count of every
    (layer, K/V) row (padded to 4 bytes), lo and w (4 B each) per channel row, alo and aw
    too with 8-bit anchors, and N 2-byte frequencies per channel row."""
    rows = 2 * shp.L * shp.C
    return int(56 + ((2 * shp.L + 3) & ~3) + rows * 8 * (2 if shp.anchor_bits == 8 else 1)
               + sum(int(b) * shp.C * 2 for b in shp.bins))


def tables_bytes(shp: Shape, tab: Tables) -> bytes:
    # a sink count above S acts as S and is stored as such
    head = np.array([TABLES_MAGIC, TABLES_VERSION, shp.L, shp.H, shp.d, shp.S, shp.G, shp.Tc,
                     min(shp.n_sink, shp.S), shp.anchor_bits, shp.outlier_ppm, 0],
                    np.uint32).tobytes()
    parts = [head, np.array([table_bytes(shp)], np.uint64).tobytes()]
    bins = np.zeros((2 * shp.L + 3) & ~3, np.uint8)
    bins[:2 * shp.L] = shp.bins
    parts += [bins.tobytes(), tab.lo.astype(np.float32).tobytes(), tab.w.astype(np.float32).tobytes()]
    if shp.anchor_bits == 8:
        parts += [tab.alo.astype(np.float32).tobytes(), tab.aw.astype(np.float32).tobytes()]
    for l in range(shp.L):
        for kv in range(2):
            N = int(shp.bins[l * 2 + kv])
            parts.append(np.ascontiguousarray(tab.freqs[l, kv, :, :N]).astype(np.uint16).tobytes())
    out = b"".join(parts)
    assert len(out) == table_bytes(shp)
    return out


def container_layout(shp: Shape, enc: Encoded) -> dict:
    """Header fields of the container (version 3): every section 256-byte aligned."""
    ng = n_groups(shp, enc.k_begin, enc.k_end)
    sa, sb = sink_tokens(shp, enc.k_begin, enc.k_end)
    h = dict(magic=CONTAINER_MAGIC, version=CONTAINER_VERSION, L=shp.L, H_kv=shp.H, d=shp.d,
             S=shp.S, group=shp.G, chunk=shp.Tc, chunk_begin=enc.k_begin, chunk_end=enc.k_end,
             n_blocks=-(-shp.C // LANES), anchor_bits=shp.anchor_bits, n_sink=sb - sa,
             outlier_ppm=shp.outlier_ppm, n_groups=ng)
    h["offsets_offset"] = _a256(160)
    h["anchors_offset"] = _a256(h["offsets_offset"] + (ng + 1) * 8)
    h["anchors_bytes"] = anchor_rows(shp, enc.k_begin, enc.k_end) * shp.C * (1 if shp.anchor_bits == 8 else 2)
    h["sinks_offset"] = _a256(h["anchors_offset"] + h["anchors_bytes"])
    end = h["sinks_offset"] + 2 * shp.L * (sb - sa) * shp.C * 2
    n_out = enc.n_outliers
    h["outliers_offset"] = _a256(end)
    if shp.outlier_ppm:
        h["outlier_keys_offset"] = _a256(h["outliers_offset"] + (ng + 1) * 8)
        h["outlier_values_offset"] = _a256(h["outlier_keys_offset"] + n_out * 4)
        end = h["outlier_values_offset"] + n_out * 2
    else:
        h["outlier_keys_offset"] = h["outlier_values_offset"] = h["outliers_offset"]
    h["n_outliers"] = n_out
    h["clamped"] = enc.clamped
    h["payload_offset"] = _a256(end)
    h["payload_words"] = int(enc.payload.size)
    h["total_bytes"] = h["payload_offset"] + 2 * h["payload_words"] + PAYLOAD_PAD
    return h


HEADER_U32 = ("magic", "version", "L", "H_kv", "d", "S", "group", "chunk", "chunk_begin",
              "chunk_end", "n_blocks", "anchor_bits", "n_sink", "outlier_ppm")
HEADER_U64 = ("n_groups", "offsets_offset", "anchors_offset", "anchors_bytes", "sinks_offset",
              "outliers_offset", "outlier_keys_offset", "outlier_values_offset", "n_outliers",
              "clamped", "payload_offset", "payload_words", "total_bytes")


def container_bytes(shp: Shape, enc: Encoded) -> bytes:
    """The whole container (version 3), zero bytes between sections and 1 KiB of zeros
    after the payload."""
    h = container_layout(shp, enc)
    buf = np.zeros(h["total_bytes"], np.uint8)
    head = (np.array([h[k] for k in HEADER_U32], np.uint32).tobytes() +
            np.array([h[k] for k in HEADER_U64], np.uint64).tobytes())
    assert len(head) == 160

    def put(off, arr):
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        buf[off:off + b.size] = b

    put(0, np.frombuffer(head, np.uint8))
    put(h["offsets_offset"], enc.offsets.astype(np.uint64))
    put(h["anchors_offset"], enc.anchors)
    if h["n_sink"]:
        put(h["sinks_offset"], enc.sinks.astype(np.uint16))
    if shp.outlier_ppm:
        put(h["outliers_offset"], enc.out_offsets.astype(np.uint64))
        if enc.n_outliers:
            put(h["outlier_keys_offset"], enc.out_keys.astype(np.uint32))
            put(h["outlier_values_offset"], enc.out_values.astype(np.uint16))
    if enc.payload.size:
        put(h["payload_offset"], enc.payload.astype(np.uint16))
    return buf.tobytes()
