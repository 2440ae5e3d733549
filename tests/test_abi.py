"""The C ABI library: it loads, exports every function include/cg.h declares, and its
argument validation answers before touching a device (runs without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cg.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cg_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from kv_cache_compression_cg_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from kv_cache_compression_cg_amd import cg
    return cg.load()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("cg_build_cdf", "cg_encode", "cg_decode", "cg_free"):
        assert required in names


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    from kv_cache_compression_cg_amd import cg
    assert sorted(cg.EXPORTED) == names


def test_validation_without_device(lib):
    from kv_cache_compression_cg_amd import cg
    h = ctypes.c_void_p()
    assert lib.cg_build_cdf(None, None, None, ctypes.byref(h)) == -1
    assert b"null" in lib.cg_last_error()
    bins = (ctypes.c_uint8 * 2)(8, 40)
    p = cg.Params(2, 1, 8, 16, 4, 8, ctypes.cast(bins, ctypes.POINTER(ctypes.c_uint8)))
    assert lib.cg_build_cdf(ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.byref(h)) == -1
    assert b"bins" in lib.cg_last_error()
    p = cg.Params(2, 1, 6, 16, 4, 8, ctypes.cast(bins, ctypes.POINTER(ctypes.c_uint8)))
    assert lib.cg_build_cdf(ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.byref(h)) == -1
    p = cg.Params(2, 1, 8, 16, 4, 20000, ctypes.cast(bins, ctypes.POINTER(ctypes.c_uint8)))
    assert lib.cg_build_cdf(ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.byref(h)) == -1
    # one (layer, K/V) row of symbols and one chunk's rows must fit 32-bit offsets
    one = (ctypes.c_uint8 * 1)(8)
    p = cg.Params(1, 1, 8192, 1 << 19, 10, 1024, ctypes.cast(one, ctypes.POINTER(ctypes.c_uint8)))
    assert lib.cg_build_cdf(ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.byref(h)) == -1
    assert b"too large" in lib.cg_last_error()
    p = cg.Params(1, 1, 1 << 17, 1 << 14, 10, 1 << 14, ctypes.cast(one, ctypes.POINTER(ctypes.c_uint8)))
    assert lib.cg_build_cdf(ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.byref(h)) == -1
    assert b"too large" in lib.cg_last_error()
    # 8-bit or fp16 anchors only
    two = (ctypes.c_uint8 * 2)(8, 8)
    p = cg.Params(2, 1, 8, 16, 4, 8, ctypes.cast(two, ctypes.POINTER(ctypes.c_uint8)), None, 0, 4)
    assert lib.cg_build_cdf(ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.byref(h)) == -1
    assert b"anchor_bits" in lib.cg_last_error()
    p = cg.Params(2, 1, 8, 16, 4, 8, ctypes.cast(two, ctypes.POINTER(ctypes.c_uint8)), None, 0, 16,
                  250001)
    assert lib.cg_build_cdf(ctypes.byref(p), ctypes.c_void_p(16), None, ctypes.byref(h)) == -1
    assert b"outlier_ppm" in lib.cg_last_error()
    assert lib.cg_tables_check(None, 0, None) == -1
    assert lib.cg_container_check(None, 0, None) == -1
    assert lib.cg_tables_import(None, 0, ctypes.byref(h)) == -1
    assert lib.cg_blob_import(None, None, 0, None, ctypes.byref(h)) == -1
    assert lib.cg_tables_serialize(None, None, 0, None) == -1
    assert lib.cg_decode_paged(None, None, None, None, None, 16, 1, None) == -1
    assert lib.cg_encode(None, None, 0, 1, None, ctypes.byref(h)) == -1
    assert lib.cg_decode(None, None, None, None, None) == -1
    assert lib.cg_quantize(None, None, 0, 1, None, None) == -1
    assert lib.cg_blob_read(None, 0, 0, None) == -1
    # streamed decode: argument checks come before any device work
    st = cg.StreamStats()
    a, b = ctypes.c_void_p(1), ctypes.c_void_p(2)
    buf = ctypes.c_void_p(16)
    assert lib.cg_stream_decode(None, 1, buf, 64, 2, buf, a, b, ctypes.byref(st)) == -1
    items = (cg.StreamItem * 1)(cg.StreamItem(None, None, None))
    assert lib.cg_stream_decode(items, 1, buf, 64, 2, buf, a, a, ctypes.byref(st)) == -1
    assert b"differ" in lib.cg_last_error()
    assert lib.cg_stream_decode(items, 1, buf, 64, 0, buf, a, b, ctypes.byref(st)) == -1
    assert lib.cg_stream_decode(items, 1, buf, 64, 2, buf, a, b, ctypes.byref(st)) == -1
    assert b"aligned" in lib.cg_last_error()
    buf = ctypes.c_void_p(4096)
    assert lib.cg_stream_decode(items, 1, buf, 256, 2, buf, a, b, ctypes.byref(st)) == -1
    assert b"cg_tables" in lib.cg_last_error()
    st.total_ms = 5.0
    assert lib.cg_stream_decode(items, 0, buf, 256, 2, buf, a, b, ctypes.byref(st)) == 0
    assert st.total_ms == 0.0 and st.copied_bytes == 0
    lib.cg_free(None)
    # a handle that is neither tables nor blob is ignored
    junk = ctypes.create_string_buffer(64)
    lib.cg_free(junk)


def _struct_fields(name):
    """Field names of a `typedef struct name { ... } name;` in cg.h, in order."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, flags=re.S).group(1)
    fields = []
    for decl in body.split(";"):
        for part in decl.split(","):
            ids = re.findall(r"[A-Za-z_]\w*", re.sub(r"\[.*?\]", "", part))
            if ids:
                fields.append(ids[-1])
    return fields


@pytest.mark.parametrize("cname,pyname", [("cg_params", "Params"),
                                          ("cg_container_header", "ContainerHeader"),
                                          ("cg_tables_header", "TablesHeader"),
                                          ("cg_tables_info", "TablesInfo"),
                                          ("cg_stream_stats", "StreamStats")])
def test_binding_structs_follow_the_header(cname, pyname):
    """The ctypes structures carry the header's fields in the header's order."""
    from kv_cache_compression_cg_amd import cg
    ours = [f for f, _ in getattr(cg, pyname)._fields_]
    assert ours == _struct_fields(cname)


# ----------------------------------------------------------------------------- stored form
def _stored(ppm=30000, anchor_bits=16, n_sink=3, rng=None):
    """Tables and a container made by the oracle (test infrastructure), to feed the
    library's host-side checks."""
    import numpy as np
    import torch
    import oracle as O
    from kv_cache_compression_cg_amd import configs, synth
    L, S, C, G, Tc = 2, 150, 72, 7, 64
    gen = configs.GenSpec(rho=0.85, heavy_tail=True, outlier_frac=0.05, outlier_mult=30.0, seed=2)
    X = np.ascontiguousarray(synth.gen_custom(L, S, C, gen).view(torch.int16).numpy().view(np.uint16))
    shp = O.Shape.make(L, 1, C, S, G, Tc, (8, 16), n_sink=n_sink, anchor_bits=anchor_bits,
                       outlier_ppm=ppm)
    tab = O.build_tables(shp, X)
    kb, ke = rng if rng else (0, shp.n_chunks)
    enc = O.encode(shp, X, tab, kb, ke)
    return shp, enc, O.tables_bytes(shp, tab), O.container_bytes(shp, enc)


@pytest.mark.parametrize("ppm,anchor_bits,rng", [(30000, 16, None), (0, 8, (1, 3)), (30000, 8, (2, 3))])
def test_stored_bytes_pass_the_checks(lib, ppm, anchor_bits, rng):
    from kv_cache_compression_cg_amd import cg
    shp, enc, tb, cb = _stored(ppm, anchor_bits, rng=rng)
    th = cg.tables_check(tb)
    assert (th["L"], th["H_kv"], th["d"], th["S"], th["group"], th["chunk"]) == (2, 1, 72, 150, 7, 64)
    assert th["outlier_ppm"] == ppm and th["anchor_bits"] == anchor_bits and th["total_bytes"] == len(tb)
    ch = cg.container_check(cb)
    assert ch["total_bytes"] == len(cb) and ch["n_outliers"] == enc.n_outliers
    assert ch["payload_words"] == enc.payload.size and ch["version"] == 3
    if ppm:
        assert enc.n_outliers > 0


def _corrupt(buf, off, fmt, value):
    import struct
    b = bytearray(buf)
    struct.pack_into(fmt, b, off, value)
    return bytes(b)


def test_damaged_containers_are_rejected_on_the_host(lib):
    """A container whose header, section layout, group offsets or outlier keys do not
    hold together is refused with CG_E_CORRUPT before any device work."""
    import struct
    from kv_cache_compression_cg_amd import cg
    shp, enc, tb, cb = _stored()
    h = cg.container_check(cb)
    names = [f for f, _ in cg.ContainerHeader._fields_]
    off = {n: (4 * i if i < 14 else 56 + 8 * (i - 14)) for i, n in enumerate(names)}
    fmt = {n: ("<I" if i < 14 else "<Q") for i, n in enumerate(names)}
    bad = [
        _corrupt(cb, 0, "<I", 0x12345678),                                   # magic
        _corrupt(cb, off["version"], "<I", 2),                               # old version
        _corrupt(cb, off["chunk_end"], "<I", 9),                             # range past S
        _corrupt(cb, off["chunk_begin"], "<I", 3),                           # empty range
        _corrupt(cb, off["anchor_bits"], "<I", 4),
        _corrupt(cb, off["anchors_offset"], "<Q", h["anchors_offset"] + 256),
        _corrupt(cb, off["payload_words"], "<Q", h["payload_words"] + 1),    # total no longer fits
        _corrupt(cb, off["n_outliers"], "<Q", h["n_outliers"] + 1),
        _corrupt(cb, off["n_groups"], "<Q", h["n_groups"] - 1),
        _corrupt(cb, off["outlier_ppm"], "<I", 0),                          # entries without table
        _corrupt(cb, h["offsets_offset"], "<Q", 5),                          # first offset not 0
        _corrupt(cb, h["offsets_offset"] + 8 * 3, "<Q", h["payload_words"] + 9),
        _corrupt(cb, h["offsets_offset"] + 8 * h["n_groups"], "<Q", h["payload_words"] - 1),
        _corrupt(cb, h["outliers_offset"] + 8, "<Q", h["n_outliers"] + 1),
        _corrupt(cb, h["outlier_keys_offset"], "<I", (200 << 6) | 3),        # token past the chunk
        cb[:len(cb) - 1025],                                                 # truncated
        cb[:100],
    ]
    # a key in the partial channel block (C = 72: 8 lanes) naming lane 9
    offs = np.frombuffer(cb, np.uint64, h["n_groups"] + 1, h["outliers_offset"])
    for g in range(int(h["n_groups"])):
        if g % 2 == 1 and offs[g + 1] > offs[g]:
            k0 = int(struct.unpack_from("<I", cb, h["outlier_keys_offset"] + 4 * int(offs[g]))[0])
            bad.append(_corrupt(cb, h["outlier_keys_offset"] + 4 * int(offs[g]), "<I", (k0 & ~63) | 9))
            break
    for i, b in enumerate(bad):
        with pytest.raises(cg.CgError) as e:
            cg.container_check(b)
        assert e.value.code == -5, i
    assert fmt["magic"] == "<I"


def test_damaged_tables_are_rejected_on_the_host(lib):
    import struct
    from kv_cache_compression_cg_amd import cg
    shp, enc, tb, cb = _stored()
    L, C = 2, 72
    fr0 = 56 + 4 + 2 * L * C * 8        # first frequency
    bad = [
        _corrupt(tb, 0, "<I", 1),
        _corrupt(tb, 4, "<I", 7),
        _corrupt(tb, 8, "<I", 0),                            # L = 0
        _corrupt(tb, 36, "<I", 12),                          # anchor_bits
        _corrupt(tb, 40, "<I", 250001),                      # outlier_ppm
        _corrupt(tb, 48, "<Q", len(tb) + 2),                 # size
        _corrupt(tb, 56, "<B", 33),                          # bins outside [2, 32]
        _corrupt(tb, 56 + 4, "<f", float("nan")),            # lo
        _corrupt(tb, 56 + 4 + 2 * L * C * 4, "<f", -1.0),    # negative width
        _corrupt(tb, fr0, "<H", 0),                          # a zero frequency
        _corrupt(tb, fr0, "<H", struct.unpack_from("<H", tb, fr0)[0] + 1),   # sum 257
        tb[:-2],
    ]
    for i, b in enumerate(bad):
        with pytest.raises(cg.CgError) as e:
            cg.tables_check(b)
        assert e.value.code == -5, i


def test_import_checks_before_device_work(lib):
    """Valid stored tables pass the check and only then reach the device (no GPU here:
    the import fails with a HIP error, not a corrupt-data error)."""
    from kv_cache_compression_cg_amd import cg
    shp, enc, tb, cb = _stored()
    buf = np.frombuffer(tb, np.uint8)
    h = ctypes.c_void_p()
    rc = lib.cg_tables_import(buf.ctypes.data, buf.size, ctypes.byref(h))
    if rc == 0:      # a device was present: the handle is valid
        lib.cg_free(h)
    else:
        assert rc in (-2, -3), lib.cg_last_error()
    bad = np.frombuffer(_corrupt(tb, 0, "<I", 1), np.uint8)
    assert lib.cg_tables_import(bad.ctypes.data, bad.size, ctypes.byref(h)) == -5
