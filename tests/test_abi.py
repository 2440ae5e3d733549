"""The C ABI library: it loads, exports every function include/cg.h declares, and its
argument validation answers before touching a device (runs without a GPU)."""
import ctypes
import os
import re

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
                                          ("cg_tables_info", "TablesInfo"),
                                          ("cg_stream_stats", "StreamStats")])
def test_binding_structs_follow_the_header(cname, pyname):
    """The ctypes structures carry the header's fields in the header's order."""
    from kv_cache_compression_cg_amd import cg
    ours = [f for f, _ in getattr(cg, pyname)._fields_]
    assert ours == _struct_fields(cname)
