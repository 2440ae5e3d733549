"""cg_encode_noalloc (the encode for callers that cannot allocate) against cg_encode:
the same container bytes, on two calls in a row, the second with a smaller input, through
the C ABI; plus its refusals (too little capacity, scratch beyond its fixed array)."""
import os
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_cg_amd import configs, synth

pytestmark = pytest.mark.gpu

HEAVY = configs.GenSpec(rho=0.85, heavy_tail=True, outlier_frac=0.05, outlier_mult=30.0, seed=4)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def cg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_compression_cg_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from kv_cache_compression_cg_amd import cg as _cg
    _cg.load()
    return _cg


def _same_as_encode(cg, X, G, Tc, bins, H, rng, **kw):
    tab = cg.build_cdf(X, G, Tc, bins, H_kv=H, **kw)
    kb, ke = rng
    ref = cg.encode(tab, X, kb, ke).read().tobytes()
    buf = torch.full((len(ref) + 4096,), 0xAB, dtype=torch.uint8, device=X.device)
    h = cg.encode_noalloc(tab, X, buf, kb, ke)
    torch.cuda.synchronize()
    assert h["total_bytes"] == len(ref)
    got = buf[:len(ref)].cpu().numpy().tobytes()
    assert got == ref
    assert (buf[len(ref):] == 0xAB).all()      # nothing written past the container
    return tab, h


def test_noalloc_equals_encode_on_two_calls(cg):
    """First a larger encode, then a smaller one on the same fixed scratch: both equal
    cg_encode's container byte for byte (sinks and the outlier table in the first, 8-bit
    anchors and a chunk range in the second)."""
    _say("[noalloc] call 1: L=2 S=1200 C=136")
    X1 = synth.gen_custom(2, 1200, 136, HEAVY, device="cuda")
    _same_as_encode(cg, X1, 10, 300, (32, 8), 17, (0, 4), n_sink=4, outlier_ppm=3000)
    _say("[noalloc] call 2: L=1 S=500 C=72, chunks 1..3")
    X2 = synth.gen_custom(1, 500, 72, HEAVY, device="cuda")
    tab, h = _same_as_encode(cg, X2, 7, 128, (16,), 9, (1, 3), anchor_bits=8)
    assert h["chunk_begin"] == 1 and h["chunk_end"] == 3


def test_noalloc_refusals(cg):
    X = synth.gen_custom(1, 600, 64, HEAVY, device="cuda")
    tab = cg.build_cdf(X, 10, 200, (8,), H_kv=1)
    need = cg.encode(tab, X).nbytes
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(cg.CgError) as e:
        cg.encode_noalloc(tab, X, small)
    assert e.value.code == -1 and "capacity" in str(e.value)
    # the header of a refused call still names the size needed
    import ctypes
    hdr = cg.ContainerHeader()
    rc = cg.load().cg_encode_noalloc(tab.handle, X.data_ptr(), 0, tab.n_chunks, small.data_ptr(),
                                     small.numel(), None, ctypes.byref(hdr))
    assert rc == -1 and hdr.total_bytes == need
    # scratch beyond the fixed array: refused before any device work
    big = torch.zeros((4, 2, 16384, 1024), dtype=torch.float16, device="cuda")
    tb = cg.build_cdf(big, 10, 1536, (8,) * 4, H_kv=8)
    out = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(cg.CgError) as e:
        cg.encode_noalloc(tb, big, out)
    assert e.value.code == -1 and "scratch" in str(e.value)
