"""Streamed decode (cg_stream_decode) against the CPU oracle.

Every chunk is decoded from a container staged out of pinned host memory, at the
compression level chosen for it; the result must equal the oracle's decode of that
chunk at that level, bit for bit."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_compression_cg_amd import configs, streamed, synth

pytestmark = pytest.mark.gpu

LEVELS3 = [(32, 16, 8), (16, 8, 4), (8, 4, 2)]
HEAVY = configs.GenSpec(rho=0.85, heavy_tail=True, outlier_frac=0.05, outlier_mult=30.0, seed=3)


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


def _u16(t: torch.Tensor) -> np.ndarray:
    return np.ascontiguousarray(t.detach().cpu().view(torch.int16).numpy().view(np.uint16))


def _oracle_stream(Xh, H, G, Tc, level_bins, levels):
    """The oracle's decode of every chunk at its level (tokens of all chunks written)."""
    L, _, S, C = Xh.shape
    ref = np.zeros(Xh.shape, np.uint16)
    encs = {}
    for lv, bins in enumerate(level_bins):
        ks = [k for k in range(len(levels)) if levels[k] == lv]
        if not ks:
            continue
        shp = O.Shape.make(L, H, C // H, S, G, Tc, bins)
        tab = O.build_tables(shp, Xh)
        for k in ks:
            enc = O.encode(shp, Xh, tab, k, k + 1)
            encs[k] = enc
            O.decode(shp, tab, enc, out=ref)
    return ref, encs


# 1 to 3 slots: windows of one chunk; 5, 8, 16: windows of 2, 4 and 8 chunks decoded by
# one launch per level
@pytest.mark.parametrize("n_slots", [1, 2, 3, 5, 8, 16])
def test_streamed_forced_levels(cg, n_slots):
    L, S, H, d, G, Tc = 3, 4000, 2, 64, 10, 300
    _say("[streamed] L=%d S=%d C=%d G=%d Tc=%d slots=%d" % (L, S, H * d, G, Tc, n_slots))
    X = synth.gen_custom(L, S, H * d, HEAVY, device="cuda")
    n = -(-S // Tc)
    force = [0, 1, 2, 2, 1, 0, 0, 2, 1, 1, 2, 0, 1, 2][:n]
    prep = streamed.prepare(X, G, Tc, LEVELS3, H_kv=H, force_levels=force)
    assert list(prep.levels) == force
    out = torch.full_like(X, float("nan"))
    stats = streamed.run(prep, out, n_slots=n_slots)
    torch.cuda.synchronize()
    ref, encs = _oracle_stream(_u16(X), H, G, Tc, LEVELS3, force)
    assert np.array_equal(_u16(out), ref)
    # the staged containers are the oracle's, word for word
    for k, (_, blob, host) in enumerate(prep.items):
        assert np.array_equal(blob.payload(), encs[k].payload)
        assert np.array_equal(blob.offsets(), encs[k].offsets)
        assert np.array_equal(host.numpy()[:blob.nbytes], blob.read())
    assert stats["copied_bytes"] == prep.streamed_bytes
    assert stats["total_ms"] > 0 and stats["copy_ms"] > 0 and stats["decode_ms"] > 0


def test_streamed_with_text_fallback_chunks(cg):
    """Chunks at level TEXT (recomputed from text) are neither streamed nor decoded: their
    rows keep what the output held; every other chunk equals the oracle's decode."""
    L, S, H, d, G, Tc = 3, 2600, 2, 64, 10, 300
    _say("[streamed] text fallback L=%d S=%d" % (L, S))
    X = synth.gen_custom(L, S, H * d, HEAVY, device="cuda")
    n = -(-S // Tc)
    T = streamed.TEXT
    force = [0, T, 2, T, T, 1, 0, 2, T][:n]
    prep = streamed.prepare(X, G, Tc, LEVELS3, H_kv=H, force_levels=force)
    assert list(prep.levels) == force and len(prep.items) == sum(v != T for v in force)
    out = torch.full_like(X, float("nan"))
    streamed.run(prep, out, n_slots=3)
    torch.cuda.synchronize()
    got = _u16(out)
    ref, _ = _oracle_stream(_u16(X), H, G, Tc, LEVELS3, force)
    nan16 = _u16(torch.full((1,), float("nan"), dtype=torch.float16))[0]
    for k, lv in enumerate(force):
        rows = slice(k * Tc, min((k + 1) * Tc, S))
        if lv == T:
            assert (got[:, :, rows] == nan16).all(), k
        else:
            assert np.array_equal(got[:, :, rows], ref[:, :, rows]), k


def test_streamed_controller_levels(cg):
    """Levels from the closed-loop controller (with text fallback), streamed and decoded:
    the levels are control_levels' over the container sizes and the trace."""
    L, S, H, d, G, Tc = 3, 3000, 2, 64, 10, 250
    X = synth.gen_custom(L, S, H * d, HEAVY, device="cuda")
    ctl = streamed.ControllerConfig(slo_s=2e-4, prior_gbps=13.0, prefill_tok_per_s=2e6)
    prep = streamed.prepare(X, G, Tc, LEVELS3, H_kv=H, seed=6, controller=ctl)
    n = prep.sizes.shape[1]
    tokens = [min(Tc, S - k * Tc) for k in range(n)]
    exp = streamed.control_levels(prep.sizes, prep.bw_gbps, tokens, ctl)[0]
    assert np.array_equal(prep.levels, exp)
    _say("[streamed] controller levels %s" % list(prep.levels))
    out = torch.zeros_like(X)
    streamed.run(prep, out, n_slots=2)
    torch.cuda.synchronize()
    keep = [int(v) for v in prep.levels]
    ref, _ = _oracle_stream(_u16(X), H, G, Tc, LEVELS3, keep)
    assert np.array_equal(_u16(out), ref)


def test_streamed_chosen_levels_and_ragged_shape(cg):
    """Levels picked from the bandwidth trace; C = 72 (a partial lane block), G = 7."""
    L, S, H, d, G, Tc = 3, 2500, 9, 8, 7, 200
    _say("[streamed] chosen levels L=%d S=%d C=%d" % (L, S, H * d))
    X = synth.gen_custom(L, S, H * d, HEAVY, device="cuda")
    prep = streamed.prepare(X, G, Tc, LEVELS3, H_kv=H, seed=4)
    exp = streamed.choose_levels(prep.sizes, prep.bw_gbps)
    assert np.array_equal(prep.levels, exp)
    out = torch.zeros_like(X)
    streamed.run(prep, out, n_slots=2)
    torch.cuda.synchronize()
    ref, _ = _oracle_stream(_u16(X), H, G, Tc, LEVELS3, list(prep.levels))
    assert np.array_equal(_u16(out), ref)


@pytest.mark.timeout(900)
def test_streamed_131k_sampled(cg):
    """The 131K-token 70B-shaped cache streamed in full at the chosen levels.  Against
    the oracle: layers 0, 30 and 79 (one per bin tier) on channel block 7, for eight
    seeded chunks and the last one, at the chosen level and at both others."""
    w = configs.LLAMA3_70B_131K
    _say("[streamed] 131K: generating")
    X = synth.gen_kv(w, device="cuda")
    _say("[streamed] 131K: preparing %d chunks x %d levels" % (w.n_chunks, len(w.levels)))
    prep = streamed.prepare(X, w.group, w.chunk, w.levels, H_kv=w.H_kv, seed=0)
    out = torch.empty_like(X)
    _say("[streamed] 131K: streaming")
    stats = streamed.run(prep, out, n_slots=3)
    torch.cuda.synchronize()
    assert stats["copied_bytes"] == prep.streamed_bytes
    layers, c0, c1 = [0, 30, 79], 7 * 64, 8 * 64
    Xs = _u16(X[layers, :, :, c0:c1].contiguous())
    outs = _u16(out[layers, :, :, c0:c1].contiguous())
    rng = np.random.default_rng([0, 55])
    ks = sorted(set(int(k) for k in rng.choice(w.n_chunks - 1, 8, replace=False)) | {w.n_chunks - 1})
    Tc, S = w.chunk, w.S
    for lv, bins in enumerate(w.levels):
        _say("[streamed] 131K: oracle level %d" % lv)
        shp = O.Shape.make(3, 1, 64, S, w.group, Tc, [bins[l] for l in layers])
        tab = O.build_tables(shp, Xs)
        ex = prep.tables[lv].export()
        for name in ("lo", "w", "r"):
            assert np.array_equal(ex[name][layers][:, :, c0:c1].view(np.uint32),
                                  getattr(tab, name).view(np.uint32)), name
        assert np.array_equal(ex["freqs"][layers][:, :, c0:c1], tab.freqs)
        for k in ks:
            enc = O.encode(shp, Xs, tab, k, k + 1)
            ref = O.decode(shp, tab, enc)
            t0, t1 = k * Tc, min((k + 1) * Tc, S)
            if prep.levels[k] == lv:
                got = outs[:, :, t0:t1]
            else:
                blob = cg.encode(prep.tables[lv], X, k, k + 1)
                cg.decode(prep.tables[lv], blob, out)
                got = _u16(out[layers, :, t0:t1, c0:c1].contiguous())
                del blob
            assert np.array_equal(got, ref[:, :, t0:t1]), (lv, k)


def test_stream_decode_rejects_bad_items(cg):
    """Checked before anything is queued: mixed shapes, a slot too small, misaligned
    staging memory."""
    X = synth.gen_custom(2, 600, 64, HEAVY, device="cuda")
    Y = synth.gen_custom(2, 700, 64, HEAVY, device="cuda")
    tx = cg.build_cdf(X, 10, 200, (8, 4), H_kv=1)
    ty = cg.build_cdf(Y, 10, 200, (8, 4), H_kv=1)
    bx = cg.encode(tx, X, 0, 1)
    by = cg.encode(ty, Y, 0, 1)
    hx = torch.from_numpy(bx.read().copy())
    hy = torch.from_numpy(by.read().copy())
    slot = (max(bx.nbytes, by.nbytes) + 255) // 256 * 256
    staging = torch.empty(2 * slot + 256, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(X)
    cs, ds = torch.cuda.Stream(), torch.cuda.Stream()
    with pytest.raises(cg.CgError) as e:
        cg.stream_decode([(tx, bx, hx), (ty, by, hy)], staging[:2 * slot], 2, out, cs, ds)
    assert e.value.code == -1
    with pytest.raises(cg.CgError) as e:
        cg.stream_decode([(tx, bx, hx)], staging[:2 * 256], 2, out, cs, ds)
    assert e.value.code == -1 and "slot" in str(e.value)
    with pytest.raises(cg.CgError) as e:
        cg.stream_decode([(tx, bx, hx)], staging[16:16 + 2 * slot], 2, out, cs, ds)
    assert e.value.code == -1 and "aligned" in str(e.value)
    # and the valid call decodes chunk 0 as cg_decode does
    ref = cg.decode(tx, bx)
    got = torch.zeros_like(X)
    cg.stream_decode([(tx, bx, hx)], staging[:2 * slot], 2, got, cs, ds)
    torch.cuda.synchronize()
    assert torch.equal(got[:, :, :200].view(torch.int16), ref[:, :, :200].view(torch.int16))


@pytest.mark.parametrize("anchor_bits", [16, 8])
def test_stream_decode_writes_sink_tokens(cg, anchor_bits):
    """Tables with attention sinks (and fp16 or 8-bit anchors): the streamed decode of
    chunks 0 to 2 (the sinks span 0 and 1) equals cg_decode's, which the parity tests
    hold to the oracle."""
    X = synth.gen_custom(2, 600, 64, HEAVY, device="cuda")
    X[:, :, 1:12] = 2000.0
    tab = cg.build_cdf(X, 5, 8, (8, 4), H_kv=1, n_sink=12, anchor_bits=anchor_bits)
    blobs = [cg.encode(tab, X, k, k + 1) for k in range(3)]
    hosts = [torch.from_numpy(b.read().copy()) for b in blobs]
    slot = (max(b.nbytes for b in blobs) + 255) // 256 * 256
    staging = torch.empty(2 * slot, dtype=torch.uint8, device="cuda")
    got = torch.zeros_like(X)
    cs, ds = torch.cuda.Stream(), torch.cuda.Stream()
    cg.stream_decode([(tab, b, h) for b, h in zip(blobs, hosts)], staging, 2, got, cs, ds)
    torch.cuda.synchronize()
    ref = torch.zeros_like(X)
    for b in blobs:
        cg.decode(tab, b, ref)
    torch.cuda.synchronize()
    assert torch.equal(got[:, :, :24].view(torch.int16), ref[:, :, :24].view(torch.int16))
    assert torch.equal(got[:, :, :12].view(torch.int16), X[:, :, :12].view(torch.int16))


@pytest.mark.parametrize("n_slots", [2, 7, 16, 64])
def test_stream_decode_multi_chunk_items(cg, n_slots):
    """Items whose containers hold one to 25 chunks, under three sets of tables (one with
    sinks and an outlier table, one with 8-bit anchors), in windows of one to 32 items:
    a window can hold more chunks than one launch takes and tables of both anchor widths.
    The result equals cg_decode of every container, which the parity tests hold to the
    oracle."""
    L, S, C, G, Tc = 2, 5000, 128, 10, 100
    _say("[streamed] multi-chunk items L=%d S=%d C=%d Tc=%d slots=%d" % (L, S, C, Tc, n_slots))
    X = synth.gen_custom(L, S, C, HEAVY, device="cuda")
    ta = cg.build_cdf(X, G, Tc, (16, 8), H_kv=2, n_sink=30, outlier_ppm=2000)
    tb = cg.build_cdf(X, G, Tc, (8, 4), H_kv=2, n_sink=30)
    tc = cg.build_cdf(X, G, Tc, (8, 4), H_kv=2, anchor_bits=8)
    n = -(-S // Tc)
    bounds, k = [], 0
    for step in (3, 1, 2, 3, 3, 1, 2, 3, 3, 2, 2):
        bounds.append((k, k + step))
        k += step
    bounds.append((k, n))
    tabs = [(tb, ta, tc)[i % 3] for i in range(len(bounds))]
    blobs = [cg.encode(t, X, a, b) for t, (a, b) in zip(tabs, bounds)]
    hosts = [torch.empty(b.nbytes, dtype=torch.uint8, pin_memory=True) for b in blobs]
    for b, h in zip(blobs, hosts):
        b.read_into(h)
    slot = (max(b.nbytes for b in blobs) + 255) // 256 * 256
    staging = torch.empty(n_slots * slot, dtype=torch.uint8, device="cuda")
    got = torch.full_like(X, float("nan"))
    cs, ds = torch.cuda.Stream(), torch.cuda.Stream()
    stats = cg.stream_decode(list(zip(tabs, blobs, hosts)), staging, n_slots, got, cs, ds,
                             wait=True)
    torch.cuda.synchronize()
    ref = torch.full_like(X, float("nan"))
    for t, b in zip(tabs, blobs):
        cg.decode(t, b, ref)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert stats["copied_bytes"] == sum(b.nbytes for b in blobs)
    assert stats["decode_ms"] > 0
