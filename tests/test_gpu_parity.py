"""GPU library (through the C ABI) against the CPU oracle, on the same seeded inputs.

Bar: bit-exact tables (lo / w / r bits, frequencies), symbols, container (offsets,
anchors, payload words) and decoded fp16 output, plus the unfused symbol path."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_compression_cg_amd import configs, synth

pytestmark = pytest.mark.gpu


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


def _gen(L, S, C, gen, device="cuda"):
    return synth.gen_custom(L, S, C, gen, device=device)


GAUSS = configs.GenSpec(rho=0.9, heavy_tail=False, outlier_frac=0.02, outlier_mult=20.0, seed=0)
HEAVY = configs.GenSpec(rho=0.85, heavy_tail=True, outlier_frac=0.05, outlier_mult=30.0, seed=1)


def full_parity(cg, X, H, G, Tc, bins, chunk_range=None, label="", bins_v=None, n_sink=0,
                anchor_bits=16, outlier_ppm=0, X_enc=None):
    """Runs both sides on the same cache and compares every product of the path: the
    stored tables and the whole container byte for byte, symbols, the fused and the
    unfused decode; then a decode from the oracle's stored bytes imported into the
    library.  X_enc: another cache of the same shape to encode with X's tables."""
    L, _, S, C = X.shape
    _say("[parity] %s L=%d S=%d C=%d G=%d Tc=%d bins=%s bins_v=%s sinks=%d anchors=%d ppm=%d"
         % (label, L, S, C, G, Tc, list(bins), None if bins_v is None else list(bins_v), n_sink,
            anchor_bits, outlier_ppm))
    Xh = _u16(X)
    Xe = X if X_enc is None else X_enc
    Xeh = Xh if X_enc is None else _u16(X_enc)
    shp = O.Shape.make(L, H, C // H, S, G, Tc, bins, bins_v=bins_v, n_sink=n_sink,
                       anchor_bits=anchor_bits, outlier_ppm=outlier_ppm)
    tab_o = O.build_tables(shp, Xh)
    kb, ke = chunk_range if chunk_range else (0, shp.n_chunks)
    enc_o = O.encode(shp, Xeh, tab_o, kb, ke)

    tab = cg.build_cdf(X, G, Tc, bins, H_kv=H, bins_v=bins_v, n_sink=n_sink,
                       anchor_bits=anchor_bits, outlier_ppm=outlier_ppm)
    assert tab.stored_bytes == O.table_bytes(shp)
    ex = tab.export()
    for name in ("lo", "w", "r"):
        assert np.array_equal(ex[name].view(np.uint32), getattr(tab_o, name).view(np.uint32)), name
    assert np.array_equal(ex["freqs"], tab_o.freqs)
    tb = tab.serialize()
    assert tb == O.tables_bytes(shp, tab_o)

    sym = cg.quantize(tab, Xe, kb, ke)
    t0, t1 = kb * Tc, min(ke * Tc, S)
    sym_o = O.quantize(shp, O.snap_anchors(shp, Xeh, tab_o), tab_o.lo, tab_o.r, t0, t1)
    assert np.array_equal(sym.cpu().numpy()[:, :, t0:t1], sym_o[:, :, t0:t1])

    blob = cg.encode(tab, Xe, kb, ke)
    assert np.array_equal(blob.offsets(), enc_o.offsets)
    assert np.array_equal(blob.anchors(), enc_o.anchors)
    assert np.array_equal(blob.payload(), enc_o.payload)
    assert blob.header["n_outliers"] == enc_o.n_outliers and blob.header["clamped"] == enc_o.clamped
    cb = O.container_bytes(shp, enc_o)
    assert blob.read().tobytes() == cb

    nan = float("nan")
    out = torch.full_like(X, nan)
    cg.decode(tab, blob, out)
    ref = O.decode(shp, tab_o, enc_o, out=_u16(out))
    torch.cuda.synchronize()
    assert np.array_equal(_u16(out), ref)

    dsym = cg.decode_symbols(tab, blob)
    assert np.array_equal(dsym.cpu().numpy()[:, :, t0:t1], sym_o[:, :, t0:t1])
    out2 = torch.full_like(X, nan)
    cg.dequantize(tab, blob, dsym, out2)
    assert np.array_equal(_u16(out2), _u16(out))

    # a receiver that holds only the stored bytes (written by the oracle)
    tab_i = cg.tables_import(O.tables_bytes(shp, tab_o), device=X.device)
    blob_i = cg.blob_import(tab_i, cb)
    out3 = torch.full_like(X, nan)
    cg.decode(tab_i, blob_i, out3)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(out3), _u16(out))
    return tab, blob, tab_o, enc_o


def test_tiny_workload(cg):
    w = configs.TINY
    X = synth.gen_kv(w, device="cuda")
    full_parity(cg, X, w.H_kv, w.group, w.chunk, w.bins, label="tiny")


def test_several_tiles_ragged_tail_odd_bins(cg):
    X = _gen(3, 1000, 192, HEAVY)
    full_parity(cg, X, 3, 7, 300, (2, 13, 32), label="ragged")


def test_partial_lane_block_and_chunk_range(cg):
    X = _gen(2, 700, 72, GAUSS)
    full_parity(cg, X, 9, 10, 256, (8, 5), label="C=72")
    full_parity(cg, X, 9, 10, 256, (8, 5), chunk_range=(1, 3), label="C=72 chunks 1..3")


def test_llama7b_shape_two_layers(cg):
    w = configs.LLAMA7B
    X = synth.gen_kv(w, device="cuda", layers=[0, 31])
    full_parity(cg, X, w.H_kv, w.group, w.chunk, (w.bins[0], w.bins[31]), label="7B layers 0,31")


@pytest.mark.parametrize("G,Tc,rng", [(7, 150, None), (10, 90, None), (10, 90, (3, 12)),
                                      (10, 240, None), (10, 60, None), (7, 70, None),
                                      (10, 60, (2, 30)), (10, 125, None)])
def test_paired_chunks(cg, G, Tc, rng):
    """Many chunks per (row, channel block), so a wavefront decodes two chunks in
    lockstep: equal and unequal chunk lengths, a partial lane block (C = 136), full and
    partial anchor groups, and a chunk range that starts mid-cache.  Chunk counts 9 to
    34 per (row, block) give blocks of 8 chunks with a partial last set, G = 7 (no
    unrolled groups) and a wavefront left with one chunk."""
    X = _gen(2, 2000, 136, HEAVY)
    full_parity(cg, X, 17, G, Tc, (32, 8), chunk_range=rng, label="paired")


def test_keys_finer_than_values(cg):
    """Separate bin counts for the V rows (keys kept finer than values): K 32 / 16 / 8,
    V 16 / 4 / 2 over three layers, a ragged last chunk, G = 7, a partial lane block."""
    X = _gen(3, 1000, 136, HEAVY)
    tab, *_ = full_parity(cg, X, 17, 7, 300, (32, 16, 8), label="K/V bins", bins_v=(16, 4, 2))
    assert tab.row_bins == (32, 16, 16, 4, 8, 2)


@pytest.mark.parametrize("S,G,Tc", [(5, 10, 5), (37, 10, 37), (41, 4, 20), (64, 1, 16),
                                    (130, 10, 16384)])
def test_edge_shapes(cg, S, G, Tc):
    X = _gen(2, S, 64, HEAVY)
    full_parity(cg, X, 1, G, Tc, (2, 32), label="edge")


def test_constant_and_signed_zero_channels(cg):
    X = _gen(1, 300, 128, GAUSS)
    X[0, 0, :, 0] = 1.5                     # constant channel
    X[0, 1, :, 1] = 0.0                     # all +0
    X[0, 1, 5::3, 2] = -0.0                 # mixes -0 and +0
    X[0, 1, :, 2] = torch.where(torch.arange(300, device="cuda") % 3 == 0,
                                torch.tensor(0.0, dtype=torch.float16, device="cuda"),
                                torch.tensor(-0.0, dtype=torch.float16, device="cuda"))
    tab, *_ = full_parity(cg, X, 2, 10, 128, (4,), label="constant/zero")
    ex = tab.export()
    assert ex["w"][0, 0, 0] == 0 and ex["lo"][0, 1, 2].view(np.uint32) == 0


@pytest.mark.parametrize("ppm,ab", [(0, 16), (1000, 16), (1000, 8)])
def test_zero_width_grids_with_off_grid_elements(cg, ppm, ab):
    """Tables from a cache with constant channels (zero-width grids: only lo is on them)
    coding a cache where those channels vary: every such delta is off its grid, counted in
    the header or stored as an outlier entry, in full and partial groups."""
    X = _gen(2, 700, 128, GAUSS)
    X[0, 0, :, 3] = 1.5                  # constant: zero-width grid
    X[1, 1, :, 64] = -0.25               # another, in the second channel block
    Xe = X.clone()
    Xe[0, 0, 100:110, 3] = 2.0           # off the grid in the encoded cache
    Xe[1, 1, 5::7, 64] = 0.5
    Xe[1, 1, 690:, 64] = -1.0            # in the short last group of the last chunk
    full_parity(cg, X, 2, 10, 256, (8, 16), label="zero-width off-grid", X_enc=Xe,
                outlier_ppm=ppm, anchor_bits=ab)


def test_nonfinite_input_is_rejected(cg):
    X = _gen(1, 64, 64, GAUSS)
    X[0, 1, 33, 7] = float("inf")
    with pytest.raises(cg.CgError) as e:
        cg.build_cdf(X, 10, 64, (8,), H_kv=1)
    assert e.value.code == -4


# fp16 bits of +Inf, -Inf, a quiet NaN, a signalling NaN and a negative NaN, each placed
# at an anchor, a coded token, a sink token and the last token, in even and odd channels
# (the low and high half of a 32-bit word)
@pytest.mark.parametrize("bits", [0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFFFF])
@pytest.mark.parametrize("t,c", [(0, 0), (20, 5), (33, 7), (2, 64), (299, 127), (151, 130)])
def test_every_nonfinite_form_is_rejected(cg, bits, t, c):
    X = _gen(1, 300, 136, GAUSS)
    X.view(torch.int16)[0, 1, t, c] = bits - 0x10000 if bits >= 0x8000 else bits
    with pytest.raises(cg.CgError) as e:
        cg.build_cdf(X, 10, 128, (8,), H_kv=1, n_sink=4)
    assert e.value.code == -4


def test_mismatched_container_is_rejected(cg):
    X = _gen(1, 64, 64, GAUSS)
    t1 = cg.build_cdf(X, 10, 64, (8,), H_kv=1)
    t2 = cg.build_cdf(X, 8, 64, (8,), H_kv=1)
    b = cg.encode(t1, X)
    with pytest.raises(cg.CgError) as e:
        cg.decode(t2, b)
    assert e.value.code == -5


@pytest.mark.parametrize("S,Tc", [(500, 128), (2000, 100)])
def test_damaged_container_decodes_without_fault(cg, S, Tc):
    """Damaged payload words and offsets: reads stay inside the container, with one
    wavefront per block (4 chunks) and four (20 chunks)."""
    _say("[damaged] S=%d Tc=%d" % (S, Tc))
    X = _gen(2, S, 128, HEAVY)
    tab = cg.build_cdf(X, 10, Tc, (16, 4), H_kv=2)
    blob = cg.encode(tab, X)
    raw = torch.from_numpy(blob.read().copy()).cuda()
    h = blob.header
    g = torch.Generator().manual_seed(0)
    pl0, pl1 = h["payload_offset"], h["payload_offset"] + 2 * h["payload_words"]
    idx = torch.randint(pl0, pl1, (200,), generator=g)
    raw[idx.cuda()] ^= 0x5A
    offs = raw[h["offsets_offset"]:h["offsets_offset"] + 8 * (h["n_groups"] + 1)].view(torch.int64)
    offs[3] = 1 << 40
    offs[5] = 0
    out = cg.decode(tab, blob, container=raw)
    torch.cuda.synchronize()
    assert out.shape == X.shape
    # anchors are untouched by the damage
    a = out[:, :, ::10][:, :, :13]
    assert torch.equal(a.view(torch.int16), X[:, :, ::10][:, :, :13].view(torch.int16))


def test_damaged_outlier_sections_decode_without_fault(cg):
    """A container's outlier sections damaged: changed values land only on their entries'
    elements; garbage offsets and keys still decode (contiguous and paged) with every
    write inside the output."""
    L, S, C, G, Tc = 2, 900, 136, 10, 120
    X = _gen(L, S, C, HEAVY)
    tab = cg.build_cdf(X, G, Tc, (32, 8), H_kv=17, outlier_ppm=20000)
    blob = cg.encode(tab, X)
    h = blob.header
    n = h["n_outliers"]
    assert n > 1000
    ref = cg.decode(tab, blob)
    raw0 = blob.read().copy()
    # values changed: the decode differs from the reference exactly at the entries
    raw = torch.from_numpy(raw0.copy()).cuda()
    vals = raw[h["outlier_values_offset"]:h["outlier_values_offset"] + 2 * n].view(torch.int16)
    vals ^= 0x0101
    out = cg.decode(tab, blob, container=raw)
    torch.cuda.synchronize()
    offs = raw0[h["outliers_offset"]:h["outliers_offset"] + 8 * (h["n_groups"] + 1)].view(np.uint64)
    keys = raw0[h["outlier_keys_offset"]:h["outlier_keys_offset"] + 4 * n].view(np.uint32)
    NB = -(-C // 64)
    mask = np.zeros((L, 2, S, C), bool)
    for gidx in range(h["n_groups"]):
        b, tmp = gidx % NB, gidx // NB
        row, k = tmp % (2 * L), tmp // (2 * L)
        for e in range(int(offs[gidx]), int(offs[gidx + 1])):
            u, c = int(keys[e]) >> 6, b * 64 + (int(keys[e]) & 63)
            mask[row // 2, row % 2, k * Tc + u, c] = True
    diff = _u16(out) != _u16(ref)
    assert np.array_equal(diff, mask)
    # offsets and keys garbage: no fault, and the output keeps its shape
    g = torch.Generator().manual_seed(1)
    raw = torch.from_numpy(raw0.copy()).cuda()
    o = raw[h["outliers_offset"]:h["outliers_offset"] + 8 * (h["n_groups"] + 1)].view(torch.int64)
    o[3], o[4], o[7] = 1 << 40, 0, n + 5
    kk = raw[h["outlier_keys_offset"]:h["outlier_keys_offset"] + 4 * n].view(torch.int32)
    sel = torch.randint(0, n, (300,), generator=g).cuda()
    kk[sel] = torch.randint(-2 ** 31, 2 ** 31 - 1, (300,), generator=g, dtype=torch.int64).to(torch.int32).cuda()
    _say("[damaged outliers] n=%d" % n)
    out = cg.decode(tab, blob, container=raw)
    P = 16
    nb = -(-S // P)
    pages = torch.zeros((L, 2, nb, P, C), dtype=torch.float16, device="cuda")
    cg.decode_paged(tab, blob, pages, torch.arange(nb, dtype=torch.int32, device="cuda"),
                    container=raw)
    torch.cuda.synchronize()
    assert out.shape == X.shape


def test_reconstruction_bound_at_scale(cg):
    """8B-shaped slice, GPU only: anchors exact, every other element within half a bin
    plus fp16 rounding (a property that holds at any size)."""
    w = configs.LLAMA3_8B
    X = synth.gen_kv(w, device="cuda", layers=[0, 20])
    bins = (w.bins[0], w.bins[20])
    tab = cg.build_cdf(X, w.group, w.chunk, bins, H_kv=w.H_kv)
    blob = cg.encode(tab, X)
    out = cg.decode(tab, blob)
    wv = torch.from_numpy(tab.export()["w"]).cuda().double()
    lo = torch.from_numpy(tab.export()["lo"]).cuda().double()
    xs, ys = X.double(), out.double()
    t = torch.arange(w.S, device="cuda")
    anchor = ((t % w.chunk) % w.group) == 0
    assert torch.equal(out[:, :, anchor].view(torch.int16), X[:, :, anchor].view(torch.int16))
    err = (xs - ys).abs()[:, :, ~anchor]
    ulp = torch.from_numpy(np.spacing(np.abs(out.cpu().numpy()).astype(np.float16))
                           .astype(np.float64)).cuda()[:, :, ~anchor]
    wb = wv[:, :, None, :]
    tol = wb / 2 * (1 + 2 ** -20) + ulp / 2 + 2 ** -22 * (
        xs.abs()[:, :, ~anchor] + ys.abs()[:, :, ~anchor] + 2 * lo.abs()[:, :, None, :] + 64 * wb)
    assert bool((err <= tol).all())


def _gather_pages(pages, bt, S):
    """[L, 2, num_pages, P, C] pages read through the block table back to [L, 2, S, C]."""
    L, _, _, P, C = pages.shape
    nb = -(-S // P)
    return pages[:, :, bt[:nb].long()].reshape(L, 2, nb * P, C)[:, :, :S]


@pytest.mark.parametrize("S,Tc,P,rng", [(1000, 300, 16, None), (2000, 90, 64, None),
                                        (700, 256, 1, None), (2000, 60, 16, (2, 30))])
def test_paged_output_matches_oracle(cg, S, Tc, P, rng):
    """cg_decode_paged through a shuffled block table equals the oracle's decode bit for
    bit; pages no block maps to, and rows of the blob's other chunks, stay untouched."""
    _say("[paged] S=%d Tc=%d P=%d chunks=%s" % (S, Tc, P, rng))
    L, C, H, G, bins = 2, 136, 17, 10, (32, 8)
    X = _gen(L, S, C, HEAVY)
    n_chunks = -(-S // Tc)
    kb, ke = rng if rng else (0, n_chunks)
    tab = cg.build_cdf(X, G, Tc, bins, H_kv=H)
    blob = cg.encode(tab, X, kb, ke)
    nb = -(-S // P)
    n_pages = nb + 5
    gen = torch.Generator().manual_seed(S + P)
    bt = torch.randperm(n_pages, generator=gen)[:nb].to(torch.int32).cuda()
    pages = torch.full((L, 2, n_pages, P, C), float("nan"), dtype=torch.float16, device="cuda")
    cg.decode_paged(tab, blob, pages, bt)
    torch.cuda.synchronize()
    Xh = _u16(X)
    shp = O.Shape.make(L, H, C // H, S, G, Tc, bins)
    tab_o = O.build_tables(shp, Xh)
    enc_o = O.encode(shp, Xh, tab_o, kb, ke)
    nan16 = _u16(torch.full((1,), float("nan"), dtype=torch.float16))[0]
    ref = O.decode(shp, tab_o, enc_o, out=np.full(Xh.shape, nan16, np.uint16))
    got = _u16(_gather_pages(pages, bt, S))
    assert np.array_equal(got, ref)
    unused = sorted(set(range(n_pages)) - set(bt.cpu().tolist()))
    assert (_u16(pages[:, :, unused]) == nan16).all()


def test_paged_output_skips_invalid_page_ids(cg):
    """Blocks mapped to a negative page id or one past the pool write nothing."""
    L, S, C, Tc, P = 2, 600, 64, 200, 16
    X = _gen(L, S, C, GAUSS)
    tab = cg.build_cdf(X, 10, Tc, (8, 8), H_kv=1)
    blob = cg.encode(tab, X)
    nb = -(-S // P)
    bt = torch.arange(nb, dtype=torch.int32)
    bad = [3, 17, 30]
    bt[3], bt[17], bt[30] = -1, nb, 1 << 30
    bt = bt.cuda()
    pages = torch.full((L, 2, nb, P, C), float("nan"), dtype=torch.float16, device="cuda")
    cg.decode_paged(tab, blob, pages, bt)
    ref = cg.decode(tab, blob)
    torch.cuda.synchronize()
    nan16 = _u16(torch.full((1,), float("nan"), dtype=torch.float16))[0]
    got = _u16(pages)
    want = _u16(ref)
    for j in range(nb):
        rows = slice(j * P, min((j + 1) * P, S))
        if j in bad:
            assert (got[:, :, j] == nan16).all(), j    # page j belongs to no valid block
        else:
            n = rows.stop - rows.start
            assert np.array_equal(got[:, :, j, :n], want[:, :, rows]), j
    bt12 = torch.zeros(-(-S // 12), dtype=torch.int32, device="cuda")
    with pytest.raises(cg.CgError):        # 12 tokens per page: not a power of two
        cg.decode_paged(tab, blob, pages[:, :, :, :12].contiguous(), bt12)
    # a pool that fits 32-bit offsets only without the page past its end is refused before
    # any memory is touched (2^21 pages of 16 rows of 64 channels: 2^32 bytes)
    lib = cg.load()
    rc = lib.cg_decode_paged(tab.handle, blob.handle, None, pages.data_ptr(), bt.data_ptr(),
                             P, 1 << 21, None)
    assert rc != 0 and b"too large" in lib.cg_last_error()


@pytest.mark.parametrize("n_sink,G,Tc,rng", [(4, 10, 300, None), (40, 5, 32, None),
                                             (40, 5, 32, (1, 5)), (4, 10, 300, (1, 3)),
                                             (2000, 10, 300, None)])
def test_attention_sinks(cg, n_sink, G, Tc, rng):
    """Sink tokens ("Guide to CacheGen", Best Practices) planted with large values: tables,
    container and decode equal the oracle's (the sinks out of ranges and histograms, and
    written back exactly); sinks spread over two chunks (Tc = 32), chunk ranges that
    start after the sinks or among them; a partial lane block (C = 72); n_sink above S
    (every token a sink: the tables see no token at all).  Also through the paged
    output."""
    L, S, C, H, bins = 2, 1000, 72, 9, (16, 4)
    X = _gen(L, S, C, HEAVY)
    X[:, :, 1:n_sink:3] = 3000.0
    tab, blob, tab_o, enc_o = full_parity(cg, X, H, G, Tc, bins, chunk_range=rng,
                                          label="sinks %d" % n_sink, n_sink=n_sink)
    kb, ke = rng if rng else (0, -(-S // Tc))
    P = 16
    nb = -(-S // P)
    bt = torch.randperm(nb, generator=torch.Generator().manual_seed(n_sink)).to(torch.int32).cuda()
    pages = torch.full((L, 2, nb, P, C), float("nan"), dtype=torch.float16, device="cuda")
    cg.decode_paged(tab, blob, pages, bt)
    torch.cuda.synchronize()
    shp = O.Shape.make(L, H, C // H, S, G, Tc, bins, n_sink=n_sink)
    nan16 = _u16(torch.full((1,), float("nan"), dtype=torch.float16))[0]
    ref = O.decode(shp, tab_o, enc_o, out=np.full((L, 2, S, C), nan16, np.uint16))
    assert np.array_equal(_u16(_gather_pages(pages, bt, S)), ref)
    t_end = min(ke * Tc, n_sink)
    if kb * Tc < t_end:
        assert np.array_equal(ref[:, :, kb * Tc:t_end], _u16(X)[:, :, kb * Tc:t_end])


def test_extreme_outlier_channel(cg):
    """One channel scaled by 500 (clamped to the fp16 range) next to regular ones, in a
    partial lane block: tables, container and decode equal the oracle's."""
    X = _gen(2, 900, 72, HEAVY)
    X[..., 37] = (X[..., 37].float() * 500.0).clamp(-65504, 65504).half()
    full_parity(cg, X, 9, 10, 300, (16, 4), label="outlier x500")


@pytest.mark.parametrize("S,C,G,Tc,rng,n_sink", [(1000, 192, 10, 300, None, 0),
                                                (700, 72, 7, 256, (1, 3), 0),
                                                (2000, 136, 10, 90, None, 4),
                                                (2000, 136, 10, 60, (2, 30), 0)])
def test_8bit_anchors(cg, S, C, G, Tc, rng, n_sink):
    """Anchors stored as 8-bit codes on a per-channel grid ("Guide to CacheGen", Solution
    pillar 2): tables, codes, payload, decode (fused and unfused) and paged decode equal
    the oracle's; several tiles, a partial lane block, paired chunks, chunk ranges and
    sinks."""
    L, H, bins = 2, (3 if C == 192 else 9 if C == 72 else 17), (32, 8)
    X = _gen(L, S, C, HEAVY)
    tab, blob, tab_o, enc_o = full_parity(cg, X, H, G, Tc, bins, chunk_range=rng,
                                          label="8-bit anchors", n_sink=n_sink, anchor_bits=8)
    assert blob.anchors().dtype == np.uint8
    P = 16
    nb = -(-S // P)
    bt = torch.randperm(nb, generator=torch.Generator().manual_seed(S)).to(torch.int32).cuda()
    pages = torch.full((L, 2, nb, P, C), float("nan"), dtype=torch.float16, device="cuda")
    cg.decode_paged(tab, blob, pages, bt)
    torch.cuda.synchronize()
    shp = O.Shape.make(L, H, C // H, S, G, Tc, bins, n_sink=n_sink, anchor_bits=8)
    nan16 = _u16(torch.full((1,), float("nan"), dtype=torch.float16))[0]
    ref = O.decode(shp, tab_o, enc_o, out=np.full((L, 2, S, C), nan16, np.uint16))
    assert np.array_equal(_u16(_gather_pages(pages, bt, S)), ref)


def test_format_variants_together(cg):
    """Keys finer than values, attention sinks and 8-bit anchors at once, on paired
    chunks and a partial lane block: everything equals the oracle's."""
    X = _gen(3, 1500, 136, HEAVY)
    X[:, :, 1:4] = 1500.0
    full_parity(cg, X, 17, 10, 100, (32, 16, 8), bins_v=(16, 8, 4), n_sink=4,
                anchor_bits=8, label="bins_v + sinks + 8-bit anchors")


@pytest.mark.parametrize("S,C,G,Tc,rng,ppm,n_sink,anchor_bits",
                         [(1000, 192, 10, 300, None, 2000, 0, 16),
                          (1000, 72, 7, 256, (1, 3), 20000, 0, 16),
                          (2000, 136, 10, 90, None, 5000, 4, 16),
                          (2000, 136, 10, 60, (2, 30), 1000, 0, 8),
                          (700, 64, 10, 700, None, 250000, 9, 8),
                          (300, 64, 1, 100, None, 50000, 0, 16)])
def test_outlier_table(cg, S, C, G, Tc, rng, ppm, n_sink, anchor_bits):
    """Sparse outlier table ("Guide to CacheGen", Solution pillar 3): clipped ranges,
    tables, every byte of the container (entries included) and the decode (fused,
    unfused, imported, paged) equal the oracle's; several tiles, partial lane blocks,
    paired chunks, chunk ranges, sinks, 8-bit anchors, G = 1 (no coded token)."""
    L, bins = 2, (32, 8)
    H = {192: 3, 72: 9, 136: 17, 64: 1}[C]
    X = _gen(L, S, C, HEAVY)
    tab, blob, tab_o, enc_o = full_parity(cg, X, H, G, Tc, bins, chunk_range=rng, label="outliers",
                                          n_sink=n_sink, anchor_bits=anchor_bits, outlier_ppm=ppm)
    if G > 1:
        assert enc_o.n_outliers > 0
    P = 16
    nb = -(-S // P)
    bt = torch.randperm(nb, generator=torch.Generator().manual_seed(S + ppm)).to(torch.int32).cuda()
    pages = torch.full((L, 2, nb, P, C), float("nan"), dtype=torch.float16, device="cuda")
    cg.decode_paged(tab, blob, pages, bt)
    torch.cuda.synchronize()
    shp = O.Shape.make(L, H, C // H, S, G, Tc, bins, n_sink=n_sink, anchor_bits=anchor_bits,
                       outlier_ppm=ppm)
    nan16 = _u16(torch.full((1,), float("nan"), dtype=torch.float16))[0]
    ref = O.decode(shp, tab_o, enc_o, out=np.full((L, 2, S, C), nan16, np.uint16))
    assert np.array_equal(_u16(_gather_pages(pages, bt, S)), ref)


@pytest.mark.parametrize("P,anchor_bits", [(1, 16), (64, 8), (256, 16)])
def test_outlier_entries_into_pages(cg, P, anchor_bits):
    """A container with outlier entries decoded into pages of 1, 64 and 256 tokens (the
    decoding wavefronts write the entries through the block table) equals its contiguous
    decode; the block mapped to an invalid page id writes nothing."""
    L, S, C, G, Tc = 2, 900, 136, 10, 120
    X = _gen(L, S, C, HEAVY)
    tab = cg.build_cdf(X, G, Tc, (32, 8), H_kv=17, anchor_bits=anchor_bits, outlier_ppm=20000)
    blob = cg.encode(tab, X)
    assert blob.header["n_outliers"] > 0
    ref = cg.decode(tab, blob)
    nb = -(-S // P)
    bt = torch.randperm(nb, generator=torch.Generator().manual_seed(P)).to(torch.int32)
    bad = nb // 2
    bt[bad] = -1
    bt = bt.cuda()
    pages = torch.full((L, 2, nb, P, C), float("nan"), dtype=torch.float16, device="cuda")
    _say("[paged outliers] P=%d anchor_bits=%d entries=%d" % (P, anchor_bits, blob.header["n_outliers"]))
    cg.decode_paged(tab, blob, pages, bt)
    torch.cuda.synchronize()
    got = _u16(pages)
    want = _u16(ref)
    btc = bt.cpu().tolist()
    nan16 = _u16(torch.full((1,), float("nan"), dtype=torch.float16))[0]
    for j in range(nb):
        n = min(P, S - j * P)
        if j == bad:
            continue
        assert np.array_equal(got[:, :, btc[j], :n], want[:, :, j * P:j * P + n]), j
    unused = sorted(set(range(nb)) - set(x for x in btc if x >= 0))
    assert (got[:, :, unused] == nan16).all()


@pytest.mark.parametrize("ppm,anchor_bits", [(0, 16), (20000, 16), (0, 8), (20000, 8)])
def test_extreme_finite_values(cg, ppm, anchor_bits):
    """Channels that span the whole fp16 range (+-65504, whose deltas reach 131008 and
    whose decoded values can round to +-Inf), subnormals and signed zeros next to
    ordinary channels: tables, container and decodes equal the oracle's bit for bit."""
    L, S, C, G, Tc = 2, 500, 80, 10, 170
    X = _gen(L, S, C, HEAVY)
    g = torch.Generator().manual_seed(5)
    big = torch.tensor([65504.0, -65504.0, 0.0, -0.0], dtype=torch.float16)
    X[0, 0, :, 3] = big[torch.randint(0, 4, (S,), generator=g)].cuda()
    X[1, 1, :, 70] = big[torch.randint(0, 2, (S,), generator=g)].cuda()
    sub = torch.tensor([1, 2, 1023, 0x8001 - 0x10000, 0x83FF - 0x10000, 0], dtype=torch.int16)  # subnormals
    X[0, 1, :, 9] = sub[torch.randint(0, 6, (S,), generator=g)].cuda().view(torch.float16)
    X[1, 0, ::7, 40] = 65504.0
    X[1, 0, 3::11, 41] = -65504.0
    full_parity(cg, X, 8, G, Tc, (32, 4), label="extreme finite", anchor_bits=anchor_bits,
                outlier_ppm=ppm)


@pytest.mark.parametrize("ppm,anchor_bits", [(0, 16), (3000, 16), (0, 8), (3000, 8)])
def test_calibration_tables_on_a_cache_with_inf_and_nan(cg, ppm, anchor_bits):
    """Tables built from a finite cache code another that holds Inf and NaN (the tables'
    build rejects such a cache, the encode with calibration tables takes it): inside a
    group's deltas, as an anchor, and in a sink row; container and decode equal the
    oracle's bit for bit."""
    L, S, C, G, Tc = 2, 600, 72, 10, 200
    X = _gen(L, S, C, HEAVY)
    Y = X.clone()
    inf, nan = float("inf"), float("nan")
    Y[0, 0, 13, 3] = inf
    Y[0, 1, 27, 70] = -inf
    Y[1, 0, 45, 10] = nan
    Y[1, 1, 100, 40] = nan      # an anchor
    Y[0, 0, 210, 5] = inf       # an anchor
    Y[1, 0, 1, 7] = nan         # a sink row
    full_parity(cg, X, 9, G, Tc, (16, 8), label="inf / nan", n_sink=2,
                anchor_bits=anchor_bits, outlier_ppm=ppm, X_enc=Y)


@pytest.mark.parametrize("ppm,anchor_bits,n_sink", [(0, 16, 4), (3000, 16, 4), (0, 8, 4),
                                                    (3000, 8, 12)])
def test_another_cache_with_calibration_tables(cg, ppm, anchor_bits, n_sink):
    """Tables built from one cache code another of the same shape: the container holds
    the new cache's own sink rows, and the elements the tables' grids cannot hold are
    counted as clamped or, with the outlier table, stored exactly; container and decode
    equal the oracle's."""
    L, S, C, G, Tc = 2, 900, 72, 10, 300
    X = _gen(L, S, C, HEAVY)
    Y = _gen(L, S, C, configs.GenSpec(rho=0.8, heavy_tail=True, outlier_frac=0.05,
                                      outlier_mult=40.0, seed=9))
    Y[:, :, 1:n_sink] = 2500.0
    Y[0, 0, 300, 5] = 3000.0          # an anchor far outside its grid
    tab, blob, tab_o, enc_o = full_parity(cg, X, 9, G, Tc, (16, 4), label="other cache",
                                          n_sink=n_sink, anchor_bits=anchor_bits,
                                          outlier_ppm=ppm, X_enc=Y)
    out = cg.decode(tab, blob)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, :n_sink].view(torch.int16), Y[:, :, :n_sink].view(torch.int16))
    if ppm:
        assert enc_o.n_outliers > 0 and blob.header["clamped"] == 0
        assert out[0, 0, 300, 5].item() == 3000.0
    else:
        assert blob.header["clamped"] == enc_o.clamped > 0


def test_import_after_the_encoder_is_gone(cg):
    """Encode, copy the stored tables and container to host memory, free every handle of
    the encoder, import into new handles and decode: equal to the oracle's decode.  Then
    a streamed decode of per-chunk containers imported from bytes."""
    L, S, C, G, Tc, H, bins = 2, 1200, 136, 10, 300, 17, (16, 8)
    X = _gen(L, S, C, HEAVY)
    tab = cg.build_cdf(X, G, Tc, bins, H_kv=H, n_sink=4, outlier_ppm=3000)
    blob = cg.encode(tab, X)
    tb, cb = tab.serialize(), blob.read().tobytes()
    per_chunk = [cg.encode(tab, X, k, k + 1).read().tobytes() for k in range(4)]
    del blob, tab
    import gc
    gc.collect()
    torch.cuda.synchronize()
    tab2 = cg.tables_import(tb)
    blob2 = cg.blob_import(tab2, cb)
    out = cg.decode(tab2, blob2)
    Xh = _u16(X)
    shp = O.Shape.make(L, H, C // H, S, G, Tc, bins, n_sink=4, outlier_ppm=3000)
    tab_o = O.build_tables(shp, Xh)
    enc_o = O.encode(shp, Xh, tab_o)
    ref = O.decode(shp, tab_o, enc_o)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(out), ref)
    assert cb == O.container_bytes(shp, enc_o) and tb == O.tables_bytes(shp, tab_o)
    # streamed decode from imported per-chunk containers
    blobs = [cg.blob_import(tab2, b) for b in per_chunk]
    hosts = [torch.from_numpy(np.frombuffer(b, np.uint8).copy()).pin_memory() for b in per_chunk]
    slot = (max(b.nbytes for b in blobs) + 255) // 256 * 256
    staging = torch.empty(2 * slot, dtype=torch.uint8, device="cuda")
    out2 = torch.full_like(X, float("nan"))
    cs, ds = torch.cuda.Stream(), torch.cuda.Stream()
    cg.stream_decode([(tab2, b, h) for b, h in zip(blobs, hosts)], staging, 2, out2, cs, ds)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(out2), ref)


def test_imported_blob_must_match_its_tables(cg):
    X = _gen(1, 300, 64, GAUSS)
    t1 = cg.build_cdf(X, 10, 100, (8,), H_kv=1)
    t2 = cg.build_cdf(X, 10, 100, (8,), H_kv=1, outlier_ppm=1000)
    t3 = cg.build_cdf(X, 10, 100, (8,), H_kv=1, n_sink=4)
    cb = cg.encode(t1, X).read().tobytes()
    for t in (t2, t3):
        with pytest.raises(cg.CgError) as e:
            cg.blob_import(t, cb)
        assert e.value.code == -5
    with pytest.raises(cg.CgError) as e:
        cg.blob_import(t1, cb[:-2000])
    assert e.value.code == -5


def _sweep_cases(n=40, seed=2024):
    """Seeded random shapes and settings for the sweep below (small enough for the oracle
    to finish each in seconds): ragged chunk and group lengths, partial lane blocks, every
    bin count from 2 to 32, the format variants in every combination, chunk ranges."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        L = int(rng.integers(1, 4))
        H = int(rng.choice([1, 2, 3]))
        d = int(rng.choice([8, 24, 64, 72]))
        S = int(rng.integers(1, 1400))
        G = int(rng.integers(1, 17))
        Tc = int(rng.integers(1, 700))
        bins = tuple(int(b) for b in rng.integers(2, 33, size=L))
        bins_v = tuple(int(b) for b in rng.integers(2, 33, size=L)) if rng.random() < 0.3 else None
        n_sink = int(rng.choice([0, 0, 1, 4, 37]))
        anchor_bits = int(rng.choice([16, 16, 8]))
        ppm = int(rng.choice([0, 0, 300, 20000, 250000]))
        nk = -(-S // Tc)
        kb = int(rng.integers(0, nk))
        ke = int(rng.integers(kb + 1, nk + 1))
        rngc = (kb, ke) if rng.random() < 0.4 else None
        gen = HEAVY if rng.random() < 0.6 else GAUSS
        cases.append((i, L, H, d, S, G, Tc, bins, bins_v, n_sink, anchor_bits, ppm, rngc, gen))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "case%d" % c[0])
def test_seeded_sweep_of_shapes_and_settings(cg, case):
    """Every product of the path (tables, stored bytes, symbols, the whole container,
    fused / unfused / imported decodes) bit for bit against the oracle over seeded random
    shapes and settings."""
    i, L, H, d, S, G, Tc, bins, bins_v, n_sink, anchor_bits, ppm, rngc, gen = case
    X = _gen(L, S, H * d, gen)
    full_parity(cg, X, H, G, Tc, bins, chunk_range=rngc, label="sweep %d" % i, bins_v=bins_v,
                n_sink=n_sink, anchor_bits=anchor_bits, outlier_ppm=ppm)


def _calibration_cases(n=60, seed=12):
    """Sweep cases whose cache is coded with tables built on another one: its own seeded
    generator, and in some cases a few Inf, NaN, +-65504 or zero elements."""
    rng = np.random.default_rng(seed + 1000)
    out = []
    for case in _sweep_cases(n=n, seed=seed):
        spec = configs.GenSpec(rho=float(rng.uniform(0.3, 0.95)), heavy_tail=bool(rng.random() < 0.5),
                               outlier_frac=float(rng.uniform(0, 0.1)),
                               outlier_mult=float(rng.uniform(5, 60)), seed=int(rng.integers(0, 10 ** 6)))
        pokes = []
        if rng.random() < 0.4:
            for _ in range(int(rng.integers(1, 6))):
                pokes.append((rng.random(), rng.random(), rng.random(), rng.random(), int(rng.integers(0, 6))))
        out.append((case, spec, pokes))
    return out


@pytest.mark.parametrize("cc", _calibration_cases(), ids=lambda c: "case%d" % c[0][0])
def test_seeded_sweep_with_calibration_tables(cg, cc):
    """As the sweep above, each cache coded with the tables of another (R28), some with
    non-finite or extreme elements (R31): every product bit for bit against the oracle."""
    case, spec, pokes = cc
    i, L, H, d, S, G, Tc, bins, bins_v, n_sink, anchor_bits, ppm, rngc, gen = case
    C = H * d
    X = _gen(L, S, C, gen)
    Y = _gen(L, S, C, spec)
    vals = [float("inf"), float("-inf"), float("nan"), 65504.0, -65504.0, 0.0]
    for a, b, c, e, v in pokes:
        Y[int(a * L), int(b * 2), int(c * S), int(e * C)] = vals[v]
    full_parity(cg, X, H, G, Tc, bins, chunk_range=rngc, label="calibration sweep %d" % i,
                bins_v=bins_v, n_sink=n_sink, anchor_bits=anchor_bits, outlier_ppm=ppm, X_enc=Y)


def test_stored_form_through_files_and_repeat_runs_are_identical(cg, tmp_path):
    """A cache kept as files (the stored tables and the container written out, read back
    by a fresh import) decodes to what the encoder's own handles decode; and every run of
    the path gives the same bytes: two table builds, two encodes, two decodes (the
    histogram and range passes use atomics; their results do not depend on order)."""
    L, S, C, G, Tc, H, bins = 3, 1500, 192, 10, 400, 3, (32, 16, 8)
    X = _gen(L, S, C, HEAVY)
    for kw in ({}, {"n_sink": 4, "outlier_ppm": 2000}, {"anchor_bits": 8}):
        tabs = [cg.build_cdf(X, G, Tc, bins, H_kv=H, **kw) for _ in range(2)]
        tbs = [t.serialize() for t in tabs]
        assert tbs[0] == tbs[1], kw
        blobs = [cg.encode(tabs[0], X), cg.encode(tabs[1], X)]
        cbs = [b.read().tobytes() for b in blobs]
        assert cbs[0] == cbs[1], kw
        outs = [cg.decode(tabs[0], blobs[0]), cg.decode(tabs[0], blobs[0])]
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), kw
        ft, fc = tmp_path / "tables.bin", tmp_path / "container.bin"
        ft.write_bytes(tbs[0])
        fc.write_bytes(cbs[0])
        tab_f = cg.tables_import(np.fromfile(ft, dtype=np.uint8).tobytes())
        blob_f = cg.blob_import(tab_f, np.fromfile(fc, dtype=np.uint8).tobytes())
        out_f = cg.decode(tab_f, blob_f)
        torch.cuda.synchronize()
        assert torch.equal(out_f.view(torch.int16), outs[0].view(torch.int16)), kw
