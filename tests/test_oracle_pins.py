"""Pins of the CPU oracle to facts fixed by the pages or by mathematics.

Every check here is independent of the oracle's own code: printed sizes from the pages,
a by-hand transcription of the pages' windowing, numpy's IEEE fp16 conversion, exact
rational arithmetic, exhaustive round trips, the coder's closed form on uniform tables
and its information bound, and a sort-based model of the stream interleaving.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle as O
from kv_cache_compression_cg_amd import configs, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
T = O.PROB_TOTAL


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


# --------------------------------------------------------------------------- sizes
def test_kv_size_formula_matches_printed_sizes():
    for name, L, H, d, S, sz, printed, div, *_ in _rows("kv_sizes.txt"):
        nbytes = 2 * int(L) * int(H) * int(d) * int(S) * int(sz)
        v = nbytes / int(div)
        p = float(printed)
        step = 10 ** -(len(printed.split(".")[1]) if "." in printed else 0)
        assert p <= v < p + step, (name, v, p)


def test_workload_raw_bytes_are_the_formula():
    for w in configs.ALL.values():
        assert w.raw_bytes == 2 * w.L * w.H_kv * w.d * w.S * 2
    assert configs.LLAMA3_70B.raw_bytes == 10_737_418_240
    assert configs.LLAMA3_70B_131K.raw_bytes == 42_949_672_960
    assert configs.LLAMA7B.raw_bytes == 637_534_208


# --------------------------------------------------------------------------- segmentation
def _page_windows(n_tokens, W):
    """Transcription of the pages' windowing: windows start at 0, W, 2W, ...; the first
    token of each window is its anchor; the last window may be short."""
    anchors, owner = [], {}
    for wi in range(math.ceil(n_tokens / W)):
        start = wi * W
        end = min(start + W, n_tokens)
        anchors.append(start)
        for t in range(start, end):
            owner[t] = start
    return anchors, owner


def test_anchor_counts_golden():
    lib = O.lib()
    for S, G, Tc, _lens, expect in _rows("anchor_counts.txt"):
        S, G, Tc, expect = int(S), int(G), int(Tc), int(expect)
        shp = O.Shape.make(1, 1, 1, S, G, Tc, [8])
        assert O.anchor_rows(shp, 0, shp.n_chunks) // 2 == expect
        assert sum(1 for t in range(S) if lib.cgo_is_anchor(t, G, Tc)) == expect


@settings(max_examples=60, deadline=None)
@given(S=st.integers(1, 300), G=st.integers(1, 40), Tc=st.integers(1, 120))
def test_segmentation_matches_page_windowing(S, G, Tc):
    lib = O.lib()
    for k in range(math.ceil(S / Tc)):
        t0 = k * Tc
        n = min(Tc, S - t0)
        assert lib.cgo_chunk_len(S, Tc, k) == n
        anchors, owner = _page_windows(n, G)
        assert lib.cgo_groups_in(n, G) == len(anchors)
        for u in range(n):
            assert bool(lib.cgo_is_anchor(t0 + u, G, Tc)) == (u in anchors)
            assert lib.cgo_anchor_of(t0 + u, G, Tc) == t0 + owner[u]


# --------------------------------------------------------------------------- fp16
def test_half_to_float_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = O.half_to_float(h)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_float_to_half_rne_against_numpy():
    rng = np.random.default_rng(1)
    halves = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    halves = halves[np.isfinite(halves)].astype(np.float32)
    # exact values, every midpoint between neighbours (ties), and points near them
    s = np.sort(np.unique(halves))
    mids = ((s[:-1].astype(np.float64) + s[1:]) / 2).astype(np.float32)
    cases = [halves, mids, np.nextafter(mids, np.float32(np.inf)),
             np.nextafter(mids, np.float32(-np.inf)),
             rng.standard_normal(200000).astype(np.float32) * np.float32(300),
             (rng.standard_normal(200000) * 1e-6).astype(np.float32),
             np.array([65504, 65519.99, 65520, 65536, 1e30, -65520, 2 ** -25, 2 ** -24,
                       3 * 2 ** -26, 2 ** -14, 0.0, -0.0], np.float32)]
    for f in cases:
        with np.errstate(over="ignore"):
            ref = f.astype(np.float16).view(np.uint16)
        got = O.float_to_half(f)
        assert np.array_equal(got, ref)


# --------------------------------------------------------------------------- tables
def _small_data(L=2, S=70, C=6, G=5, Tc=33, bins=(4, 8), seed=3, heavy=True):
    gen = configs.GenSpec(rho=0.85, heavy_tail=heavy, outlier_frac=0.2, outlier_mult=30.0,
                          seed=seed)
    X = synth.gen_custom(L, S, C, gen).view(torch.int16).numpy().view(np.uint16)
    shp = O.Shape.make(L, 1, C, S, G, Tc, bins)
    return shp, np.ascontiguousarray(X)


def _deltas(shp, X, l, kv, c):
    """(t, anchor, Delta) with Delta from numpy's float32 arithmetic."""
    xs = X[l, kv, :, c].view(np.float16).astype(np.float32)
    out = []
    for t in range(shp.S):
        u = t % shp.Tc
        if u % shp.G == 0:
            continue
        a = t - u + (u // shp.G) * shp.G
        out.append((t, a, np.float32(xs[t] - xs[a])))
    return out


def test_range_is_min_max_of_deltas():
    shp, X = _small_data()
    tab = O.build_tables(shp, X)
    for l in range(shp.L):
        for kv in range(2):
            for c in range(shp.C):
                d = np.array([x for _, _, x in _deltas(shp, X, l, kv, c)], np.float32)
                lo, hi = d.min(), d.max()
                assert tab.lo[l, kv, c] == lo
                w = np.float32(np.float32(hi - lo) / np.float32(shp.bins[l * 2 + kv] - 1))
                assert tab.w[l, kv, c] == w
                assert tab.r[l, kv, c] == (np.float32(1) / w if w > 0 else 0)


def test_quantizer_picks_nearest_grid_point_exactly():
    """q must minimise |Delta - (lo + q*w)| over the N grid points (exact rationals);
    a different choice is only allowed within 2^-20 relative of a tie."""
    shp, X = _small_data(L=2, S=90, C=5, bins=(3, 16))
    tab = O.build_tables(shp, X)
    sym = O.quantize(shp, X, tab.lo, tab.r, 0, shp.S)
    checked = 0
    for l in range(shp.L):
        for kv in range(2):
            N = int(shp.bins[l * 2 + kv])
            for c in range(shp.C):
                lo, w = Fraction(float(tab.lo[l, kv, c])), Fraction(float(tab.w[l, kv, c]))
                for t, _, dlt in _deltas(shp, X, l, kv, c):
                    D = Fraction(float(dlt))
                    q = int(sym[l, kv, t, c])
                    err = abs(D - (lo + q * w))
                    best = min(abs(D - (lo + j * w)) for j in range(N))
                    assert err <= best + w * Fraction(1, 2 ** 20)
                    assert err <= w / 2 * (1 + Fraction(1, 2 ** 20))
                    checked += 1
    assert checked > 1000


def test_constant_channel_and_all_anchor_edge_cases():
    S, C, G, Tc = 23, 3, 4, 10
    X = np.zeros((1, 2, S, C), np.uint16)
    X[0, 0, :, 0] = np.float16(1.5).view(np.uint16)           # constant channel
    X[0, 0, :, 1] = np.arange(S).astype(np.float16).view(np.uint16)  # deltas 1, 2, 3
    shp = O.Shape.make(1, 1, C, S, G, Tc, [3])                        # grid 1, 2, 3
    tab = O.build_tables(shp, X)
    assert tab.w[0, 0, 0] == 0 and tab.r[0, 0, 0] == 0 and tab.lo[0, 0, 0] == 0
    enc = O.encode(shp, X, tab)
    assert np.array_equal(O.decode(shp, tab, enc), X)         # exact for both channels
    # G = 1: every token is an anchor, the payload is empty, decode is a copy
    shp1 = O.Shape.make(1, 1, C, S, 1, Tc, [8])
    tab1 = O.build_tables(shp1, X)
    enc1 = O.encode(shp1, X, tab1)
    assert enc1.payload.size == 0 and np.array_equal(O.decode(shp1, tab1, enc1), X)


@settings(max_examples=200, deadline=None)
@given(N=st.integers(2, 32), data=st.data())
def test_frequency_table_invariants(N, data):
    counts = data.draw(st.lists(st.one_of(st.integers(0, 3), st.integers(0, 10 ** 6)),
                                min_size=N, max_size=N))
    f = O.freqs_from_counts(counts, N).astype(np.int64)
    assert f.sum() == T and (f >= 1).all()
    n = sum(counts)
    for a in range(N):
        for b in range(N):
            if counts[a] > counts[b]:
                assert f[a] >= f[b]
        if n:
            assert abs(Fraction(int(f[a]), T) - Fraction(counts[a], n)) <= Fraction(N + 1, T)
    if n == 0:
        assert f[0] == T - N + 1 and (f[1:] == 1).all()


def _freqs_by_rule(counts, N):
    """The frequency rule written out from its statement, in Python integers: every
    symbol gets 1 plus its share of the other T - N units, floor(c * (T - N) / n), and
    the units left over go to the most frequent symbol, the lowest index among equals.
    With no counts every share is 0."""
    n = sum(counts)
    f = [1 + (c * (T - N) // n if n else 0) for c in counts]
    top = max(counts)
    best = counts.index(top)
    f[best] += T - sum(f)
    return f


# hand-worked cases (T = 256): counts -> frequencies, with the arithmetic
FREQ_CASES = [
    # n = 9, shares floor(3 * 253 / 9) = 84 -> f = 85 each, sum 255, the 1 left over
    # goes to index 0 (three-way tie, lowest index)
    ([3, 3, 3], [86, 85, 85]),
    # n = 5, shares 252/5 = 50.4 -> 50, 100.8 -> 100 twice, 0 -> 0; f = 51, 101, 101, 1
    # (sum 254); the 2 left over go to index 1 (tie between 1 and 2, lowest index)
    ([1, 2, 2, 0], [51, 103, 101, 1]),
    # n = 15, shares 0, 252/15 = 16.8 -> 16, 7 * 252/15 = 117.6 -> 117 twice;
    # f = 1, 17, 118, 118 (sum 254); the 2 left over go to index 2 (tie of 2 and 3)
    ([0, 1, 7, 7], [1, 17, 120, 118]),
    # n = 0: every f = 1 and the 254 left over go to index 0 (all counts tie at 0)
    ([0, 0], [255, 1]),
    ([0, 0, 0, 0, 0], [252, 1, 1, 1, 1]),
    # exact shares: 128 * 254 / 256 = 127, no remainder
    ([128, 128], [128, 128]),
    # one symbol takes everything: f = 1 + 254 = 255 and 1 for the other
    ([0, 1000], [1, 255]),
]


@pytest.mark.parametrize("counts,expect", FREQ_CASES)
def test_frequency_rule_hand_worked(counts, expect):
    assert sum(expect) == T
    assert _freqs_by_rule(counts, len(counts)) == expect
    assert list(O.freqs_from_counts(counts, len(counts))) == expect


@settings(max_examples=400, deadline=None)
@given(N=st.integers(2, 32), data=st.data())
def test_frequency_rule_recomputed_independently(N, data):
    """The oracle's frequencies equal the rule recomputed in Python integers, on drawn
    counts that include many ties (small values), zeros and large values."""
    counts = data.draw(st.lists(st.one_of(st.integers(0, 2), st.integers(0, 50),
                                          st.integers(0, 2 ** 40)), min_size=N, max_size=N))
    assert list(O.freqs_from_counts(counts, N)) == _freqs_by_rule(counts, N)


@pytest.mark.parametrize("L,S,C,G,Tc,n_sink", [(2, 70, 6, 5, 33, 0), (2, 97, 9, 4, 30, 4),
                                                (1, 50, 3, 7, 50, 9), (2, 41, 5, 10, 16, 13),
                                                (1, 12, 2, 1, 5, 0)])
def test_histogram_counts_are_a_direct_count(L, S, C, G, Tc, n_sink):
    """counts[l, kv, c, s] is the number of tokens t >= n_sink that are not anchors (by
    the pages' windowing, restarted at every chunk) whose symbol is s, over all chunks:
    recounted here with numpy's bincount.  Ragged last chunks, sinks that reach past the
    first chunk's groups, and G = 1 (no symbol at all) are included."""
    _, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8,) * L)
    shp = O.Shape.make(L, 1, C, S, G, Tc, [5 + 3 * l for l in range(L)], n_sink=n_sink)
    tab = O.build_tables(shp, X)
    sym = O.quantize(shp, X, tab.lo, tab.r, 0, S)
    coded = []
    for k in range(math.ceil(S / Tc)):
        n = min(Tc, S - k * Tc)
        anchors, _ = _page_windows(n, G)
        coded += [k * Tc + u for u in range(n) if u not in anchors and k * Tc + u >= n_sink]
    for l in range(L):
        for kv in range(2):
            N = int(shp.bins[l * 2 + kv])
            for c in range(C):
                ref = np.bincount(sym[l, kv, coded, c].astype(np.int64), minlength=O.MAX_BINS)
                assert ref.size == O.MAX_BINS
                assert np.array_equal(tab.counts[l, kv, c], ref.astype(np.uint64)), (l, kv, c)
                assert ref[N:].sum() == 0
    assert tab.counts.sum() == len(coded) * 2 * L * C


# --------------------------------------------------------------------------- rANS coder
FREQ_SETS = [[T // 2, T // 2], [1, T - 1], [T - 1, 1], [1, 1, T - 3, 1], [60, 60, 60, 76],
             [1, 2, 3, T - 6], [7, 241, 7, 1]]
STATE_LOW = 2 ** 16


def _check_steps(steps, m):
    """Two state words read before step 0, then at most one word per step, never after
    the last symbol, in increasing step order."""
    assert list(steps[:2]) == [-1, -1]
    rest = [int(v) for v in steps[2:]]
    assert rest == sorted(set(rest)) and all(0 <= v <= m - 2 for v in rest)


def test_coder_exhaustive_round_trip_and_final_state():
    n_cases = 0
    for f in FREQ_SETS:
        N = len(f)
        for m in range(0, 7):
            for x in itertools.product(range(N), repeat=m):
                words, steps = O.rans_encode(x, f)
                if m == 0:
                    assert words.size == 0
                    continue
                _check_steps(steps, m)
                dec, used, fin = O.rans_decode(words, m, f)
                assert list(dec) == list(x) and used == len(words)
                assert fin == STATE_LOW  # the decoder retraces the encoder to its start
                n_cases += 1
    assert n_cases > 10000


@pytest.mark.parametrize("bits", [1, 2, 3, 5])
def test_coder_uniform_tables_insert_symbol_bits(bits):
    """With N = 2^b equal frequencies f = 256 / N, one coding step writes the symbol's b
    bits into the state at bit 8 - b and moves the bits above up (floor(x / f) * 256 +
    x mod f + s * f).  From x = 2^16 and while no word is shifted out (b * m <= 15) the
    stream is the two halves of 2^(16 + b m) + sum_i x_i 2^(8 - b + b i)."""
    N = 2 ** bits
    f = [T // N] * N
    rng = np.random.default_rng(bits)
    for m in range(1, 15 // bits + 1):
        for _ in range(20):
            x = [int(v) for v in rng.integers(0, N, m)]
            state = 2 ** (16 + bits * m) + sum(s << (8 - bits + bits * i) for i, s in enumerate(x))
            words, steps = O.rans_encode(x, f)
            assert list(words) == [state >> 16, state & 0xFFFF]
            assert list(steps) == [-1, -1]


@settings(max_examples=150, deadline=None)
@given(data=st.data())
def test_coder_random_streams_round_trip_and_length_bound(data):
    N = data.draw(st.integers(2, 32))
    counts = data.draw(st.lists(st.integers(0, 5000), min_size=N, max_size=N))
    f = O.freqs_from_counts(counts, N)
    p = f / f.sum()
    m = data.draw(st.integers(1, 1500))
    rng = np.random.default_rng(data.draw(st.integers(0, 2 ** 31)))
    x = rng.choice(N, size=m, p=p)
    words, steps = O.rans_encode(x, f)
    _check_steps(steps, m)
    dec, used, fin = O.rans_decode(words, m, f)
    assert np.array_equal(dec, x) and used == len(words) and fin == STATE_LOW
    # log2 of the state plus 16 per word shifted out grows by at most log2(256 / f) +
    # log2(1 + 2^-8) per step (the state is >= 2^8 f when coded), starts at 16 and ends
    # at >= 16 + 16 * (words - 2)
    ideal = float(np.sum(np.log2(T / f[x].astype(np.float64))))
    assert 16 * len(words) <= ideal + m * math.log2(1 + 2 ** -8) + 32 + 1e-6


def test_coded_size_close_to_empirical_entropy():
    """Over realistic streams the coder spends what the frequency tables imply (their
    cross-entropy against the counts, within the per-step bound, plus the two state
    words per stream), and that is within a few percent of the empirical entropy."""
    shp, X = _small_data(L=2, S=1200, C=8, G=10, Tc=400, bins=(8, 32), seed=5)
    tab = O.build_tables(shp, X)
    enc = O.encode(shp, X, tab)
    cnt = tab.counts.astype(np.float64)
    n = cnt.sum(-1, keepdims=True)
    p = np.where(cnt > 0, cnt / np.maximum(n, 1), 1.0)
    h_emp_bits = float(-(cnt * np.log2(p)).sum())
    n_streams = shp.L * 2 * shp.C * shp.n_chunks
    f = np.maximum(tab.freqs.astype(np.float64), 1.0)
    cross_bits = float((cnt * np.log2(T / f)).sum())
    coded = enc.payload.size * 16
    assert coded <= cross_bits + cnt.sum() * math.log2(1 + 2 ** -8) + 32 * n_streams + 1e-6
    assert cross_bits <= 1.05 * h_emp_bits
    assert coded >= h_emp_bits * 0.99


# --------------------------------------------------------------------------- interleaving
def test_group_words_follow_lockstep_read_order():
    """Sort-based model: every word of every lane, keyed by (read step, lane, index)."""
    shp, X = _small_data(L=1, S=150, C=70, G=6, Tc=64, bins=(16,), seed=9)
    tab = O.build_tables(shp, X)
    enc = O.encode(shp, X, tab)
    sym = O.quantize(shp, X, tab.lo, tab.r, 0, shp.S)
    NB = -(-shp.C // O.LANES)
    g = 0
    for k in range(shp.n_chunks):
        t0 = k * shp.Tc
        toks = [t for t in range(t0, min(t0 + shp.Tc, shp.S)) if (t - t0) % shp.G]
        for l in range(shp.L):
            for kv in range(2):
                for b in range(NB):
                    keyed = []
                    for lane in range(min(O.LANES, shp.C - b * O.LANES)):
                        c = b * O.LANES + lane
                        x = [int(sym[l, kv, t, c]) for t in toks]
                        words, steps = O.rans_encode(x, tab.freqs[l, kv, c, :shp.bins[l * 2 + kv]])
                        keyed += [((int(s), lane, j), int(wd))
                                  for j, (wd, s) in enumerate(zip(words, steps))]
                    expect = [wd for _, wd in sorted(keyed)]
                    got = enc.payload[enc.offsets[g]:enc.offsets[g + 1]]
                    assert list(got) == expect
                    g += 1
    assert g == len(enc.offsets) - 1


# --------------------------------------------------------------------------- reconstruction
def _check_reconstruction(shp, X, tab, Y):
    C = shp.C
    xs = X.view(np.float16).astype(np.float64)
    ys = Y.view(np.float16).astype(np.float64)
    for t in range(shp.S):
        u = t % shp.Tc
        a = t - u + (u // shp.G) * shp.G
        if a == t:
            assert np.array_equal(Y[:, :, t], X[:, :, t])
            continue
        wv = tab.w.astype(np.float64)
        ulp = np.spacing(np.abs(ys[:, :, t]).astype(np.float16)).astype(np.float64)
        tol = (wv / 2 * (1 + 2 ** -20) + ulp / 2 +
               2 ** -22 * (np.abs(xs[:, :, t]) + np.abs(xs[:, :, a]) + np.abs(tab.lo) + 32 * wv))
        assert (np.abs(xs[:, :, t] - ys[:, :, t]) <= tol).all()
    assert C > 0


def test_round_trip_error_is_at_most_half_a_bin():
    for heavy in (False, True):
        shp, X = _small_data(L=3, S=333, C=16, G=10, Tc=128, bins=(2, 8, 32), heavy=heavy)
        tab = O.build_tables(shp, X)
        enc = O.encode(shp, X, tab)
        Y = O.decode(shp, tab, enc)
        _check_reconstruction(shp, X, tab, Y)
        sym = O.quantize(shp, X, tab.lo, tab.r, 0, shp.S)
        assert np.array_equal(O.dequantize(shp, tab, sym, X, 0, shp.S), Y)


def test_brute_force_tiny_tensor_exact_rationals():
    """L=1, S=12, C=2, G=4, N=4: grid, symbols and reconstruction from exact rationals."""
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((1, 2, 12, 2)) * 3).astype(np.float16).view(np.uint16)
    X = np.ascontiguousarray(X)
    shp = O.Shape.make(1, 1, 2, 12, 4, 12, [4])
    tab = O.build_tables(shp, X)
    enc = O.encode(shp, X, tab)
    Y = O.decode(shp, tab, enc)
    xf = X.view(np.float16)
    for kv in range(2):
        for c in range(2):
            D = {t: Fraction(float(np.float32(np.float32(xf[0, kv, t, c]) -
                                              np.float32(xf[0, kv, t - t % 4, c]))))
                 for t in range(12) if t % 4}
            lo, hi = min(D.values()), max(D.values())
            assert Fraction(float(tab.lo[0, kv, c])) == lo
            w = (hi - lo) / 3
            assert abs(Fraction(float(tab.w[0, kv, c])) - w) <= w * Fraction(1, 2 ** 23)
            for t, d in D.items():
                grid = [lo + j * w for j in range(4)]
                j = min(range(4), key=lambda j: (abs(d - grid[j]), -j))
                y = Fraction(float(xf[0, kv, t - t % 4, c])) + grid[j]
                got = Fraction(float(Y[0, kv, t, c].view(np.float16)))
                assert abs(got - y) <= abs(y) * Fraction(1, 2 ** 10) + Fraction(1, 2 ** 20)


def test_decode_of_damaged_payload_stays_in_bounds():
    shp, X = _small_data(L=1, S=200, C=64, G=10, Tc=100, bins=(16,), seed=2)
    tab = O.build_tables(shp, X)
    enc = O.encode(shp, X, tab)
    rng = np.random.default_rng(0)
    bad = enc.payload.copy()
    bad[rng.integers(0, bad.size, 50)] ^= np.uint16(0x5A5A)
    Y = O.decode(shp, tab, enc, payload=bad)
    assert Y.shape == X.shape
    trunc = enc.payload[: enc.payload.size // 2]
    O.decode(shp, tab, O.Encoded(enc.k_begin, enc.k_end,
                                 np.minimum(enc.offsets, trunc.size).astype(np.uint64),
                                 trunc, enc.anchors))


def test_zero_bounds_are_positive_zero():
    """Deltas of +0 and -0 compare equal; the stored bound is +0 either way."""
    S, C = 30, 2
    X = np.zeros((1, 2, S, C), np.uint16)
    X[0, 0, 1::3, 0] = 0x8000                     # -0 at some tokens
    X[0, 1, :, 1] = 0x8000                        # all -0: deltas are +0
    shp = O.Shape.make(1, 1, C, S, 10, 30, [4])
    tab = O.build_tables(shp, X)
    assert (tab.lo.view(np.uint32) == 0).all() and (tab.w.view(np.uint32) == 0).all()


def test_key_and_value_rows_take_their_own_bin_counts():
    """Keys finer than values ("Guide to CacheGen", Solution pillar 1): with separate bin
    counts for the V rows, every K row is coded exactly as in a run where all rows use the
    K counts, and every V row as in a run with the V counts, since ranges, widths, tables
    and streams all belong to one (layer, K/V, channel).  Checked on tables, symbols,
    every group's payload words and the decoded rows (a partial channel block, C = 70)."""
    L, C, S, G, Tc = 2, 70, 90, 5, 40
    bk, bv = (16, 5), (4, 9)
    _, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=bk)
    shp = O.Shape.make(L, 1, C, S, G, Tc, bk, bins_v=bv)
    assert list(shp.bins) == [16, 4, 5, 9]
    ref = {0: O.Shape.make(L, 1, C, S, G, Tc, bk), 1: O.Shape.make(L, 1, C, S, G, Tc, bv)}
    tab = O.build_tables(shp, X)
    tabs = {kv: O.build_tables(s, X) for kv, s in ref.items()}
    for kv in range(2):
        for name in ("lo", "w", "r", "freqs"):
            assert np.array_equal(getattr(tab, name)[:, kv], getattr(tabs[kv], name)[:, kv]), name
    sym = O.quantize(shp, X, tab.lo, tab.r, 0, S)
    for kv in range(2):
        sref = O.quantize(ref[kv], X, tabs[kv].lo, tabs[kv].r, 0, S)
        assert np.array_equal(sym[:, kv], sref[:, kv])
        assert int(sym[:, kv].max()) < max(bk if kv == 0 else bv)
    enc = O.encode(shp, X, tab)
    encs = {kv: O.encode(ref[kv], X, tabs[kv]) for kv in range(2)}
    NB = -(-C // O.LANES)
    for k in range(shp.n_chunks):
        for l in range(L):
            for kv in range(2):
                for b in range(NB):
                    g = ((k * 2 * L) + l * 2 + kv) * NB + b
                    mine = enc.payload[int(enc.offsets[g]):int(enc.offsets[g + 1])]
                    e = encs[kv]
                    theirs = e.payload[int(e.offsets[g]):int(e.offsets[g + 1])]
                    assert np.array_equal(mine, theirs), (k, l, kv, b)
    out = O.decode(shp, tab, enc)
    for kv in range(2):
        assert np.array_equal(out[:, kv], O.decode(ref[kv], tabs[kv], encs[kv])[:, kv])


@pytest.mark.parametrize("G", [4, 3])
def test_sink_tokens_are_kept_in_fp16_and_left_out_of_the_tables(G):
    """Attention sinks ("Guide to CacheGen", Best Practices): the first four tokens come
    back exactly, and their values reach neither the ranges nor the frequency tables.
    Planting huge values on the sinks that are not anchors (tokens 1-3 at G = 4, 1-2 at
    G = 3, where token 3 anchors the next group and so still feeds its deltas) changes no
    table and no decoded token from 4 on.  Without sinks the plant widens the range; the
    ranges with sinks are the brute-force min / max of the deltas of tokens >= 4."""
    L, C, S, Tc, n_sink = 2, 9, 70, 30, 4
    shp0, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8, 4))
    shp = O.Shape.make(L, 1, C, S, G, Tc, (8, 4), n_sink=n_sink)
    P = X.copy()
    for t in range(1, n_sink):
        if t % G:
            P[:, :, t] = np.float16(30000.0).view(np.uint16)
    tx, tp = O.build_tables(shp, X), O.build_tables(shp, P)
    for name in ("lo", "w", "r", "counts", "freqs"):
        assert np.array_equal(getattr(tx, name), getattr(tp, name)), name
    assert (O.build_tables(shp0, P).w > tx.w).any()
    for l in range(L):
        for kv in range(2):
            for c in range(C):
                ds = [d for t, _, d in _deltas(shp, X, l, kv, c) if t >= n_sink]
                assert tx.lo[l, kv, c] == np.float32(min(ds)) + np.float32(0.0)
                assert tx.lo[l, kv, c] + tx.w[l, kv, c] * (shp.bins[l * 2 + kv] - 1) >= max(ds) - 1e-3
    enc = O.encode(shp, P, tp)
    out = O.decode(shp, tp, enc)
    assert np.array_equal(out[:, :, :n_sink], P[:, :, :n_sink])
    assert np.array_equal(enc.sinks, P[:, :, :n_sink])
    ref = O.decode(shp, tx, O.encode(shp, X, tx))
    assert np.array_equal(out[:, :, n_sink:], ref[:, :, n_sink:])
    # the sink rows belong to the container: tables built from X code P's sinks exactly
    assert np.array_equal(O.decode(shp, tx, O.encode(shp, P, tx))[:, :, :n_sink], P[:, :, :n_sink])
    # a decode of chunk 1 alone writes no sink row
    part = O.decode(shp, tp, O.encode(shp, P, tp, 1, 2))
    assert (part[:, :, :Tc] == 0).all()
    assert O.table_bytes(shp) == O.table_bytes(shp0)


def test_outlier_channel_leaves_the_other_channels_alone():
    """Outlier channels ("Guide to CacheGen", Solution pillar 3: kept apart so that they do
    not distort the distribution of regular channels).  Tables are per (layer, K/V,
    channel), so scaling one channel by 500 changes that channel's range and frequencies
    only: every other channel keeps its tables, symbols and decoded values bit for bit,
    and the outlier channel still meets the half-bin bound."""
    L, C, S, G, Tc = 1, 70, 90, 5, 40
    shp, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8,))
    Y = X.copy()
    oc = 37
    v = Y[:, :, :, oc].view(np.float16).astype(np.float32) * 500.0
    Y[:, :, :, oc] = np.clip(v, -65504, 65504).astype(np.float16).view(np.uint16)
    tx, ty = O.build_tables(shp, X), O.build_tables(shp, Y)
    keep = [c for c in range(C) if c != oc]
    for name in ("lo", "w", "r", "freqs"):
        assert np.array_equal(getattr(tx, name)[:, :, keep], getattr(ty, name)[:, :, keep]), name
    assert ty.w[0, 0, oc] > 100 * tx.w[0, 0, oc]
    ox = O.decode(shp, tx, O.encode(shp, X, tx))
    oy = O.decode(shp, ty, O.encode(shp, Y, ty))
    assert np.array_equal(ox[..., keep], oy[..., keep])
    y = Y[..., oc].view(np.float16).astype(np.float64)
    d = oy[..., oc].view(np.float16).astype(np.float64)
    wv = ty.w[:, :, oc].astype(np.float64)[:, :, None]
    assert (np.abs(y - d) <= wv / 2 * (1 + 2 ** -20) + np.abs(d) * 2 ** -11 + 1e-30).all()


@pytest.mark.parametrize("G,Tc", [(5, 40), (10, 90)])
def test_8bit_anchors(G, Tc):
    """Anchors quantized to 8 bits ("Guide to CacheGen", Solution pillar 2): the grid of
    a channel spans its anchor tokens (brute-force min / max, width / 255); each code is
    the nearest grid point (checked against all 256); decoded anchors are the grid values,
    within half a grid step of the input; every other token still meets the delta grid's
    half-bin bound, since its delta is taken against the decoded anchor.  The container's
    payload equals an fp16-anchor encode of the cache whose anchors hold their grid
    values, and its anchors section is half the size."""
    L, C, S = 2, 70, 200
    shp16, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(16, 4))
    shp = O.Shape.make(L, 1, C, S, G, Tc, (16, 4), anchor_bits=8)
    tab = O.build_tables(shp, X)
    xf = X.view(np.float16).astype(np.float64)
    anc = [t for t in range(S) if (t % Tc) % G == 0]
    amin, amax = xf[:, :, anc].min(axis=2), xf[:, :, anc].max(axis=2)
    assert np.array_equal(tab.alo, (amin.astype(np.float32) + np.float32(0)))
    assert np.array_equal(tab.aw, ((amax - amin).astype(np.float32) / np.float32(255)).astype(np.float32))
    enc = O.encode(shp, X, tab)
    assert enc.anchors.dtype == np.uint8
    # codes against brute force, anchor rows in container order (chunk, l, kv, group)
    r = 0
    grid = tab.alo.astype(np.float64)[..., None] + np.arange(256) * tab.aw.astype(np.float64)[..., None]
    for k in range(shp.n_chunks):
        for l in range(L):
            for kv in range(2):
                for t in range(k * Tc, min((k + 1) * Tc, S), G):
                    dist = np.abs(xf[l, kv, t][:, None] - grid[l, kv])
                    code = enc.anchors[r].astype(np.int64)
                    best = dist.min(axis=1)
                    got = dist[np.arange(C), code]
                    assert (got <= best + 1e-6 * (1 + np.abs(xf[l, kv, t]))).all(), (k, l, kv, t)
                    r += 1
    assert r == enc.anchors.shape[0]
    out = O.decode(shp, tab, enc)
    of = out.view(np.float16).astype(np.float64)
    aw = tab.aw.astype(np.float64)[:, :, None, :]
    ea = np.abs(of[:, :, anc] - xf[:, :, anc])
    assert (ea <= aw / 2 * (1 + 2 ** -20) + np.abs(of[:, :, anc]) * 2 ** -11 + 1e-30).all()
    non = [t for t in range(S) if (t % Tc) % G]
    wv = tab.w.astype(np.float64)[:, :, None, :]
    en = np.abs(of[:, :, non] - xf[:, :, non])
    assert (en <= wv / 2 * (1 + 2 ** -20) + np.abs(of[:, :, non]) * 2 ** -11 + 1e-30).all()
    Xs = O.snap_anchors(shp, X, tab)
    t16 = O.build_tables(shp16, Xs)
    for name in ("lo", "w", "r", "freqs"):
        assert np.array_equal(getattr(t16, name), getattr(tab, name)), name
    e16 = O.encode(shp16, Xs, t16)
    assert np.array_equal(e16.payload, enc.payload) and np.array_equal(e16.offsets, enc.offsets)
    assert np.array_equal(O.decode(shp16, t16, e16), out)
    assert enc.anchors.nbytes * 2 == e16.anchors.nbytes
    assert O.table_bytes(shp) == O.table_bytes(shp16) + 2 * L * C * 8
    assert enc.clamped == 0 and e16.clamped == 0


# --------------------------------------------------------------------------- outlier table
def _grid_dist(D, lo, w, N):
    """Exact distance from a delta to the nearest of the N points lo + j*w."""
    D, lo, w = Fraction(float(D)), Fraction(float(lo)), Fraction(float(w))
    return min(abs(D - (lo + j * w)) for j in range(N))


def _coded_deltas(shp, Xs, l, kv, c):
    """(t, Delta) of the coded tokens (not anchors, t >= n_sink) of one channel row."""
    return [(t, d) for t, _, d in _deltas(shp, Xs, l, kv, c) if t >= shp.n_sink]


@pytest.mark.parametrize("ppm", [20000, 100000, 250000])
def test_outlier_clip_leaves_at_most_the_budget_out_at_each_end(ppm):
    """The clipped range [lo', hi'] of every channel row lies inside the deltas' range,
    leaves at most b = floor(n * ppm / 10^6) deltas below lo' and at most b above hi',
    and is not narrower than the fine grid needs: one more fine interval (width
    (hi - lo) / 256) dropped at an end would leave more than b out there."""
    L, S, C, G, Tc = 2, 400, 7, 5, 130
    _, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8, 8), seed=5)
    shp = O.Shape.make(L, 1, C, S, G, Tc, (16, 4), n_sink=3, outlier_ppm=ppm)
    tab = O.build_tables(shp, X)
    narrowed = 0
    for l in range(L):
        for kv in range(2):
            N = int(shp.bins[l * 2 + kv])
            for c in range(C):
                d = np.array([x for _, x in _coded_deltas(shp, X, l, kv, c)], np.float64)
                n, b = d.size, d.size * ppm // 10 ** 6
                lo, hi = d.min(), d.max()
                lo_c = float(tab.lo[l, kv, c])
                hi_c = lo_c + float(tab.w[l, kv, c]) * (N - 1)
                assert lo <= lo_c <= hi and lo_c <= hi_c <= hi * (1 + 2 ** -20) + 2 ** -30
                assert (d < lo_c).sum() <= b
                assert (d > hi_c * (1 + 2 ** -20) + 2 ** -30).sum() <= b
                wf = (hi - lo) / 256
                if lo_c + 2.01 * wf < hi_c:
                    assert (d < lo_c + 1.001 * wf).sum() > b
                if hi_c - 2.01 * wf > lo_c:
                    assert (d > hi_c - 1.001 * wf).sum() > b
                narrowed += (hi_c - lo_c) < 0.9 * (hi - lo)
    assert narrowed > 0


def test_outlier_table_off_or_empty_budget_changes_nothing():
    """ppm = 0, or a budget that rounds down to 0 deltas, keeps the full range: tables,
    streams and decoded values are those of the plain codec."""
    shp0, X = _small_data(L=2, S=120, C=6, G=5, Tc=60, bins=(8, 4))
    t0 = O.build_tables(shp0, X)
    e0 = O.encode(shp0, X, t0)
    shp = O.Shape.make(2, 1, 6, 120, 5, 60, (8, 4), outlier_ppm=1000)  # n ~ 96: b = 0
    t1 = O.build_tables(shp, X)
    for name in ("lo", "w", "r", "freqs"):
        assert np.array_equal(getattr(t0, name), getattr(t1, name)), name
    e1 = O.encode(shp, X, t1)
    assert np.array_equal(e0.payload, e1.payload) and e1.n_outliers == 0 and e0.clamped == 0
    assert np.array_equal(O.decode(shp0, t0, e0), O.decode(shp, t1, e1))


@pytest.mark.parametrize("anchor_bits", [16, 8])
def test_outlier_entries_are_exactly_the_off_grid_elements(anchor_bits):
    """Every element whose nearest grid point is more than half a step away (exact
    rationals, up to 2^-20 relative at the boundary) has an entry, and no other element
    has one; entries are grouped like the payload (chunk, layer, K/V, 64-channel block),
    in ascending token then lane, and hold the element's fp16 bits; the decode returns
    them exactly and every other element within half a step of the clipped grid."""
    L, S, C, G, Tc, ppm = 2, 300, 70, 10, 128, 30000
    _, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8, 8), seed=7)
    shp = O.Shape.make(L, 1, C, S, G, Tc, (8, 32), n_sink=2, anchor_bits=anchor_bits,
                       outlier_ppm=ppm)
    tab = O.build_tables(shp, X)
    enc = O.encode(shp, X, tab)
    Xs = O.snap_anchors(shp, X, tab)
    expect = set()
    for l in range(L):
        for kv in range(2):
            N = int(shp.bins[l * 2 + kv])
            for c in range(C):
                w = Fraction(float(tab.w[l, kv, c]))
                for t, D in _coded_deltas(shp, Xs, l, kv, c):
                    dist = _grid_dist(D, tab.lo[l, kv, c], tab.w[l, kv, c], N)
                    if dist > w / 2 * (1 + Fraction(1, 2 ** 20)) or (w == 0 and dist > 0):
                        expect.add((l, kv, t, c))
                    elif dist >= w / 2 * (1 - Fraction(1, 2 ** 20)) and w > 0:
                        expect.add((l, kv, t, c, "edge"))
    got = []
    NB = -(-C // O.LANES)
    g = 0
    for k in range(shp.n_chunks):
        for l in range(L):
            for kv in range(2):
                for b in range(NB):
                    beg, end = int(enc.out_offsets[g]), int(enc.out_offsets[g + 1])
                    keys = [int(v) for v in enc.out_keys[beg:end]]
                    assert keys == sorted(keys)
                    for e in range(beg, end):
                        t = k * Tc + (int(enc.out_keys[e]) >> 6)
                        c = b * O.LANES + (int(enc.out_keys[e]) & 63)
                        assert enc.out_values[e] == X[l, kv, t, c]
                        got.append((l, kv, t, c))
                    g += 1
    assert g == len(enc.out_offsets) - 1 and int(enc.out_offsets[-1]) == len(got)
    hard = {e for e in expect if len(e) == 4}
    edge = {e[:4] for e in expect if len(e) == 5}
    assert hard <= set(got) and set(got) <= hard | edge
    assert len(got) > 0
    out = O.decode(shp, tab, enc)
    for (l, kv, t, c) in got:
        assert out[l, kv, t, c] == X[l, kv, t, c]
    # the rest within half a step of the clipped grid (anchors exact with fp16 anchors)
    xs, ys = X.view(np.float16).astype(np.float64), out.view(np.float16).astype(np.float64)
    wv = tab.w.astype(np.float64)[:, :, None, :]
    err = np.abs(xs - ys)
    if anchor_bits == 8:
        err[:, :, [t for t in range(S) if (t % Tc) % G == 0]] = 0
    assert (err <= wv / 2 * (1 + 2 ** -20) + np.abs(ys) * 2 ** -11 + 1e-30).all()
    # without the table the same elements are coded clamped and only counted
    shp_off = O.Shape.make(L, 1, C, S, G, Tc, (8, 32), n_sink=2, anchor_bits=anchor_bits)
    tab_off = O.Tables(tab.lo, tab.w, tab.r, tab.counts, tab.freqs, tab.alo, tab.aw, tab.ar)
    e_off = O.encode(shp_off, X, tab_off)
    assert e_off.clamped == len(got) and e_off.n_outliers == 0
    assert np.array_equal(e_off.payload, enc.payload)


@pytest.mark.parametrize("anchor_bits", [16, 8])
def test_another_cache_is_coded_within_the_bound_with_the_table(anchor_bits):
    """Tables profiled on one cache ("Guide to CacheGen", Solution pillar 3: calibration
    tables) coding another: with the outlier table, every element the tables' grids
    cannot hold within half a step -- including, with 8-bit anchors, anchors beyond
    their grid -- is stored exactly; without it those elements are counted as clamped.
    Both counts equal a brute-force count over the new cache."""
    L, S, C, G, Tc = 1, 200, 9, 5, 100
    _, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8,), seed=1)
    _, Y = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8,), seed=2)
    Y = Y.copy()
    Y[0, 0, 50, 3] = np.float16(2000.0).view(np.uint16)     # an anchor (t = 50) far out
    Y[0, 1, 57, 4] = np.float16(-3000.0).view(np.uint16)    # a non-anchor far out
    on = O.Shape.make(L, 1, C, S, G, Tc, (8,), anchor_bits=anchor_bits, outlier_ppm=5000)
    off = O.Shape.make(L, 1, C, S, G, Tc, (8,), anchor_bits=anchor_bits)
    t_on, t_off = O.build_tables(on, X), O.build_tables(off, X)
    e_on, e_off = O.encode(on, Y, t_on), O.encode(off, Y, t_off)
    Ys_on, Ys_off = O.snap_anchors(on, Y, t_on), O.snap_anchors(off, Y, t_off)

    def brute(shp, tab, Ys):
        n = 0
        for kv in range(2):
            for c in range(C):
                w = Fraction(float(tab.w[0, kv, c]))
                for t, D in _coded_deltas(shp, Ys, 0, kv, c):
                    dist = _grid_dist(D, tab.lo[0, kv, c], tab.w[0, kv, c], 8)
                    n += dist > w / 2 * (1 + Fraction(1, 2 ** 20)) or (w == 0 and dist > 0)
                if anchor_bits == 8:
                    aw = Fraction(float(tab.aw[0, kv, c]))
                    for t in range(0, S, G):
                        x = Fraction(float(Y[0, kv, t, c].view(np.float16)))
                        a = _grid_dist(x, tab.alo[0, kv, c], tab.aw[0, kv, c], 256)
                        n += a > aw / 2 * (1 + Fraction(1, 2 ** 20))
        return n

    assert e_on.n_outliers == brute(on, t_on, Ys_on) and e_on.n_outliers >= 2
    assert e_off.clamped == brute(off, t_off, Ys_off) and e_off.clamped >= 2
    out = O.decode(on, t_on, e_on)
    assert out[0, 1, 57, 4] == Y[0, 1, 57, 4] and out[0, 0, 50, 3] == Y[0, 0, 50, 3]
    ys, xs = out.view(np.float16).astype(np.float64), Y.view(np.float16).astype(np.float64)
    tol = t_on.w.astype(np.float64)[:, :, None, :] / 2 * (1 + 2 ** -20) + np.abs(ys) * 2 ** -11
    if anchor_bits == 8:
        tol[:, :, ::G] = t_on.aw.astype(np.float64)[:, :, None, :] / 2 * (1 + 2 ** -20) + np.abs(ys[:, :, ::G]) * 2 ** -11
    assert (np.abs(xs - ys) <= tol + 1e-30).all()


@pytest.mark.parametrize("anchor_bits", [16, 8])
def test_non_finite_elements_of_another_cache_are_stored_exactly(anchor_bits):
    """Calibration tables coding a cache that holds NaN and Inf (reading: no grid point
    holds a NaN delta, so such an element is off its grid like one beyond the range):
    with the outlier table the entries are those of the finite cache plus exactly the
    non-finite elements (and, with fp16 anchors, the rest of a group whose anchor is
    NaN, all of whose deltas are NaN; with 8-bit anchors the NaN anchor itself), each
    holding its fp16 bits, which the decode returns; without the table they are the
    clamped count."""
    L, S, C, G, Tc = 1, 200, 9, 5, 100
    _, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8,), seed=1)
    on = O.Shape.make(L, 1, C, S, G, Tc, (8,), anchor_bits=anchor_bits, outlier_ppm=5000)
    off = O.Shape.make(L, 1, C, S, G, Tc, (8,), anchor_bits=anchor_bits)
    tab = O.build_tables(on, X)

    def entries(enc):
        NB = -(-C // O.LANES)
        got, g = set(), 0
        for k in range(on.n_chunks):
            for kv in range(2):
                for b in range(NB):
                    for e in range(int(enc.out_offsets[g]), int(enc.out_offsets[g + 1])):
                        key = int(enc.out_keys[e])
                        got.add((kv, k * Tc + (key >> 6), b * O.LANES + (key & 63)))
                    g += 1
        return got

    base = entries(O.encode(on, X, tab))
    nan16 = np.float16(np.nan).view(np.uint16)
    nanp = np.uint16(nan16 | 0x0123)                   # a NaN with a payload
    inf16, ninf16 = np.float16(np.inf).view(np.uint16), np.float16(-np.inf).view(np.uint16)
    plain = {(0, 7, 2): nan16, (1, 13, 5): inf16, (0, 33, 8): ninf16, (1, 118, 0): nanp}
    anchor = (1, 60, 1)                                # t = 60 anchors tokens 61..64
    group = {(1, t, 1) for t in range(61, 65)}
    new = set(plain) | (group if anchor_bits == 16 else {anchor})
    assert not (new | group | {anchor}) & base         # all on their grids in X
    Y = X.copy()
    for (kv, t, c), v in plain.items():
        Y[0, kv, t, c] = v
    Y[0, anchor[0], anchor[1], anchor[2]] = nan16
    enc = O.encode(on, Y, tab)
    got = entries(enc)
    if anchor_bits == 16:
        assert got == base | new
    else:
        # the NaN anchor is coded 0, so the group's deltas are taken against the lowest
        # point of the anchor grid and some of them may leave the delta grid
        assert base | new <= got <= base | new | group
    out = O.decode(on, tab, enc)
    for (kv, t, c) in got:
        assert out[0, kv, t, c] == Y[0, kv, t, c]
    if anchor_bits == 16:                              # the anchor row itself is exact
        assert out[0, anchor[0], anchor[1], anchor[2]] == nan16
    tab_off = O.Tables(tab.lo, tab.w, tab.r, tab.counts, tab.freqs, tab.alo, tab.aw, tab.ar)
    e_off = O.encode(off, Y, tab_off)
    assert e_off.clamped == len(got) and e_off.n_outliers == 0


def test_outlier_brute_force_tiny():
    """L=1, S=30, C=2, G=3, N=4, 10% budget: the clipped range, the entries and the
    decode worked out from exact rationals and a sort."""
    rng = np.random.default_rng(4)
    x = rng.standard_t(2, size=(1, 2, 30, 2)) * 2
    X = np.ascontiguousarray(x.astype(np.float16).view(np.uint16))
    shp = O.Shape.make(1, 1, 2, 30, 3, 30, [4], outlier_ppm=100000)
    tab = O.build_tables(shp, X)
    enc = O.encode(shp, X, tab)
    out = O.decode(shp, tab, enc)
    xf = X.view(np.float16)
    n_entries = 0
    for kv in range(2):
        for c in range(2):
            D = {t: Fraction(float(np.float32(np.float32(xf[0, kv, t, c]) -
                                              np.float32(xf[0, kv, t - t % 3, c]))))
                 for t in range(30) if t % 3}
            vals = sorted(D.values())
            n, b = len(vals), len(vals) // 10
            lo_c, w = Fraction(float(tab.lo[0, kv, c])), Fraction(float(tab.w[0, kv, c]))
            hi_c = lo_c + 3 * w
            assert sum(v < lo_c for v in vals) <= b and sum(v > hi_c * (1 + Fraction(1, 2 ** 20)) for v in vals) <= b
            for t, d in D.items():
                dist = min(abs(d - (lo_c + j * w)) for j in range(4))
                if dist > w / 2 * (1 + Fraction(1, 2 ** 20)):
                    n_entries += 1
                    assert out[0, kv, t, c] == X[0, kv, t, c]
                else:
                    y = Fraction(float(xf[0, kv, t - t % 3, c])) + lo_c + \
                        min(range(4), key=lambda j: (abs(d - (lo_c + j * w)), -j)) * w
                    got = Fraction(float(out[0, kv, t, c].view(np.float16)))
                    assert abs(got - y) <= abs(y) * Fraction(1, 2 ** 10) + Fraction(1, 2 ** 20)
    assert n_entries == enc.n_outliers and n_entries > 0


# --------------------------------------------------------------------------- stored bytes
def _parse_header(buf):
    import struct
    u32 = struct.unpack_from("<14I", buf, 0)
    u64 = struct.unpack_from("<13Q", buf, 56)
    return dict(zip(O.HEADER_U32, u32)) | dict(zip(O.HEADER_U64, u64))


@pytest.mark.parametrize("ppm,anchor_bits,n_sink,rng", [(0, 16, 0, None), (30000, 16, 5, None),
                                                         (30000, 8, 5, (1, 3)), (0, 8, 200, (0, 2)),
                                                         (0, 16, 900, None)])
def test_container_and_table_bytes_follow_their_layout(ppm, anchor_bits, n_sink, rng):
    """The stored bytes: every section 256-byte aligned after a 160-byte header, in the
    order offsets, anchors, sinks, outlier offsets / keys / values, payload, with the
    sizes their arrays give, zero bytes between sections and 1 KiB of zeros after the
    payload; the tables' 56-byte header, bins, lo, w (alo, aw), then N frequencies per
    channel row."""
    L, S, C, G, Tc = 2, 260, 70, 10, 64
    _, X = _small_data(L=L, S=S, C=C, G=G, Tc=Tc, bins=(8, 8), seed=9)
    shp = O.Shape.make(L, 1, C, S, G, Tc, (8, 5), n_sink=n_sink, anchor_bits=anchor_bits,
                       outlier_ppm=ppm)
    tab = O.build_tables(shp, X)
    kb, ke = rng if rng else (0, shp.n_chunks)
    enc = O.encode(shp, X, tab, kb, ke)
    buf = O.container_bytes(shp, enc)
    h = _parse_header(buf)
    assert h["magic"] == 0x31474B43 and h["version"] == 3 and h["total_bytes"] == len(buf)
    assert (h["L"], h["H_kv"], h["d"], h["S"], h["group"], h["chunk"]) == (L, 1, C, S, G, Tc)
    assert (h["chunk_begin"], h["chunk_end"], h["n_blocks"]) == (kb, ke, 2)
    ng = (ke - kb) * L * 2 * 2
    sa, sb = kb * Tc, max(kb * Tc, min(ke * Tc, S, n_sink))
    secs = [("offsets_offset", (ng + 1) * 8),
            ("anchors_offset", enc.anchors.nbytes),
            ("sinks_offset", 2 * L * (sb - sa) * C * 2),
            ("outliers_offset", (ng + 1) * 8 if ppm else 0),
            ("outlier_keys_offset", enc.n_outliers * 4),
            ("outlier_values_offset", enc.n_outliers * 2),
            ("payload_offset", enc.payload.size * 2)]
    end = 160
    for name, size in secs:
        off = h[name]
        assert off % 256 == 0 and off >= end and off - end < 256 and not any(buf[end:off])
        end = off + size
    assert h["anchors_bytes"] == enc.anchors.nbytes and h["n_sink"] == sb - sa
    assert h["payload_words"] == enc.payload.size and h["n_outliers"] == enc.n_outliers
    assert len(buf) == end + 1024 and not any(buf[end:])
    p = h["payload_offset"]
    assert np.array_equal(np.frombuffer(buf, np.uint16, enc.payload.size, p), enc.payload)
    assert np.array_equal(np.frombuffer(buf, np.uint64, ng + 1, h["offsets_offset"]), enc.offsets)
    if sb > sa:
        got = np.frombuffer(buf, np.uint16, 2 * L * (sb - sa) * C, h["sinks_offset"])
        assert np.array_equal(got.reshape(L, 2, sb - sa, C), X[:, :, sa:sb])
    tb = O.tables_bytes(shp, tab)
    assert len(tb) == O.table_bytes(shp)
    import struct
    t32 = struct.unpack_from("<12I", tb, 0)
    assert t32[:2] == (0x31544743, 1)
    assert t32[2:11] == (L, 1, C, S, G, Tc, min(n_sink, S), anchor_bits, ppm)
    assert struct.unpack_from("<Q", tb, 48)[0] == len(tb)
    off = 56 + 4
    assert list(tb[56:56 + 2 * L]) == list(shp.bins)
    lo = np.frombuffer(tb, np.float32, 2 * L * C, off)
    assert np.array_equal(lo, tab.lo.reshape(-1))
    off += 2 * L * C * 4 * (4 if anchor_bits == 8 else 2)
    fr = np.frombuffer(tb, np.uint16, (len(tb) - off) // 2, off)
    assert fr.size == C * sum(int(b) for b in shp.bins)
    assert int(fr[:8].astype(np.int64).sum()) == T   # the first channel row's table
