#!/usr/bin/env python3
"""Benchmark of the KV-cache codec on one MI355X.

One step = one pass of the whole hot path over the Llama-3-70B-shaped cache
(L=80, H_kv=8, d=128, S=32768, fp16, 10.74 GB; anchor interval 10, 1536-token chunks,
bins 32 / 16 / 8 for layers 0-19 / 20-39 / 40-79): cg_build_cdf (range, quantize,
histogram, frequency tables), cg_encode (delta + quantize, rANS coding, interleaving)
and cg_decode (rANS decode fused with dequantize + anchor-add) back to fp16.

Reported `value`: cg_decode throughput in GB/s of raw fp16 KV reconstructed (the
metric), from HIP events around each decode on the stream it runs on, averaged over
`--decode-reps` back-to-back decodes of the last step's container after the timed steps
and two untimed decodes (the container resident in HBM).  `decode_ms_in_step` is the decode inside the steps,
right after each step's encode.  `ms_per_step` is the wall time of a whole step.

Beside it: the encode (cg_build_cdf + cg_encode) time and % of HBM, a measured device copy
bandwidth, bits per symbol against the empirical entropy per bin tier, and the oracle's
encode and decode throughput on the host CPUs (`cpu_baseline`).

An object "paged" decodes the same container into a paged cache (16-token pages, a
shuffled block table); "outliers" codes the cache with the sparse outlier table (ratio,
entries, error, decode throughput); "kv_asymmetric" covers the same cache with the V rows
one step coarser than the K rows, "sinks" with the first four tokens kept in fp16, and
"anchors8" with 8-bit anchors (decode throughput and ratio).  An object "streamed" covers the streamed
decode of the 131K-token cache
(L=80, S=131072, 42.95 GB): every chunk encoded at three levels, one level per chunk
chosen from a seeded bandwidth trace, the chosen containers copied from pinned host
memory on one HIP stream while earlier chunks decode on another.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-streamed]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, vendor figure
METRIC = "cg_decode GB/s of raw fp16 KV reconstructed (% HBM peak); compression ratio"
CPU_SAMPLE_LAYERS = tuple(range(0, 80, 5))   # 16 layers; bin tiers 32:16:8 in the ratio 2:2:4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k3_decode_llama3_70b_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the sources the decode kernel is built from."""
    csrc = os.path.join(ROOT, "kv_cache_compression_cg_amd", "csrc")
    h = hashlib.sha256()
    for name in ("cg_kernels_decode.hip", "cg_device.h", "cg_internal.h"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def table_bytes_read(tables) -> int:
    """Decode-table bytes the decoder stages into LDS: per (layer, K/V, 64-channel
    block), bins entries x 64 lanes x 4 bytes plus the 256-slot x 64-lane byte table."""
    nb = -(-tables.C // 64)
    return sum(nb * (b * 64 * 4 + 256 * 64) for b in tables.row_bins)


def measured_traffic(alg_bytes: float):
    """HBM bytes per decode launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters, if they were taken on the current kernel source."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def host_info() -> dict:
    """Host CPU facts for the oracle leg: logical CPUs, the ones this process may use,
    the cgroup CPU quota if any, and the CPU model."""
    info = {"nproc": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        info["cgroup_cpu_quota"] = None if q == "max" else round(int(q) / int(per), 2)
    except (OSError, ValueError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return info


def cpu_baseline(w, X, max_threads: int, gpu_out=None) -> dict:
    """The oracle (as it stands) encoding and decoding a bounded sample of the same
    workload: 16 of the 80 layers (every fifth, the bin tiers in the workload's 2:2:4
    ratio), all chunks, K and V.  Encode = tables (range, quantize, histogram,
    frequencies) + coding of every chunk; decode = every chunk back to fp16.  Layers and
    chunk ranges are spread over a thread pool of the host CPUs this GPU's share allows.
    With gpu_out (the GPU's decode of the whole cache), the sampled layers of both decodes
    must be equal bit for bit (a layer's tables and decoded values do not depend on the
    other layers)."""
    import numpy as np
    import torch

    import oracle as O

    hinfo = host_info()
    avail = hinfo.get("affinity") or os.cpu_count() or 1
    if hinfo.get("cgroup_cpu_quota"):
        avail = min(avail, max(1, int(hinfo["cgroup_cpu_quota"])))
    cores = max(1, min(max_threads, avail))
    layers = CPU_SAMPLE_LAYERS
    host = {l: np.ascontiguousarray(X[l:l + 1].cpu().view(torch.int16).numpy().view(np.uint16))
            for l in layers}
    shapes = {l: O.Shape.make(1, w.H_kv, w.d, w.S, w.group, w.chunk, [w.bins[l]]) for l in layers}
    with cf.ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        tabs = dict(zip(layers, ex.map(lambda l: O.build_tables(shapes[l], host[l]), layers)))
        t_tab = time.perf_counter() - t0
        # split each layer into chunk ranges so the work spreads over every thread
        per = max(1, -(-w.n_chunks * len(layers) // (2 * cores)))
        items = [(l, k0, min(k0 + per, w.n_chunks)) for l in layers
                 for k0 in range(0, w.n_chunks, per)]
        t0 = time.perf_counter()
        encs = list(ex.map(lambda it: O.encode(shapes[it[0]], host[it[0]], tabs[it[0]],
                                               it[1], it[2]), items))
        t_enc = time.perf_counter() - t0
        outs = {l: np.zeros((1, 2, w.S, w.C), np.uint16) for l in layers}
        t0 = time.perf_counter()
        list(ex.map(lambda ie: O.decode(shapes[ie[0][0]], tabs[ie[0][0]], ie[1],
                                        out=outs[ie[0][0]]), zip(items, encs)))
        t_dec = time.perf_counter() - t0
    tt = np.arange(w.S)
    anchor = ((tt % w.chunk) % w.group) == 0
    for l in layers:
        assert np.array_equal(outs[l][:, :, anchor], host[l][:, :, anchor])
        if gpu_out is not None:
            g = gpu_out[l:l + 1].cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(outs[l], g), "oracle and GPU decodes differ on layer %d" % l
    raw = len(layers) * 2 * w.C * w.S * 2
    log("[cpu] oracle on %d threads: tables %.2fs, encode %.2fs, decode %.2fs (%.2f GB raw)"
        % (cores, t_tab, t_enc, t_dec, raw / 1e9))
    res = {"value": round(raw / t_dec / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": "oracle decode of layers %s (all %d chunks, K and V; %.2f GB raw), "
                     "%d threads over (layer, chunk-range) items, %.2fs wall"
                     % (list(layers), w.n_chunks, raw / 1e9, cores, t_dec),
           "decode_GBps": round(raw / t_dec / 1e9, 4),
           "encode_GBps": round(raw / (t_tab + t_enc) / 1e9, 4),
           "encode_s": {"tables": round(t_tab, 3), "coding": round(t_enc, 3)},
           "decode_s": round(t_dec, 3), "sample_raw_bytes": raw,
           "equals_gpu_decode": gpu_out is not None}
    res.update(hinfo)
    return res


def copy_bandwidth(dev, reps: int = 5, nbytes: int = 4 << 30) -> dict:
    """A plain device-to-device copy (torch, one kernel) of 4 GiB, timed with HIP events:
    read + write bytes per second, the practical HBM ceiling on this machine."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    del src, dst
    torch.cuda.empty_cache()
    gbps = 2 * nbytes / (ms[len(ms) // 2] * 1e-3) / 1e9
    return {"bytes": nbytes, "reps": reps, "median_ms": round(ms[len(ms) // 2], 4),
            "GBps_read_plus_write": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}


def access_form_bandwidth(dev, reps: int = 5, nbytes: int = 4 << 30) -> dict:
    """HBM rate of the decoder's own access forms alone, 4 GiB each (libcg_calib.so,
    grid-stride kernels of 2048 x 256 threads), timed with HIP events: 2-byte
    non-temporal stores, 128 contiguous bytes per wavefront (the output rows), 4-byte ones
    (256 bytes per wavefront, for comparison), 4- and 2-byte non-temporal loads (payload
    words, anchor rows), and a plain streaming read of 16-byte loads (the rate the
    encoder's passes over the cache could reach).  The store rate bounds how fast the
    decoder can write its rows however little it computes."""
    import ctypes

    import torch

    from kv_cache_compression_cg_amd import build as _b
    calib = ctypes.CDLL(_b.CALIB_LIB)
    calib.cg_calib_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64,
                                   ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2048, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    res = {"bytes": nbytes, "reps": reps}
    for kind, name in ((2, "write2_nt"), (3, "write4_nt"), (0, "read4_nt"), (1, "read2_nt"),
                       (4, "read16_nt")):
        assert calib.cg_calib_run(kind, buf.data_ptr(), nbytes, sink.data_ptr(), sp) == 0
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            assert calib.cg_calib_run(kind, buf.data_ptr(), nbytes, sink.data_ptr(), sp) == 0
            e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
        res[name + "_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    return res


def entropy_report(w, X, tab, blob) -> dict:
    """Bits per coded symbol against the empirical entropy, per bin tier: the symbols
    (cg_quantize) counted per channel row over the coded tokens, H_emp = sum n H(counts/n),
    the tables' cross-entropy sum count * log2(256 / f), and the payload's 16 bits per word
    (the groups' word counts from the container's offsets)."""
    import numpy as np
    import torch

    from kv_cache_compression_cg_amd import cg
    dev = X.device
    tt = torch.arange(w.S, device=dev)
    coded = ((tt % w.chunk) % w.group) != 0
    freqs = torch.from_numpy(tab.export()["freqs"].astype(np.float64)).to(dev)  # [L,2,C,32]
    offs = blob.offsets().astype(np.int64)
    words = offs[1:] - offs[:-1]
    NB = -(-w.C // 64)
    per_layer = words.reshape(w.n_chunks, w.L, 2, NB).sum(axis=(0, 2, 3))
    tiers = {}
    sym = cg.quantize(tab, X)                          # uint8 [L, 2, S, C]
    for l in range(w.L):
        s = sym[l][:, coded].long()                     # [2, T, C]
        idx = (torch.arange(2 * w.C, device=dev).view(2, 1, w.C) * 32 + s).reshape(-1)
        cnt = torch.bincount(idx, minlength=2 * w.C * 32).double().view(2, w.C, 32)
        n = cnt.sum(-1, keepdim=True)
        p = cnt / n.clamp_min(1)
        h_emp = float(-(cnt * torch.log2(p.clamp_min(1e-300))).sum())
        f = freqs[l]
        h_tab = float((cnt * torch.log2(256.0 / f.clamp_min(1))).sum())
        b = w.bins[l]
        t = tiers.setdefault(str(b), {"layers": 0, "symbols": 0, "H_emp_bits": 0.0,
                                      "table_bits": 0.0, "payload_bits": 0})
        t["layers"] += 1
        t["symbols"] += int(n.sum())
        t["H_emp_bits"] += h_emp
        t["table_bits"] += h_tab
        t["payload_bits"] += int(per_layer[l]) * 16
    del sym
    out = {}
    for b, t in tiers.items():
        m = t["symbols"]
        out["bins_" + b] = {"layers": t["layers"], "symbols": m,
                            "H_emp_bits_per_symbol": round(t["H_emp_bits"] / m, 4),
                            "table_cross_entropy_bits_per_symbol": round(t["table_bits"] / m, 4),
                            "payload_bits_per_symbol": round(t["payload_bits"] / m, 4),
                            "payload_over_H_emp": round(t["payload_bits"] / t["H_emp_bits"], 4)}
    torch.cuda.empty_cache()
    return out


def streamed_report(dev, n_slots: int = 32, reps: int = 3, seed: int = 0) -> dict:
    """The 131K-token cache streamed chunk by chunk from pinned host memory, each chunk
    at the level its bandwidth-trace entry allows, decoded while later chunks copy."""
    import numpy as np
    import torch

    from kv_cache_compression_cg_amd import configs, streamed, synth

    w = configs.LLAMA3_70B_131K
    t = time.time()
    X = synth.gen_kv(w, device=dev)
    prep = streamed.prepare(X, w.group, w.chunk, w.levels, H_kv=w.H_kv, seed=seed)
    log("[streamed] %s: %d chunks encoded at %d levels, chosen containers in pinned memory "
        "(%.1fs)" % (w.name, w.n_chunks, len(w.levels), time.time() - t))
    out = torch.empty_like(X)
    # one pipeline (staging slots and streams) for every run below: slots fit any chunk's
    # container at any level
    pipe = streamed.Pipeline(prep, dev, n_slots, slot_bytes=int(prep.sizes.max()))
    runs = [streamed.run(prep, out, n_slots=n_slots, pipe=pipe) for _ in range(reps + 1)][1:]
    tt = torch.arange(w.S, device=dev)
    anchor = ((tt % w.chunk) % w.group) == 0
    assert torch.equal(out[:, :, anchor].view(torch.int16), X[:, :, anchor].view(torch.int16))
    mean = {k: sum(r[k] for r in runs) / len(runs) for k in ("total_ms", "copy_ms", "decode_ms")}
    copied = runs[0]["copied_bytes"]
    raw = w.raw_bytes
    chunk_raw = np.array([2 * w.L * w.C * min(w.chunk, w.S - k * w.chunk) * 2
                          for k in range(w.n_chunks)], dtype=np.float64)
    lv, cnt = np.unique(prep.levels, return_counts=True)
    res = {
        "workload": w.name, "L": w.L, "H_kv": w.H_kv, "d": w.d, "S": w.S, "chunk": w.chunk,
        "group": w.group, "raw_bytes": raw, "chunks": w.n_chunks,
        "levels": "bins 32/16/8, 16/8/4, 8/4/2 for layers 0-19 / 20-39 / 40-79",
        "chunks_per_level": {str(int(a)): int(b) for a, b in zip(lv, cnt)},
        "streamed_bytes": copied, "table_bytes": prep.table_bytes,
        "compression_ratio": round(raw / (copied + prep.table_bytes), 4),
        "n_slots": n_slots, "reps": reps,
        "total_ms": round(mean["total_ms"], 3), "copy_ms": round(mean["copy_ms"], 3),
        "decode_ms": round(mean["decode_ms"], 3),
        "end_to_end_GBps": round(raw / (mean["total_ms"] * 1e-3) / 1e9, 2),
        "decode_only_GBps": round(raw / (mean["decode_ms"] * 1e-3) / 1e9, 2),
        "h2d_GBps": round(copied / (mean["copy_ms"] * 1e-3) / 1e9, 2),
        "overlap": round((mean["copy_ms"] + mean["decode_ms"] - mean["total_ms"])
                         / min(mean["copy_ms"], mean["decode_ms"]), 4),
        "network_s_trace": round(streamed.network_seconds(prep.sizes, prep.levels,
                                                          prep.bw_gbps), 4),
        "raw_fp16_network_s_trace": round(float(np.sum(chunk_raw * 8 / (prep.bw_gbps * 1e9))), 4),
    }
    log("[streamed] end-to-end %.1f GB/s raw-equivalent (copies %.1f GB/s, decode-only "
        "%.1f GB/s, overlap %.2f), ratio %.3f"
        % (res["end_to_end_GBps"], res["h2d_GBps"], res["decode_only_GBps"], res["overlap"],
           res["compression_ratio"]))
    sizes = prep.sizes
    del prep
    res["controller"] = controller_report(w, X, out, n_slots, sizes,
                                          streamed.bandwidth_trace(w.n_chunks, seed),
                                          "uniform 1-25 Gbit/s per chunk", pipe)
    # a link whose rate drifts: the estimator has something to follow
    res["controller_correlated"] = controller_report(
        w, X, out, n_slots, sizes, streamed.correlated_trace(w.n_chunks, seed),
        "log-rate AR(1), lag-one correlation 0.97, clipped to 1-25 Gbit/s", pipe)
    del pipe
    del out, X
    torch.cuda.empty_cache()
    return res


CONTROLLER_PREFILL_TOK_S = 4000.0  # modelled recompute rate of the text fallback


def controller_report(w, X, out, n_slots: int, sizes, bw, kind: str, pipe=None) -> dict:
    """The closed-loop controller choosing the levels over one bandwidth trace.  The SLO
    is the time the reference level (level 1 for every chunk) takes over the trace; the
    open-loop rule's time (which knows every chunk's rate in advance) is given beside it.
    The controller estimates the link from the chunks already sent (an average of the time
    per bit, newest chunk weighted 0.8), plans the remaining chunks at the lower of that
    estimate and the last rate against 95% of the SLO, spends a quarter of its slack, and
    falls back to text
    where recomputing (at a modelled 4000 tokens/s) is predicted to be faster than the
    coarsest container of a late chunk.  The chosen containers are streamed and decoded
    once; text chunks are not.  `sizes`: container bytes [levels][chunks]."""
    import numpy as np
    import torch

    from kv_cache_compression_cg_amd import streamed
    n = w.n_chunks
    tokens = [min(w.chunk, w.S - k * w.chunk) for k in range(n)]
    ref = np.full(n, streamed.REFERENCE_LEVEL)
    slo_s = streamed.network_seconds(sizes, ref, bw)
    open_loop_s = streamed.network_seconds(sizes, streamed.choose_levels(sizes, bw), bw)
    ctl = streamed.ControllerConfig(slo_s=slo_s, prior_gbps=13.0, alpha=0.8, slack_share=0.25,
                                    cautious=True, harmonic=True, margin=0.05,
                                    prefill_tok_per_s=CONTROLLER_PREFILL_TOK_S)
    prep = streamed.prepare(X, w.group, w.chunk, w.levels, H_kv=w.H_kv, trace=bw,
                            controller=ctl, sizes=sizes)
    levels, est, fetch_s = streamed.control_levels(prep.sizes, bw, tokens, ctl)
    stats = streamed.run(prep, out, n_slots=n_slots, pipe=pipe)
    torch.cuda.synchronize()
    lv, cnt = np.unique(levels, return_counts=True)
    names = {streamed.TEXT: "text"}
    ref_bytes = int(np.asarray(sizes)[streamed.REFERENCE_LEVEL].sum())
    res = {"trace": kind, "slo": "reference level (1) for every chunk over the trace",
           "slo_s": round(slo_s, 4), "open_loop_fetch_s": round(open_loop_s, 4),
           "prefill_tok_per_s_model": CONTROLLER_PREFILL_TOK_S,
           "alpha": ctl.alpha, "prior_gbps": ctl.prior_gbps, "slack_share": ctl.slack_share,
           "cautious": ctl.cautious, "harmonic": ctl.harmonic, "margin": ctl.margin,
           "chunks_per_level": {names.get(int(a), str(int(a))): int(b) for a, b in zip(lv, cnt)},
           "fetch_s_trace": round(fetch_s, 4), "slo_met": bool(fetch_s <= slo_s),
           "rate_estimate_median_rel_error": round(float(np.median(np.abs(est[1:] - bw[1:])
                                                                     / bw[1:])), 4),
           "streamed_bytes": prep.streamed_bytes, "reference_level_bytes": ref_bytes,
           "total_ms": round(stats["total_ms"], 3), "decode_ms": round(stats["decode_ms"], 3)}
    log("[controller] %s: levels %s, fetch %.2f s over the trace (SLO %.2f s, open loop %.2f s), "
        "estimate off by %.0f%% (median), streamed %.2f GB (reference level %.2f GB)"
        % (kind, res["chunks_per_level"], fetch_s, slo_s, open_loop_s,
           100 * res["rate_estimate_median_rel_error"], prep.streamed_bytes / 1e9,
           ref_bytes / 1e9))
    del prep
    return res


PAGE_TOKENS = 16
DECODE_WARMUP = 2  # untimed decodes before the timed ones of the decode phase


def paged_report(w, tab, blob, out, reps: int) -> dict:
    """The same container decoded into a paged cache (the Guide's Best Practices: write
    straight into the serving engine's KV blocks): 16-token pages, a seeded shuffled
    block table, back-to-back decodes; checked against the contiguous decode in `out`
    on the first and last layer."""
    import torch

    from kv_cache_compression_cg_amd import cg
    nb = -(-w.S // PAGE_TOKENS)
    gen = torch.Generator().manual_seed(0)
    bt = torch.randperm(nb, generator=gen).to(torch.int32).to(out.device)
    pages = torch.empty((w.L, 2, nb, PAGE_TOKENS, w.C), dtype=torch.float16, device=out.device)
    stream = torch.cuda.current_stream(out.device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps + 2)]
    for e0, e1 in ev:
        e0.record(stream)
        cg.decode_paged(tab, blob, pages, bt)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev[2:]]
    dec = sum(ms) / len(ms)
    for l in (0, w.L - 1):
        got = pages[l][:, bt.long()].reshape(2, nb * PAGE_TOKENS, w.C)[:, :w.S]
        assert torch.equal(got.view(torch.int16), out[l].view(torch.int16))
    res = {"workload": w.name, "page_tokens": PAGE_TOKENS, "pages": nb,
           "block_table": "seeded permutation", "decode_ms": round(dec, 4),
           "decode_reps": len(ms), "value_GBps": round(w.raw_bytes / (dec * 1e-3) / 1e9, 2),
           "pct_hbm_peak": round(100 * w.raw_bytes / (dec * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
    log("[paged] decode into %d-token pages %.3f ms (%.1f GB/s)"
        % (PAGE_TOKENS, dec, res["value_GBps"]))
    del pages
    torch.cuda.empty_cache()
    return res


def _variant_decode(w, X, out, reps: int, **build_kw):
    """Tables and container of a format variant of the cache, then back-to-back decodes
    of the resident container; checks anchors exact and the half-bin bound on layer 0."""
    import torch

    from kv_cache_compression_cg_amd import cg
    tab = cg.build_cdf(X, w.group, w.chunk, w.bins, H_kv=w.H_kv, **build_kw)
    blob = cg.encode(tab, X)
    stream = torch.cuda.current_stream(X.device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps + 2)]
    for e0, e1 in ev:
        e0.record(stream)
        cg.decode(tab, blob, out)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev[2:]]
    dec = sum(ms) / len(ms)
    tt = torch.arange(w.S, device=X.device)
    anchor = ((tt % w.chunk) % w.group) == 0
    a8 = build_kw.get("anchor_bits", 16) == 8
    if not a8:  # 8-bit anchors are within half a step of their own grid instead
        assert torch.equal(out[:, :, anchor].view(torch.int16), X[:, :, anchor].view(torch.int16))
    n_sink = build_kw.get("n_sink", 0)
    keep = (tt >= n_sink) & ~anchor if a8 else tt >= n_sink
    wv = torch.from_numpy(tab.export()["w"][0]).to(X.device)[:, None, :]
    err = (X[0][:, keep].float() - out[0][:, keep].float()).abs()
    assert bool((err <= wv / 2 * 1.001 + 2 ** -10 * X[0][:, keep].float().abs() + 1e-6).all())
    comp = cg.compressed_bytes(tab, [blob])
    res = {"workload": w.name, "decode_ms": round(dec, 4), "decode_reps": len(ms),
           "value_GBps": round(w.raw_bytes / (dec * 1e-3) / 1e9, 2),
           "pct_hbm_peak": round(100 * w.raw_bytes / (dec * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
           "compression_ratio": round(w.raw_bytes / comp, 4), "compressed_bytes": comp}
    del blob, tab
    return res


def kv_asymmetric_report(w, X, out, reps: int) -> dict:
    """Keys finer than values ("Guide to CacheGen", Solution pillar 1): the V rows take one
    step coarser bin counts than the K rows (K 32 / 16 / 8, V 16 / 8 / 4 by layer tier).
    Decode throughput over back-to-back decodes of the resident container, and the ratio."""
    res = {"bins_k": "32 / 16 / 8 (layers 0-19 / 20-39 / 40-79)", "bins_v": "16 / 8 / 4"}
    res.update(_variant_decode(w, X, out, reps, bins_v=[max(2, b // 2) for b in w.bins]))
    log("[kv-asymmetric] decode %.3f ms (%.1f GB/s), ratio %.3f"
        % (res["decode_ms"], res["value_GBps"], res["compression_ratio"]))
    return res


def anchors8_report(w, X, out, reps: int) -> dict:
    """8-bit anchors ("Guide to CacheGen", Solution pillar 2: the anchor quantized with
    high precision): each anchor a code on a 256-level grid of its channel, the deltas
    taken against the grid value; half the anchor bytes."""
    res = {"anchor_bits": 8}
    res.update(_variant_decode(w, X, out, reps, anchor_bits=8))
    log("[anchors8] decode %.3f ms (%.1f GB/s), ratio %.3f"
        % (res["decode_ms"], res["value_GBps"], res["compression_ratio"]))
    return res


def sinks_report(w, X, out, reps: int, n_sink: int = 4) -> dict:
    """Attention sinks ("Guide to CacheGen", Best Practices): the first four tokens kept
    in fp16 and out of the tables; the decode writes them back exactly (checked)."""
    import torch
    res = {"n_sink": n_sink}
    res.update(_variant_decode(w, X, out, reps, n_sink=n_sink))
    assert torch.equal(out[:, :, :n_sink].view(torch.int16), X[:, :, :n_sink].view(torch.int16))
    log("[sinks] decode %.3f ms (%.1f GB/s), ratio %.3f"
        % (res["decode_ms"], res["value_GBps"], res["compression_ratio"]))
    return res


OUTLIER_PPM = 1000          # 0.1% of each channel row's deltas may fall out at each end
ERROR_LAYERS = (0, 40, 79)  # one layer of each bin tier


def outliers_report(w, X, out_plain, tab_plain, reps: int) -> dict:
    """Sparse outlier table ("Guide to CacheGen", Solution pillar 3): each channel row's
    grid spans the central range leaving at most 0.1% of its deltas out at each end, and
    every element off the grid is stored exactly.  Reported: the ratio and the entries,
    the decode throughput over back-to-back decodes, the narrowing of the bin widths, and
    the reconstruction error against the plain codec on one layer of each bin tier."""
    import numpy as np
    import torch

    from kv_cache_compression_cg_amd import cg
    tab = cg.build_cdf(X, w.group, w.chunk, w.bins, H_kv=w.H_kv, outlier_ppm=OUTLIER_PPM)
    blob = cg.encode(tab, X)
    out = torch.empty_like(X)
    stream = torch.cuda.current_stream(X.device)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps + 2)]
    for e0, e1 in ev:
        e0.record(stream)
        cg.decode(tab, blob, out)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev[2:]]
    dec = sum(ms) / len(ms)
    h = blob.header
    w_full, w_clip = tab_plain.export()["w"], tab.export()["w"]
    ok = w_full > 0
    narrow = np.median(w_clip[ok] / w_full[ok])
    errs = {}
    for name, y in (("plain", out_plain), ("outliers", out)):
        tot, n, mx = 0.0, 0, 0.0
        for l in ERROR_LAYERS:
            e = (X[l].float() - y[l].float()).abs()
            wf = torch.from_numpy(w_full[l]).to(X.device)[:, None, :]
            tot += float(e.double().sum())
            n += e.numel()
            mx = max(mx, float((e / (wf / 2).clamp_min(1e-30)).max()))
        errs[name] = {"mean_abs_error": tot / n, "max_error_over_full_half_bin": round(mx, 4)}
    comp = cg.compressed_bytes(tab, [blob])
    res = {"outlier_ppm": OUTLIER_PPM, "workload": w.name,
           "n_outliers": int(h["n_outliers"]),
           "outlier_fraction": round(h["n_outliers"] / (w.raw_bytes / 2), 6),
           "outlier_section_bytes": int(h["payload_offset"] - h["outliers_offset"]),
           "compression_ratio": round(w.raw_bytes / comp, 4), "compressed_bytes": comp,
           "median_bin_width_clipped_over_full": round(float(narrow), 4),
           "error_layers": list(ERROR_LAYERS), "error": errs,
           "mean_abs_error_ratio": round(errs["outliers"]["mean_abs_error"]
                                         / errs["plain"]["mean_abs_error"], 4),
           "decode_ms": round(dec, 4), "decode_reps": len(ms),
           "value_GBps": round(w.raw_bytes / (dec * 1e-3) / 1e9, 2),
           "pct_hbm_peak": round(100 * w.raw_bytes / (dec * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
    log("[outliers] %d entries (%.4f%%), ratio %.3f, bin width x%.3f, mean |error| x%.3f, "
        "decode %.3f ms (%.1f GB/s)" % (res["n_outliers"], 100 * res["outlier_fraction"],
                                       res["compression_ratio"], narrow,
                                       res["mean_abs_error_ratio"], dec, res["value_GBps"]))
    del blob, tab, out
    torch.cuda.empty_cache()
    return res


def decode_loop(w, dev, n: int) -> dict:
    """One encode of the workload, then n decodes back to back on one stream, each timed
    with HIP events; the rest of the step is left out, so that a counter run or a power
    reading taken meanwhile sees the decoder alone."""
    import torch

    from kv_cache_compression_cg_amd import cg, synth
    X = synth.gen_kv(w, device=dev)
    tab = cg.build_cdf(X, w.group, w.chunk, w.bins, H_kv=w.H_kv)
    blob = cg.encode(tab, X)
    out = torch.empty_like(X)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    log("[decode-loop] %d decodes of %s" % (n, w.name))
    t0 = time.time()
    for e0, e1 in ev:
        e0.record(stream)
        cg.decode(tab, blob, out)
        e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.time() - t0
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return {"decode_loop": n, "workload": w.name, "raw_bytes": w.raw_bytes,
            "decode_ms_mean": round(sum(ms) / n, 4), "decode_ms_median": round(ms[n // 2], 4),
            "decode_ms_min": round(ms[0], 4), "wall_s": round(wall, 3),
            "GBps_mean": round(w.raw_bytes / (sum(ms) / n) / 1e6, 1)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_70b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-streamed", action="store_true",
                    help="skip the streamed decode of the 131K-token cache")
    ap.add_argument("--only-streamed", action="store_true",
                    help="run only the streamed decode of the 131K-token cache (profiling)")
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="oracle threads: the host CPUs one GPU's share of the box allows")
    ap.add_argument("--no-entropy", action="store_true",
                    help="skip the bits-per-symbol against empirical entropy report")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 4 GiB through a plain copy and through the decoder's access "
                         "forms (memory-counter calibration)")
    ap.add_argument("--no-kv-asymmetric", action="store_true",
                    help="skip the paged-output, keys-finer-than-values and sink objects")
    ap.add_argument("--decode-reps", type=int, default=20,
                    help="back-to-back decodes after the timed steps that give `value`")
    ap.add_argument("--decode-loop", type=int, default=0, metavar="N",
                    help="only encode the workload once and decode it N times back to back "
                         "(for counters and for sampling board power during the decode)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the codec runs on a single MI355X "
              "(sharding across GPUs is not built)", file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy:
        # known byte counts for the memory counters: a plain 4 GiB device copy (torch),
        # then 4 GiB through each of the decoder's access forms (libcg_calib.so):
        # 4-byte non-temporal loads, 2-byte non-temporal loads, 2-byte non-temporal stores
        import ctypes
        from kv_cache_compression_cg_amd import build as _b
        if not os.path.exists(_b.CALIB_LIB):
            _b.build()
        calib = ctypes.CDLL(_b.CALIB_LIB)
        calib.cg_calib_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_void_p]
        n = 4 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        sink = torch.zeros(2048, dtype=torch.int32, device="cuda:0")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(3):
            dst.copy_(src)
        for kind in (0, 1, 2):
            for _ in range(3):
                assert calib.cg_calib_run(kind, src.data_ptr(), n, sink.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_bytes": n, "reps": 3,
                          "kernels": ["copy (torch)", "read4_nt", "read2_nt", "write2_nt"]}),
              flush=True)
        return 0

    from kv_cache_compression_cg_amd import build, configs, synth
    if not os.path.exists(build.LIB):
        build.build()
    from kv_cache_compression_cg_amd import cg

    w = configs.ALL[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode_loop:
        print(json.dumps(decode_loop(w, dev, args.decode_loop)), flush=True)
        return 0
    if args.only_streamed:
        print(json.dumps({"streamed": streamed_report(dev)}), flush=True)
        return 0
    t = time.time()
    X = synth.gen_kv(w, device=dev)
    out = torch.empty_like(X)
    torch.cuda.synchronize()
    log("[bench] %s: generated %.2f GB in %.1fs" % (w.name, w.raw_bytes / 1e9, time.time() - t))

    stream = torch.cuda.current_stream(dev)

    def step():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ts = time.perf_counter()
        ev[0].record(stream)
        tab = cg.build_cdf(X, w.group, w.chunk, w.bins, H_kv=w.H_kv)
        blob = cg.encode(tab, X)
        ev[1].record(stream)
        tw = time.perf_counter()
        ev[2].record(stream)
        cg.decode(tab, blob, out)
        ev[3].record(stream)
        torch.cuda.synchronize()
        te = time.perf_counter()
        return (ev[2].elapsed_time(ev[3]), (te - ts) * 1e3, ev[0].elapsed_time(ev[1]),
                (tw - ts) * 1e3, tab, blob)

    copy = copy_bandwidth(dev)
    log("[bench] device copy of 4 GiB: %.1f GB/s read + write" % copy["GBps_read_plus_write"])
    forms = access_form_bandwidth(dev)
    forms["rows_of_the_decode_ms_at_write2_nt"] = round(w.raw_bytes / forms["write2_nt_GBps"]
                                                        / 1e6, 4)
    log("[bench] decoder access forms alone: %s" % json.dumps(forms))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs, last = [], None
    t0 = time.perf_counter()
    for _ in range(args.steps):
        last = None                      # the previous step's handles are released here
        dms, sms, ems, ewall, tab, blob = step()
        recs.append((dms, sms, ems, ewall))
        last = (tab, blob)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    tab, blob = last
    in_step_ms = [r[0] for r in recs]
    step_ms = [r[1] for r in recs]
    enc_ev_ms = [r[2] for r in recs]
    enc_wall_ms = [r[3] for r in recs]
    # Decode phase: cg_decode of the last step's container, back to back, each launch timed
    # with HIP events.  Inside a step the decode follows that step's encode directly and
    # runs while the encoder's freshly written container and scratch are still being
    # evicted; decoding a resident container is the operation the metric names (the pages'
    # encode is offline), so `value` is taken here and the in-step figure is reported too.
    # Two untimed decodes come first, as for the variant objects below: the first decodes
    # after the steps still overlap the eviction of the encoder's output.
    for _ in range(DECODE_WARMUP):
        cg.decode(tab, blob, out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.decode_reps)]
    for e0, e1 in ev:
        e0.record(stream)
        cg.decode(tab, blob, out)
        e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    dec_mean = sum(dec_ms) / len(dec_ms)
    dec_sorted = sorted(dec_ms)
    value = w.raw_bytes / (dec_mean * 1e-3) / 1e9

    # sanity: anchors bit-exact, first layer within half a bin
    tt = torch.arange(w.S, device=dev)
    anchor = ((tt % w.chunk) % w.group) == 0
    assert torch.equal(out[:, :, anchor].view(torch.int16), X[:, :, anchor].view(torch.int16))
    ex = tab.export()
    wv = torch.from_numpy(ex["w"][0]).to(dev)[:, None, :]
    err = (X[0].float() - out[0].float()).abs()
    assert bool((err <= wv / 2 * 1.001 + 2 ** -10 * X[0].float().abs() + 1e-6).all())

    comp = cg.compressed_bytes(tab, [blob])
    alg = w.raw_bytes + blob.nbytes + table_bytes_read(tab)
    achieved = alg / (dec_mean * 1e-3) / 1e9
    roofline = {"kernel": "k3_decode", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(alg),
                "algorithmic_bytes_per_launch": alg}
    h = blob.header
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32+f32", "data": "synthetic",
        "config": {"workload": w.name, "L": w.L, "H_kv": w.H_kv, "d": w.d, "S": w.S,
                   "group": w.group, "chunk": w.chunk,
                   "bins": "32 (layers 0-19) / 16 (20-39) / 8 (40-79)",
                   "raw_bytes": w.raw_bytes, "seed": w.gen.seed, "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "compression_ratio": round(w.raw_bytes / comp, 4),
        "compressed_bytes": {"total": comp, "payload": 2 * h["payload_words"],
                             "anchors": h["anchors_bytes"],
                             "header_offsets_padding": comp - 2 * h["payload_words"]
                             - h["anchors_bytes"] - tab.stored_bytes,
                             "tables": tab.stored_bytes},
        "value_loop": "decode phase: %d back-to-back cg_decode calls of the last step's "
                      "resident container, each timed with HIP events on the library's "
                      "stream, after %d untimed ones" % (len(dec_ms), DECODE_WARMUP),
        "decode_ms": round(dec_mean, 4), "decode_ms_min": round(dec_sorted[0], 4),
        "decode_ms_median": round(dec_sorted[len(dec_sorted) // 2], 4),
        "decode_ms_max": round(dec_sorted[-1], 4),
        "decode_reps": len(dec_ms), "decode_warmup": DECODE_WARMUP,
        "decode_ms_in_step": round(sum(in_step_ms) / len(in_step_ms), 4),
        "pct_hbm_peak_in_step": round(100 * w.raw_bytes / (sum(in_step_ms) / len(in_step_ms)
                                                          * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "target_pct_hbm_peak": 40.0,
        "encode_ms": round(sum(enc_ev_ms) / len(enc_ev_ms), 3),
        "encode_ms_wall": round(sum(enc_wall_ms) / len(enc_wall_ms), 3),
        "encode_timing": "cg_build_cdf + cg_encode, HIP events on the library's stream "
                         "before the first and after the last call (host work between "
                         "kernels included); wall: host clock around both calls",
        "copy": copy,
        "access_forms": forms,
        "roofline": roofline,
    }
    res["encode_GBps"] = round(w.raw_bytes / (res["encode_ms"] * 1e-3) / 1e9, 2)
    res["encode_pct_hbm_peak"] = round(100 * res["encode_GBps"] / HBM_PEAK_GBPS, 2)
    # The encode as HBM passes: the cache is read three times (min/max, histograms, the
    # fused coder), the coder writes the anchors and its words, the compaction reads the
    # words back and writes the payload.  The one-pass minimum (read the cache, write the
    # container) is reported beside it.
    payload_b = 2 * h["payload_words"]
    enc_bytes = 3 * w.raw_bytes + h["anchors_bytes"] + 3 * payload_b
    enc_s = res["encode_ms"] * 1e-3
    res["encode_roofline"] = {
        "kernels": "k0_minmax + k1_hist + k5_code + k5_compact (and the small table kernels)",
        "bound": "hbm", "achieved": round(enc_bytes / enc_s / 1e9, 1), "peak": HBM_PEAK_GBPS,
        "unit": "GB/s", "frac": round(enc_bytes / enc_s / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes_per_encode": enc_bytes,
        "one_pass_bytes": w.raw_bytes + blob.nbytes,
        "one_pass_frac": round((w.raw_bytes + blob.nbytes) / enc_s / 1e9 / HBM_PEAK_GBPS, 4)}
    log("[bench] decode %.3f ms (%.1f GB/s, %.1f%% of HBM peak; %.3f ms inside the steps), "
        "step %.1f ms, ratio %.3f" % (dec_mean, value, res["pct_hbm_peak"],
                                     res["decode_ms_in_step"], res["ms_per_step"],
                                     res["compression_ratio"]))
    if not args.no_entropy:
        res["entropy"] = entropy_report(w, X, tab, blob)
        log("[entropy] %s" % json.dumps(res["entropy"]))
    if not args.no_kv_asymmetric:
        res["paged"] = paged_report(w, tab, blob, out, args.decode_reps)
        res["outliers"] = outliers_report(w, X, out, tab, args.decode_reps)
        res["kv_asymmetric"] = kv_asymmetric_report(w, X, out, args.decode_reps)
        res["sinks"] = sinks_report(w, X, out, args.decode_reps)
        res["anchors8"] = anchors8_report(w, X, out, args.decode_reps)
    if not args.no_cpu_baseline:
        cg.decode(tab, blob, out)   # the main container again (the objects above reused `out`)
        torch.cuda.synchronize()
        res["cpu_baseline"] = cpu_baseline(w, X, args.cpu_threads, gpu_out=out)
    if not args.no_streamed:
        del X, out, tab, blob, last
        torch.cuda.empty_cache()
        res["streamed"] = streamed_report(dev)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
