"""Streamed decode of a long cache, each chunk at a compression level picked for the
bandwidth of the moment.

The pages have the cache sent chunk by chunk, each chunk's compression level set by the
available bandwidth, and GPU decoding running alongside the transfer: chunk i decodes
while chunk i+1 is in transit ("Guide to CacheGen", section 4, Overlapped Streaming
Decoder Pipeline; gptget summary of arXiv 2310.07240, Methodology).  They give no rule
for the choice.  The rule used here: each chunk has a deadline, the time its container at
the reference level would take at the trace's mean rate, and takes the finest level whose
container meets that deadline at the chunk's own rate, else the coarsest level.

Host logic only: the copies and decodes run in libcg (cg_stream_decode), on two HIP
streams.  32 staging slots by default: the chunks are decoded in windows of half the
slots, one launch per window.  The decoder stages one chunk's tables per block and a
block decodes only chunks that share them, so a window of 16 chunks over three levels
gives each block about five chunks; with one chunk a launch it fills too little of the
GPU.  With only two or three slots a copy that must wait for the decode freeing its slot
also leaves the copy engine idle for a while.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import cg

TRACE_LO_GBPS = 1.0
TRACE_HI_GBPS = 25.0
REFERENCE_LEVEL = 1


def bandwidth_trace(n_chunks: int, seed: int = 0) -> np.ndarray:
    """Per-chunk link rate in Gbit/s, uniform on [1, 25], seeded."""
    rng = np.random.default_rng([seed, 5])
    return rng.uniform(TRACE_LO_GBPS, TRACE_HI_GBPS, size=n_chunks)


def correlated_trace(n_chunks: int, seed: int = 0, rho: float = 0.97) -> np.ndarray:
    """Per-chunk link rate in Gbit/s that drifts rather than jumps: the log-rate follows a
    seeded AR(1) process around the geometric middle of [1, 25] with lag-one correlation
    rho, spread so that the stationary range covers [1, 25] at about two standard
    deviations, and is clipped to [1, 25].  A link whose rate persists from one chunk to
    the next is what a rate estimated from the chunks already sent can follow."""
    rng = np.random.default_rng([seed, 6])
    lo, hi = np.log(TRACE_LO_GBPS), np.log(TRACE_HI_GBPS)
    mu, sigma = 0.5 * (lo + hi), 0.25 * (hi - lo)
    z = np.empty(n_chunks)
    prev = rng.standard_normal()
    for k in range(n_chunks):
        prev = rho * prev + np.sqrt(1.0 - rho * rho) * rng.standard_normal() if k else prev
        z[k] = prev
    return np.clip(np.exp(mu + sigma * z), TRACE_LO_GBPS, TRACE_HI_GBPS)


def choose_levels(sizes: np.ndarray, bw_gbps: np.ndarray, ref_level: int = REFERENCE_LEVEL,
                  ref_gbps: Optional[float] = None) -> np.ndarray:
    """sizes: bytes [levels][chunks], level 0 the finest.  Returns the level per chunk."""
    sizes = np.asarray(sizes, dtype=np.float64)
    bw = np.asarray(bw_gbps, dtype=np.float64)
    n_levels, n = sizes.shape
    if bw.shape != (n,):
        raise ValueError("one rate per chunk expected")
    mean = 0.5 * (TRACE_LO_GBPS + TRACE_HI_GBPS) if ref_gbps is None else ref_gbps
    deadline = sizes[ref_level] * 8.0 / (mean * 1e9)
    out = np.full(n, n_levels - 1, dtype=np.int64)
    for k in range(n):
        for lv in range(n_levels):
            if sizes[lv, k] * 8.0 / (bw[k] * 1e9) <= deadline[k]:
                out[k] = lv
                break
    return out


TEXT = -1   # level of a chunk sent as text and recomputed instead of as KV


@dataclass
class ControllerConfig:
    """Closed-loop level choice under a fetch-time SLO.

    The pages have the compression level of each part of the context follow the bandwidth
    so that the fetch meets its delay objective, and fall back to sending text for the
    model to recompute when the bandwidth is too low (gptget summary of arXiv 2310.07240,
    Methodology and abstract; phantomic12 notes).  They give no estimator or rule; the
    ones here: the rate is estimated from the chunks already sent (an exponentially
    weighted mean of the rate, or with `harmonic` of its inverse, `alpha` on the newest).  The time left in the SLO first covers every
    remaining chunk at its coarsest level (at the estimate); what is left over, the
    slack, is shared equally, so chunk k may spend its coarsest time plus slack / (chunks
    left) and takes the finest level predicted to fit.  With a right estimate a feasible
    SLO is then always met.  When the slack is negative (the SLO cannot be met even at
    the coarsest level) and sending the chunk's tokens as text and recomputing them
    (`prefill_tok_per_s`, a modelled rate; 0 disables the fallback) is predicted to be
    faster than its coarsest container, the chunk falls back to text."""
    slo_s: float
    alpha: float = 0.5
    prior_gbps: float = 10.0
    prefill_tok_per_s: float = 0.0
    text_bytes_per_token: int = 4
    # the share of its slack a chunk may spend (1: all of it), and whether the remaining
    # chunks are budgeted at the lower of the estimate and the last measured rate (a
    # rate that has just fallen is then planned for before the estimate has caught up)
    slack_share: float = 1.0
    cautious: bool = False
    # average the time per bit (1 / rate) instead of the rate: a chunk's transfer time is
    # proportional to 1 / rate, and where the rate varies from chunk to chunk the mean of
    # 1 / rate exceeds 1 / (mean rate), so an average of the rate under-predicts times
    harmonic: bool = False
    # the share of the SLO held back: the controller plans against (1 - margin) x SLO, a
    # reserve for the chunks whose rates the estimate misses
    margin: float = 0.0


def control_levels(sizes: np.ndarray, bw_gbps: np.ndarray, chunk_tokens: Sequence[int],
                   cfg: ControllerConfig):
    """sizes: container bytes [levels][chunks], level 0 the finest; bw_gbps: the link
    rate each chunk actually meets (unknown to the controller until it has been sent).
    Returns (level per chunk, TEXT for a fallback chunk; the rate estimate each choice
    used; the simulated fetch time: transfers at the actual rates plus recomputation)."""
    sizes = np.asarray(sizes, dtype=np.float64)
    bw = np.asarray(bw_gbps, dtype=np.float64)
    n_levels, n = sizes.shape
    if bw.shape != (n,) or len(chunk_tokens) != n:
        raise ValueError("one rate and one token count per chunk expected")
    est = float(cfg.prior_gbps)
    last = est
    elapsed = 0.0
    levels = np.zeros(n, dtype=np.int64)
    estimates = np.zeros(n, dtype=np.float64)
    for k in range(n):
        estimates[k] = est
        pred = sizes[:, k] * 8.0 / (est * 1e9)
        plan = min(est, last) if cfg.cautious else est
        slack = (cfg.slo_s * (1.0 - cfg.margin) - elapsed
                 - float(np.sum(sizes[-1, k:])) * 8.0 / (plan * 1e9))
        allowed = pred[-1] + cfg.slack_share * max(slack, 0.0) / (n - k)
        choice = int(np.nonzero(pred <= allowed)[0][0])   # the coarsest level always fits
        text_bytes = float(chunk_tokens[k]) * cfg.text_bytes_per_token
        recompute = (float(chunk_tokens[k]) / cfg.prefill_tok_per_s
                     if cfg.prefill_tok_per_s > 0 else float("inf"))
        if slack < 0.0 and text_bytes * 8.0 / (est * 1e9) + recompute < pred[-1]:
            choice = TEXT
        sent = text_bytes if choice == TEXT else sizes[choice, k]
        elapsed += sent * 8.0 / (bw[k] * 1e9) + (recompute if choice == TEXT else 0.0)
        # the transfer just made measures the link rate of this chunk
        if cfg.harmonic:
            est = 1.0 / (cfg.alpha / bw[k] + (1.0 - cfg.alpha) / est)
        else:
            est = cfg.alpha * bw[k] + (1.0 - cfg.alpha) * est
        last = bw[k]
        levels[k] = choice
    return levels, estimates, elapsed


def network_seconds(sizes: np.ndarray, levels: np.ndarray, bw_gbps: np.ndarray) -> float:
    """Time to send the chosen containers over the trace (no overlap with decoding)."""
    sizes = np.asarray(sizes, dtype=np.float64)
    chosen = sizes[np.asarray(levels), np.arange(sizes.shape[1])]
    return float(np.sum(chosen * 8.0 / (np.asarray(bw_gbps, dtype=np.float64) * 1e9)))


@dataclass
class Prepared:
    tables: List[cg.Tables]       # one per level
    items: list                   # (Tables, Blob, pinned host tensor) per chunk, in order
    levels: np.ndarray            # chosen level per chunk
    sizes: np.ndarray             # container bytes [levels][chunks]
    bw_gbps: np.ndarray
    slot_bytes: int

    @property
    def streamed_bytes(self) -> int:
        return int(sum(b.nbytes for _, b, _ in self.items))

    @property
    def table_bytes(self) -> int:
        used = sorted(set(int(v) for v in self.levels if v != TEXT))
        return int(sum(self.tables[v].stored_bytes for v in used))


def prepare(kv: torch.Tensor, group: int, chunk: int, level_bins: Sequence[Sequence[int]],
            H_kv: int, seed: int = 0, force_levels: Optional[Sequence[int]] = None,
            controller: Optional[ControllerConfig] = None,
            trace: Optional[np.ndarray] = None,
            sizes: Optional[np.ndarray] = None) -> Prepared:
    """Builds the tables of every level, encodes every chunk at every level, picks one
    level per chunk and keeps that container in pinned host memory.  A chunk at level
    TEXT (recomputed from text) is not kept.  With `controller`, the levels come from
    control_levels over the trace: the container sizes of every chunk at every level are
    taken first (a sender has them: the containers are encoded ahead of time), or from
    `sizes` ([levels][chunks] bytes of an earlier prepare of the same cache and levels).
    `trace`: the per-chunk link rates (default: the uniform trace of `seed`)."""
    tables = [cg.build_cdf(kv, group, chunk, bins, H_kv=H_kv) for bins in level_bins]
    n = tables[0].n_chunks
    bw = bandwidth_trace(n, seed) if trace is None else np.asarray(trace, dtype=np.float64)
    if controller is not None:
        if sizes is not None:
            all_sizes = np.asarray(sizes, dtype=np.int64)
            if all_sizes.shape != (len(tables), n):
                raise ValueError("sizes: one row per level, one column per chunk expected")
        else:
            all_sizes = np.array([[cg.encode(t, kv, k, k + 1).nbytes for k in range(n)]
                                  for t in tables], dtype=np.int64)
        tokens = [min(chunk, kv.shape[2] - k * chunk) for k in range(n)]
        force_levels = list(control_levels(all_sizes, bw, tokens, controller)[0])
    sizes = np.zeros((len(tables), n), dtype=np.int64)
    levels = np.zeros(n, dtype=np.int64)
    items = []
    slot = 0
    for k in range(n):
        blobs = [cg.encode(t, kv, k, k + 1) for t in tables]
        sizes[:, k] = [b.nbytes for b in blobs]
        if force_levels is not None:
            lv = int(force_levels[k])
        else:
            lv = int(choose_levels(sizes[:, k:k + 1], bw[k:k + 1])[0])
        levels[k] = lv
        if lv == TEXT:   # recomputed from text: nothing to stream or decode
            del blobs
            continue
        host = torch.empty(blobs[lv].nbytes, dtype=torch.uint8, pin_memory=True)
        blobs[lv].read_into(host)
        items.append((tables[lv], blobs[lv], host))
        slot = max(slot, blobs[lv].nbytes)
        del blobs
    slot = (slot + 255) // 256 * 256  # slots start on 256-byte boundaries
    return Prepared(tables, items, levels, sizes, bw, slot)


class Pipeline:
    """Staging slots and the copy / decode streams, made once and reused: a stream's
    first use and a fresh allocation would otherwise fall inside the timed run."""

    def __init__(self, prep: Prepared, device, n_slots: int = 32, slot_bytes: int = 0):
        """slot_bytes: at least prep's (a larger slot lets later preparations of the same
        cache at other levels reuse the pipeline)."""
        self.n_slots = n_slots
        slot = max(prep.slot_bytes, (int(slot_bytes) + 255) // 256 * 256)
        self.staging = torch.empty(n_slots * slot, dtype=torch.uint8, device=device)
        self.copy_stream = torch.cuda.Stream(device=device)
        self.decode_stream = torch.cuda.Stream(device=device)


def run(prep: Prepared, out: torch.Tensor, n_slots: int = 32,
        pipe: Optional[Pipeline] = None) -> dict:
    """Streams every chunk into `out` and returns the event timings."""
    if pipe is None or pipe.staging.numel() < n_slots * prep.slot_bytes:
        pipe = Pipeline(prep, out.device, n_slots)
    # the output and staging memory come from torch's current stream
    cur = torch.cuda.current_stream(out.device)
    pipe.copy_stream.wait_stream(cur)
    pipe.decode_stream.wait_stream(cur)
    stats = cg.stream_decode(prep.items, pipe.staging[:n_slots * prep.slot_bytes], n_slots, out,
                             pipe.copy_stream, pipe.decode_stream, wait=True)
    return stats
