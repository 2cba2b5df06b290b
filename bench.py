"""Benchmark of the DSA lightning-indexer hot path on one MI355X.

One step = one pass of the whole path over one decode batch, inputs resident in HBM: every
row's query quantized with its head weights, the step's new keys normalized, quantized and
inserted, the decode_layout row bounds, scoring that also writes the top-k segment
histograms, and topk_scored. With one row per request the first four are one launch
(index_score_hist), and where every row's keys also lie in one scoring workgroup the whole
step is (index_score_topk); otherwise index_inputs_layout + score_paged_hist. The other forms
are timed too (per_config ..._fused_inputs, ..._separate_inputs, ..._unfused, ..._tiled). Prints ONE JSON line: scored (row, key) pairs per second of
the whole step, plus the scoring kernel's key-cache GB/s and its roofline fraction (HIP events
on the launch stream around the scoring launch of sampled timed steps, created without the
system-scope cache fence a default event's record adds), and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config long_mxfp4] [--configs all|none|a,b]

The key cache is replicated and the replicas rotate across steps, so every step reads its
keys from HBM rather than from the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer scored (row,key) pairs/s + key-cache HBM GB/s (fraction of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
# MI355X dense matrix peaks (TFLOP/s) of the contraction each key format runs on
MFMA_PEAK_TFLOPS = {"mxfp4": 10100.0, "fp8": 2500.0, "fp8_mx": 2500.0}
MAIN_CONFIG = "long_mxfp4"
# rocprofv3 byte counters per scoring kernel, and the sources that kernel is built from (the
# counters count only while those are unchanged)
PROFILE_PMC = os.path.join(ROOT, "profiles", "{kernel}_{workload}_pmc.txt")
SCORE_SOURCES = [os.path.join(ROOT, "sparse_attention_indexer_quant_amd", "csrc", f)
                 for f in ("score.hip", "device_common.h", "key_norm.h", "select.h", "topk_layout.h")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=MAIN_CONFIG)
    ap.add_argument("--configs", default="all",
                    help="other workloads reported under per_config: all, none, or a comma list")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU budget of the oracle baseline sample of the main workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-rotation-mb", type=float, default=768.0)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a plain copy "
                         "kernel of known size, to scale HBM byte counters)")
    return ap.parse_args()


def _hip_runtime():
    """The HIP runtime this process already uses (the one torch loaded), by its mapped path."""
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64.so" in os.path.basename(path):
                return ctypes.CDLL(path)
    return ctypes.CDLL("libamdhip64.so")


class TimingEvent:
    """A HIP event created with hipEventDisableSystemFence (0x20000000). A default event's
    record writes back and invalidates the caches at system scope, which adds that cost to the
    interval it closes; this flag, documented for timing-only events, leaves it out. Recorded
    on the stream the kernels run on."""

    _hip = None
    FLAGS = 0x20000000

    def __init__(self):
        if TimingEvent._hip is None:
            TimingEvent._hip = _hip_runtime()
        self.ev = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev),
                                                       ctypes.c_uint(self.FLAGS))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = TimingEvent._hip.hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        """Milliseconds from this event to `end` (waits for `end`)."""
        hip = TimingEvent._hip
        if hip.hipEventSynchronize(end.ev) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.ev:
            TimingEvent._hip.hipEventDestroy(self.ev)


class Prepared:
    """A C-ABI call with its arguments converted to their C types once: each call then passes
    the ready ctypes values to an unchecked handle of the same entry point (converting 30-odd
    Python integers per call cost the host 1-1.5 us per launch, which the small workloads'
    steps, bound by the host's launch rate, paid in full)."""

    def __init__(self, fn, *args):
        self.fn = fn
        assert len(args) == len(fn.argtypes), fn.__name__
        self.args = tuple(a if a is None or isinstance(a, ctypes._SimpleCData) else t(a)
                          for t, a in zip(fn.argtypes, args))
        self.raw = getattr(ctypes.CDLL(fn_library_path()), fn.__name__)
        self.raw.restype = fn.restype

    def __call__(self):
        st = self.raw(*self.args)
        if st != 0:
            raise RuntimeError(f"{self.fn.__name__} returned status {st}")


def fn_library_path():
    import sparse_attention_indexer_quant_amd as dsa
    return dsa.LIBRARY


def packed_rows(wl):
    """Packed projection rows of a step's tokens, one per query row, [key 128 | weights H]
    BF16 bits, and each row's key slot (-1 for graph padding rows)."""
    sk = wl.step_key_index()
    live = sk.size
    proj = np.zeros((wl.num_rows, 128 + wl.heads), np.uint16)
    proj[:live, :128] = wl.key_bits[sk]
    proj[:, 128:] = wl.wv_bits
    slots = np.full(wl.num_rows, -1, np.int64)
    slots[:live] = wl.key_slots[sk]
    return proj, slots


def hist_segment_keys(wl):
    """Keys per scoring workgroup (the top-k segment score_paged_hist writes histograms for)."""
    import sparse_attention_indexer_quant_amd as dsa
    return dsa.score_segment_keys(wl.num_requests, wl.max_blocks)


def histogram_bytes(logits, ends, seg, width):
    """Bytes the scorer writes for the selection's histograms: per (row, segment of `seg`
    keys) holding keys of the row, 64 coarse 16-bit counts and one 128-B block of fine counts
    for every coarse bin (top 6 bits of the order-preserving key, -0 as +0) its logits reach."""
    total = 0
    for r, e in enumerate(ends):
        e = int(min(max(int(e), 0), width))
        if e == 0:
            continue
        u = np.ascontiguousarray(logits[r, :e]).view(np.uint32)
        u = np.where(u == 0x80000000, np.uint32(0), u)
        key = np.where(u >> 31 == 1, ~u, u | np.uint32(0x80000000))
        coarse = key >> 26
        for s0 in range(0, e, seg):
            total += 128 + 128 * np.unique(coarse[s0:s0 + seg]).size
    return int(total)


class Setup:
    """Device buffers of one workload, the cache replicas, and the prepared step calls."""

    def __init__(self, name, min_rotation_mb):
        import torch
        import sparse_attention_indexer_quant_amd as dsa
        from sparse_attention_indexer_quant_amd.workloads import config

        t0 = time.perf_counter()
        self.wl = wl = config(name)
        lib = dsa.library()
        dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream(dev)
        sp = self.stream.cuda_stream

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        def bf16(bits):
            return up(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)

        fmt = dsa._FORMATS[wl.fmt]
        self.gamma, self.beta = up(wl.gamma), up(wl.beta)
        cache0 = torch.full((wl.cache_bytes,), 0xA5, dtype=torch.uint8, device=dev)
        chunk = 1 << 21
        fill = []  # the whole cache's keys and slots, in chunks
        for s in range(0, wl.total_keys, chunk):
            e = min(wl.total_keys, s + chunk)
            fill.append((bf16(wl.key_bits[s:e]), up(wl.key_slots[s:e])))
            dsa.store_keys(fill[-1][0], self.gamma, self.beta, wl.eps, fill[-1][1], cache0,
                           wl.num_pages, wl.page_stride, wl.fmt, wl.section_offset)
        reps = int(np.ceil(min_rotation_mb * 1e6 / max(wl.key_bytes(), 1))) + 1
        reps = max(2, min(reps, 16))
        self.caches = [cache0] + [cache0.clone() for _ in range(reps - 1)]
        # bulk fill (store_keys of every key of the workload, timed): the same keys into the
        # same slots of replica 1 leave its bytes as they are
        fills = [(TimingEvent(), TimingEvent()) for _ in range(4)]
        for a, b in fills:  # back to back, read after the last
            a.record(self.stream)
            for keys, slots in fill:
                dsa.store_keys(keys, self.gamma, self.beta, wl.eps, slots, self.caches[1],
                               wl.num_pages, wl.page_stride, wl.fmt, wl.section_offset)
            b.record(self.stream)
        torch.cuda.synchronize()
        fill_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in fills[1:]]))
        fill_bytes = wl.total_keys * (256 + 8 + wl.section_bytes // 64)
        self.bulk_fill = {"keys": int(wl.total_keys), "launches": len(fill), "fills_timed": 3,
                          "us": fill_us,
                          "algorithmic_bytes": int(fill_bytes),
                          "GBps": fill_bytes / fill_us / 1e3}
        del fill
        self.q = bf16(wl.q_bits)
        self.wv = bf16(wl.wv_bits)
        sk = wl.step_key_index()
        self.new_keys = bf16(wl.key_bits[sk])
        self.new_slots = up(wl.key_slots[sk])
        # packed projection rows of the step's tokens, one per query row: [key 128 | weights H]
        # (padding rows carry no key: slot -1)
        self.proj_np, self.row_slots_np = packed_rows(wl)
        self.projected = bf16(self.proj_np)
        self.row_slots = up(self.row_slots_np)
        self.seq_lens, self.query_lens = up(wl.seq_lens), up(wl.query_lens)
        self.block_table = up(wl.block_table)
        rb = dsa.query_row_bytes(fmt, wl.heads)
        self.q_rows = torch.empty((wl.num_rows, rb), dtype=torch.uint8, device=dev)
        self.w_out = torch.empty((wl.num_rows, wl.heads), dtype=torch.bfloat16, device=dev)
        self.starts = torch.empty(wl.num_requests + 1, dtype=torch.int32, device=dev)
        self.ends = torch.empty(wl.num_rows, dtype=torch.int32, device=dev)
        self.logits = torch.empty((wl.num_rows, wl.width), dtype=torch.float32, device=dev)
        self.idx = torch.empty((wl.num_rows, wl.topk), dtype=torch.int32, device=dev)
        wsb = dsa.topk_workspace_bytes(wl.num_rows, wl.width, wl.topk)
        self.ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        hwsb = dsa.score_topk_workspace_bytes(wl.num_requests, wl.max_blocks, wl.num_rows)
        self.hws = torch.empty(max(hwsb, 1), dtype=torch.uint8, device=dev)

        self.quant = Prepared(lib.dsaidx_quantize_queries, fmt, self.q.data_ptr(), wl.num_rows,
                              wl.heads, self.q.stride(0), self.q.stride(1), self.wv.data_ptr(),
                              self.wv.stride(0), self.q_rows.data_ptr(), self.q_rows.stride(0),
                              self.w_out.data_ptr(), self.w_out.stride(0), sp)
        self.layout = Prepared(lib.dsaidx_decode_layout, self.seq_lens.data_ptr(),
                               self.query_lens.data_ptr(), wl.num_requests, wl.num_rows, 0, 1, 1,
                               self.starts.data_ptr(), self.ends.data_ptr(), sp)

        self.topk = Prepared(lib.dsaidx_topk, self.logits.data_ptr(), wl.num_rows, wl.width,
                             self.logits.stride(0), self.ends.data_ptr(), wl.topk,
                             self.idx.data_ptr(), self.idx.stride(0), self.ws.data_ptr(), wsb, sp)
        self.topk_scored = Prepared(lib.dsaidx_topk_scored, self.logits.data_ptr(), wl.num_rows,
                                    self.logits.stride(0), self.ends.data_ptr(), wl.topk,
                                    self.idx.data_ptr(), self.idx.stride(0), wl.num_requests,
                                    wl.max_blocks, self.hws.data_ptr(), hwsb, sp)
        # bounded logits: rows in tiles of decode_tile_size rows (max_model_len = the width)
        self.tile_rows = dsa.decode_tile_size(wl.width, wl.width, wl.topk, wl.heads)
        self.tiles = -(-wl.num_rows // self.tile_rows)
        twsb = int(lib.dsaidx_score_topk_tiled_workspace_bytes(wl.num_requests, wl.max_blocks,
                                                               self.tile_rows, wl.max_query_len))
        self.tws = torch.empty(max(twsb, 1), dtype=torch.uint8, device=dev)
        self.logits_tile = torch.empty((self.tile_rows, wl.width), dtype=torch.float32, device=dev)
        self.tiled = []
        self.store, self.score, self.inputs, self.score_hist = [], [], [], []
        self.inputs_layout, self.index_score = [], []
        # the step's inputs made inside the scorer: at most 4 rows per request (MXFP4), 2 (FP8)
        self.inline_ok = wl.max_query_len <= (4 if wl.fmt == "mxfp4" else 2)
        # ... and the step timed as the workload's step where every request has one row. With
        # several rows per request every scoring workgroup of a request would read and quantize
        # the request's BF16 query rows again (on the verify workload about 21 MB more reads per
        # step than its 26 MB of quantized rows); the separate input launch measured faster
        # there (117.3 against 112.7 us per step), and the fused step is reported beside it.
        self.inline_step = self.inline_ok and wl.max_query_len <= 1
        # ... in one launch with the selection (index_score_topk) where each row's keys lie in
        # one scoring workgroup
        self.one_launch = self.inline_step and hist_segment_keys(wl) >= wl.width
        self.index_topk = []
        for c in self.caches:
            base = c.data_ptr() + wl.section_offset
            self.inputs.append(Prepared(
                lib.dsaidx_index_inputs, fmt, self.projected.data_ptr(), wl.num_rows,
                self.projected.stride(0), 0, 128, self.q.data_ptr(), wl.heads, self.q.stride(0),
                self.q.stride(1), self.gamma.data_ptr(), self.beta.data_ptr(), ctypes.c_float(wl.eps),
                self.row_slots.data_ptr(), base, wl.num_pages, wl.page_stride,
                self.q_rows.data_ptr(), self.q_rows.stride(0), self.w_out.data_ptr(),
                self.w_out.stride(0), sp))
            self.inputs_layout.append(Prepared(
                lib.dsaidx_index_inputs_layout, fmt, self.projected.data_ptr(), wl.num_rows,
                self.projected.stride(0), 0, 128, self.q.data_ptr(), wl.heads, self.q.stride(0),
                self.q.stride(1), self.gamma.data_ptr(), self.beta.data_ptr(), ctypes.c_float(wl.eps),
                self.row_slots.data_ptr(), base, wl.num_pages, wl.page_stride,
                self.q_rows.data_ptr(), self.q_rows.stride(0), self.w_out.data_ptr(),
                self.w_out.stride(0), self.seq_lens.data_ptr(), self.query_lens.data_ptr(),
                wl.num_requests, wl.num_rows, 0, 1, 1, self.starts.data_ptr(),
                self.ends.data_ptr(), sp))
            self.store.append(Prepared(
                lib.dsaidx_store_keys, fmt, self.new_keys.data_ptr(), self.new_keys.shape[0],
                self.new_keys.stride(0), self.gamma.data_ptr(), self.beta.data_ptr(),
                ctypes.c_float(wl.eps), self.new_slots.data_ptr(), base, wl.num_pages,
                wl.page_stride, sp))
            self.score.append(Prepared(
                lib.dsaidx_score_paged, fmt, self.q_rows.data_ptr(), self.q_rows.stride(0),
                wl.heads, self.w_out.data_ptr(), self.w_out.stride(0), base, wl.num_pages,
                wl.page_stride, self.block_table.data_ptr(), wl.num_requests, wl.max_blocks,
                self.starts.data_ptr(), self.ends.data_ptr(), wl.num_rows, wl.max_query_len,
                self.logits.data_ptr(), self.logits.stride(0), sp))
            if self.inline_ok:
                self.index_score.append(Prepared(
                    lib.dsaidx_index_score_hist, fmt, self.projected.data_ptr(),
                    self.projected.stride(0), 0, 128, self.q.data_ptr(), wl.heads,
                    self.q.stride(0), self.q.stride(1), self.gamma.data_ptr(),
                    self.beta.data_ptr(), ctypes.c_float(wl.eps), self.seq_lens.data_ptr(),
                    self.query_lens.data_ptr(), wl.num_requests, wl.num_rows, wl.max_query_len,
                    base, wl.num_pages, wl.page_stride, self.block_table.data_ptr(),
                    wl.max_blocks, self.starts.data_ptr(), self.ends.data_ptr(),
                    self.logits.data_ptr(), self.logits.stride(0), self.hws.data_ptr(), hwsb, sp))
            if self.one_launch:
                self.index_topk.append(Prepared(
                    lib.dsaidx_index_score_topk, fmt, self.projected.data_ptr(),
                    self.projected.stride(0), 0, 128, self.q.data_ptr(), wl.heads,
                    self.q.stride(0), self.q.stride(1), self.gamma.data_ptr(),
                    self.beta.data_ptr(), ctypes.c_float(wl.eps), self.seq_lens.data_ptr(),
                    self.query_lens.data_ptr(), wl.num_requests, wl.num_rows, wl.max_query_len,
                    base, wl.num_pages, wl.page_stride, self.block_table.data_ptr(),
                    wl.max_blocks, self.starts.data_ptr(), self.ends.data_ptr(),
                    self.logits.data_ptr(), self.logits.stride(0), wl.topk, self.idx.data_ptr(),
                    self.idx.stride(0), self.hws.data_ptr(), hwsb, sp))
            self.tiled.append(Prepared(
                lib.dsaidx_score_topk_tiled, fmt, self.q_rows.data_ptr(), self.q_rows.stride(0),
                wl.heads, self.w_out.data_ptr(), self.w_out.stride(0), base, wl.num_pages,
                wl.page_stride, self.block_table.data_ptr(), wl.num_requests, wl.max_blocks,
                self.starts.data_ptr(), self.ends.data_ptr(), wl.num_rows, wl.max_query_len,
                wl.topk, self.idx.data_ptr(), self.idx.stride(0), self.tile_rows,
                self.logits_tile.data_ptr(), self.logits_tile.stride(0), self.tws.data_ptr(),
                twsb, sp))
            self.score_hist.append(Prepared(
                lib.dsaidx_score_paged_hist, fmt, self.q_rows.data_ptr(), self.q_rows.stride(0),
                wl.heads, self.w_out.data_ptr(), self.w_out.stride(0), base, wl.num_pages,
                wl.page_stride, self.block_table.data_ptr(), wl.num_requests, wl.max_blocks,
                self.starts.data_ptr(), self.ends.data_ptr(), wl.num_rows, wl.max_query_len,
                self.logits.data_ptr(), self.logits.stride(0), self.hws.data_ptr(), hwsb, sp))
        self.layout()
        torch.cuda.synchronize()
        self.setup_s = time.perf_counter() - t0
        # row bounds for the byte and pair accounting: this workload's decode_layout output
        ends = self.ends.cpu().numpy()
        self.pairs = wl.scored_pairs(ends)
        # algorithmic bytes of one score launch: unique key bytes + logits written + query rows
        # + head weights
        per_row_q = rb + 2 * wl.heads
        self.score_bytes = wl.key_bytes() + 4 * self.pairs + wl.num_rows * per_row_q
        self.score_flops = 2 * wl.heads * 128 * self.pairs
        # score_paged_hist also writes, per (row, scoring workgroup) holding keys of the row, the
        # 64 coarse counts (128 B) and the 128-B fine block of each coarse bin its logits reach
        # (counted from the logits of one step)
        seg = hist_segment_keys(wl)
        if self.inline_ok:
            self.step_inline(0)
        else:
            self.step(0)
        torch.cuda.synchronize()
        self.hist_bytes = histogram_bytes(self.logits.cpu().numpy(), ends, seg, wl.width)
        self.score_hist_bytes = self.score_bytes + self.hist_bytes
        # index_score_hist reads the BF16 query rows, raw head weights and pre-norm keys instead
        # of the quantized rows and weights, and also writes the step's keys and row layout
        live = int(wl.query_lens.sum())
        self.inline_bytes = (self.score_hist_bytes - wl.num_rows * per_row_q
                             + wl.num_rows * (wl.heads * 256 + 2 * wl.heads + 256)
                             + live * (wl.section_bytes // 64)
                             + 4 * wl.num_rows + 4 * (wl.num_requests + 1) + 8 * wl.num_requests)
        # index_score_topk writes the row's positions instead of the histograms (it reads its
        # own logits back within the launch: on-chip traffic, not counted)
        self.one_launch_bytes = self.inline_bytes - self.hist_bytes + 4 * wl.topk * wl.num_rows

    def prologue(self, i):
        """index_inputs and decode_layout in one launch (index_inputs_layout). (Running
        decode_layout on a second stream beside index_inputs measured 20-40 us slower per step:
        the cross-stream waits cost more than the kernel they would hide.)"""
        self.inputs_layout[i % len(self.caches)]()

    def step(self, i, ev=None):
        """index_inputs, decode_layout, score_paged_hist (timed), topk_scored."""
        self.prologue(i)
        if ev is not None:
            ev[0].record(self.stream)
        self.score_hist[i % len(self.caches)]()
        if ev is not None:
            ev[1].record(self.stream)
        self.topk_scored()

    def step_inline(self, i, ev=None):
        """index_score_hist (the step's inputs and layout made inside the scorer; timed),
        topk_scored."""
        if ev is not None:
            ev[0].record(self.stream)
        self.index_score[i % len(self.caches)]()
        if ev is not None:
            ev[1].record(self.stream)
        self.topk_scored()

    def step_one_launch(self, i, ev=None):
        """index_score_topk: the step's inputs, layout, logits and every row's top-k in one
        scoring launch (timed)."""
        if ev is not None:
            ev[0].record(self.stream)
        self.index_topk[i % len(self.caches)]()
        if ev is not None:
            ev[1].record(self.stream)

    def step_tiled(self, i, ev=None):
        """index_inputs, decode_layout, then score_topk_tiled (scoring + selection per tile of
        decode_tile_size rows: logits and selection scratch bounded to one tile; timed)."""
        self.prologue(i)
        if ev is not None:
            ev[0].record(self.stream)
        self.tiled[i % len(self.caches)]()
        if ev is not None:
            ev[1].record(self.stream)

    def step_unfused(self, i, ev=None):
        """index_inputs, decode_layout, score_paged (timed), topk."""
        self.prologue(i)
        if ev is not None:
            ev[0].record(self.stream)
        self.score[i % len(self.caches)]()
        if ev is not None:
            ev[1].record(self.stream)
        self.topk()


# The score launch of every EVENT_EVERY-th timed step is bracketed by a pair of timing events:
# each event record costs the stream about 1.5 us, which would otherwise add 3 us to every step
# of the throughput the same loop measures.
EVENT_EVERY = 4


# At least this many sampled score launches back every roofline figure: when the timed loop
# has fewer sampled steps, the loop carries on (after the wall clock stops) with more steps,
# sampled the same way, until it has them.
MIN_SAMPLES = 25


def time_steps(s: Setup, steps: int, warmup: int, mode: str = "fused"):
    """Wall time of `steps` steps (after `warmup` untimed ones) and the score launch times
    (ms) of the sampled steps inside that timed loop (and of the steps after it that bring the
    samples to MIN_SAMPLES)."""
    import torch
    step = {"inline": s.step_inline, "fused": s.step, "unfused": s.step_unfused,
            "tiled": s.step_tiled, "one_launch": s.step_one_launch}[mode]
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    total = max(steps, EVENT_EVERY * MIN_SAMPLES)
    evs = {i: (TimingEvent(), TimingEvent()) for i in range(0, total, EVENT_EVERY)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps, total):
        step(warmup + i, evs.get(i))
    torch.cuda.synchronize()
    score_ms = np.array([a.elapsed_time(b) for a, b in evs.values()])
    return wall, score_ms


def kernel_times(s: Setup, reps: int = 30, score_reps: int = 100):
    """Per-kernel HIP-event times (ms, median) of each stage launched on its own (repeated
    back to back, not inside the step): `score_reps` launches for the scoring kernels,
    `reps` for the others."""
    import torch
    out = {}
    stages = [("index_inputs_layout", lambda i: s.inputs_layout[i % len(s.caches)]()),
              ("index_inputs", lambda i: s.inputs[i % len(s.caches)]()),
              ("quantize_queries", lambda i: s.quant()),
              ("store_keys", lambda i: s.store[i % len(s.caches)]()),
              ("decode_layout", lambda i: s.layout()),
              ("score_paged", lambda i: s.score[i % len(s.caches)]()),
              ("topk", lambda i: s.topk()),
              ("score_paged_hist", lambda i: s.score_hist[i % len(s.caches)]()),
              ("topk_scored", lambda i: s.topk_scored())]
    if s.inline_ok:
        stages.append(("index_score_hist", lambda i: s.index_score[i % len(s.caches)]()))
    if s.one_launch:
        stages.append(("index_score_topk", lambda i: s.index_topk[i % len(s.caches)]()))
    for name, fn in stages:
        # launched back to back, each between its own pair of events, read after the last
        n = score_reps if name.startswith(("score", "index_score")) else reps
        evs = [(TimingEvent(), TimingEvent()) for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            a.record(s.stream)
            fn(i)
            b.record(s.stream)
        torch.cuda.synchronize()
        out[name] = float(np.median([a.elapsed_time(b) for a, b in evs]))
    return out


def stream_ceiling(key_bytes: int, grids=(256, 512, 1024, 2048, 4096, 8192), reps: int = 20):
    """The device's contiguous read rate at the scorer's key bytes, 300 MB and 1 GB: read_stream
    (16-byte loads, eight in flight per lane) at each grid size, each launch reading a
    different region of a buffer of at least 768 MB (so reads come from HBM, not the 256 MB
    Infinity Cache), launched back to back between HIP events read after the last launch.
    Returns the best grid's mean GB/s per size."""
    import torch
    import sparse_attention_indexer_quant_amd as dsa
    lib = dsa.library()
    sizes = [int(key_bytes) // 16 * 16, 300_000_000, 1_000_000_000]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    res = []
    for size in sizes:
        regions = max(2, -(-768_000_000 // size) + 1)
        buf = torch.ones(size * regions, dtype=torch.uint8, device="cuda")
        out = torch.zeros(4 * max(grids), dtype=torch.int32, device="cuda")
        best = None
        per_grid = {}
        for g in grids:
            calls = [Prepared(lib.dsaidx_read_stream, buf.data_ptr() + r * size, size, g,
                              out.data_ptr(), out.numel(), sp) for r in range(regions)]
            for i in range(3):
                calls[i % regions]()
            evs = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
            for i, (a, b) in enumerate(evs):
                a.record(stream)
                calls[i % regions]()
                b.record(stream)
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs]))
            per_grid[g] = size / us / 1e3
            if best is None or per_grid[g] > best[1]:
                best = (g, per_grid[g], us)
        res.append({"bytes": size, "best_workgroups": best[0], "GBps": best[1], "us_mean": best[2],
                    "GBps_by_workgroups": per_grid})
        del buf, out
        torch.cuda.empty_cache()
    return res


def read_reference(s: Setup, reps: int = 24, warmup: int = 4):
    """HIP-event times of read_sections (a plain read of the same key sections in the scorer's
    grid, no arithmetic) over the rotating replicas: with the workload's page table and
    stride, and with the same pages laid out contiguously (page stride = section)."""
    import torch
    import sparse_attention_indexer_quant_amd as dsa
    wl = s.wl
    lib = dsa.library()
    fmt = dsa._FORMATS[wl.fmt]
    dev = s.block_table.device
    words = int(lib.dsaidx_read_sections_words(wl.num_requests, wl.max_blocks))
    out = torch.empty(max(words, 1), dtype=torch.int32, device=dev)
    # the same pages, consecutive: request q's blocks get the next ceil(seq_q / 64) page ids
    nblk = np.minimum((np.maximum(wl.seq_lens.astype(np.int64), 0) + 63) // 64, wl.max_blocks)
    bt_c = np.full((wl.num_requests, wl.max_blocks), -1, np.int32)
    nxt = 0
    for q in range(wl.num_requests):
        bt_c[q, :nblk[q]] = np.arange(nxt, nxt + nblk[q], dtype=np.int32)
        nxt += int(nblk[q])
    bt_contig = torch.from_numpy(bt_c).to(dev)
    sp = s.stream.cuda_stream
    key_bytes = int(nblk.sum()) * wl.section_bytes

    def timed(paged):
        calls = []
        for c in s.caches:
            if paged:
                args = (fmt, c.data_ptr() + wl.section_offset, wl.num_pages, wl.page_stride,
                        s.block_table.data_ptr())
            else:
                args = (fmt, c.data_ptr(), nxt, wl.section_bytes, bt_contig.data_ptr())
            calls.append(Prepared(lib.dsaidx_read_sections, *args, wl.num_requests,
                                  wl.max_blocks, s.seq_lens.data_ptr(), out.data_ptr(),
                                  out.numel(), sp))
        # back to back with the events between them, read after the last launch (as the
        # scorer's launches are timed inside the step loop): waiting on each pair would leave
        # the GPU idle between launches
        evs = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
        for i in range(warmup):
            calls[i % len(calls)]()
        for i, (a, b) in enumerate(evs):
            a.record(s.stream)
            calls[i % len(calls)]()
            b.record(s.stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs]))

    paged_us, contig_us = timed(True), timed(False)
    return {"kernel": "read_sections", "key_bytes": key_bytes,
            "paged_us_mean": paged_us, "paged_GBps": key_bytes / paged_us / 1e3,
            "contiguous_us_mean": contig_us, "contiguous_GBps": key_bytes / contig_us / 1e3}


def cpu_baseline(s: Setup, budget_s: float):
    """The oracle, untuned, on the host cores: score + top-k of a bounded sample of rows
    (plus the step's query quantization and key inserts), scaled to pairs/s."""
    import oracle
    wl = s.wl
    ocache = np.full(wl.cache_bytes, 0xA5, np.uint8)
    oracle.store_keys(wl.key_bits, wl.gamma, wl.beta, wl.eps, wl.key_slots, ocache, wl.num_pages,
                      wl.page_stride, wl.section_offset, wl.fmt)
    starts, ends = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
    live = [r for r in range(wl.num_rows) if ends[r] > 0]
    # probe one row to size the sample to the budget
    scratch = ocache.copy()
    t0 = time.perf_counter()
    oq, ow = oracle.index_inputs(s.proj_np, 0, 128, wl.q_bits, wl.gamma, wl.beta, wl.eps,
                                 s.row_slots_np, scratch, wl.num_pages, wl.page_stride,
                                 wl.section_offset, wl.fmt)
    fixed = time.perf_counter() - t0
    del scratch
    t0 = time.perf_counter()
    lg = oracle.score_paged(oq, wl.heads, ow, ocache, wl.num_pages, wl.page_stride, wl.block_table,
                            starts, ends, wl.fmt, wl.section_offset, rows_subset=[live[0]])
    oracle.topk(np.nan_to_num(lg[[live[0]]], nan=0.0), ends[[live[0]]], wl.topk)
    per_row = max(time.perf_counter() - t0, 1e-6)
    n = int(max(1, min(len(live), budget_s / per_row)))
    rows = live[:: max(1, len(live) // n)][:n]
    t0 = time.perf_counter()
    lg = oracle.score_paged(oq, wl.heads, ow, ocache, wl.num_pages, wl.page_stride, wl.block_table,
                            starts, ends, wl.fmt, wl.section_offset, rows_subset=rows)
    oracle.topk(np.nan_to_num(lg[rows], nan=0.0), ends[rows], wl.topk)
    el = time.perf_counter() - t0
    pairs = int(np.minimum(ends[rows], wl.width).sum())
    # the whole step on the CPU would take fixed + el * (all pairs / sampled pairs)
    step_s = fixed + el * (s.pairs / max(pairs, 1))
    affinity = len(os.sched_getaffinity(0))
    return {"value": s.pairs / step_s, "unit": "pairs/s",
            # OpenMP threads the oracle ran, each on its own core of the affinity mask
            "cores": min(oracle.num_threads(), affinity), "omp_threads": oracle.num_threads(),
            "affinity_cores": affinity,
            "kind": "oracle",
            "sample": f"{wl.name}: score_paged + topk of {len(rows)} of {len(live)} live rows "
                      f"({pairs} pairs, {el:.2f} s), plus index_inputs of all {wl.num_rows} rows "
                      f"and the step's {int((s.row_slots_np >= 0).sum())} keys ({fixed:.2f} s), "
                      f"scaled to the whole step",
            "score_topk_pairs_per_s": pairs / el,
            "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def scorer_source_hash():
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 counter
    summary, if it was taken on the current scorer sources; else None."""
    try:
        text = open(PROFILE_PMC.format(kernel=kernel, workload=workload)).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("scorer_sources_sha256_16") != scorer_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_config(name, args, steps, warmup, cpu_budget):
    import torch
    s = Setup(name, args.min_rotation_mb)
    wall_u, score_ms_u = time_steps(s, steps, warmup, mode="unfused")
    wall_f, score_ms_f = time_steps(s, steps, warmup, mode="fused")
    wall_t, tiled_ms = time_steps(s, steps, warmup, mode="tiled")
    # the step for this workload: the inputs made inside the scorer where every request has one
    # row (with the selection in the same launch where every row's keys lie in one scoring
    # workgroup), else the separate input launch (the fused forms are timed as well where they
    # apply)
    wall_i = score_ms_i = wall_o = score_ms_o = None
    if s.inline_ok:
        wall_i, score_ms_i = time_steps(s, steps, warmup, mode="inline")
    if s.one_launch:
        wall_o, score_ms_o = time_steps(s, steps, warmup, mode="one_launch")
    if s.one_launch:
        wall, score_ms = wall_o, score_ms_o
        kernel, kbytes = "index_score_topk", s.one_launch_bytes
    elif s.inline_step:
        wall, score_ms = wall_i, score_ms_i
        kernel, kbytes = "index_score_hist", s.inline_bytes
    else:
        wall, score_ms = wall_f, score_ms_f
        kernel, kbytes = "score_paged_hist", s.score_hist_bytes
    ms_step = wall / steps * 1e3
    score_us = float(score_ms.mean() * 1e3)
    score_us_f = float(score_ms_f.mean() * 1e3)
    score_us_u = float(score_ms_u.mean() * 1e3)
    res = {
        "workload": name,
        "fmt": s.wl.fmt, "heads": s.wl.heads, "rows": s.wl.num_rows, "requests": s.wl.num_requests,
        "topk": s.wl.topk, "page_stride": s.wl.page_stride, "seed": s.wl.seed,
        "scored_pairs": s.pairs,
        "ms_per_step": ms_step,
        "step_pairs_per_s": s.pairs / (ms_step / 1e3),
        "score_us_mean": score_us,
        "score_launches_timed": int(score_ms.size),
        "score_us_p10_p50_p90": [float(np.percentile(score_ms, p) * 1e3) for p in (10, 50, 90)],
        "score_pairs_per_s": s.pairs / (score_us / 1e6),
        "score_key_GBps": s.wl.key_bytes() / (score_us / 1e6) / 1e9,
        "score_key_bytes": s.wl.key_bytes(),
        "score_algorithmic_GBps": kbytes / (score_us / 1e6) / 1e9,
        "score_algorithmic_bytes": kbytes,
        "score_histogram_bytes": s.hist_bytes,
        "score_kernel": kernel,
        "step": "index_score_topk (one launch)" if s.one_launch else
                "index_score_hist + topk_scored" if s.inline_step else
                "index_inputs_layout + score_paged_hist + topk_scored",
        "ms_per_step_one_launch": wall_o / steps * 1e3 if wall_o is not None else None,
        "ms_per_step_fused_inputs": wall_i / steps * 1e3 if wall_i is not None else None,
        "index_score_hist_us_mean": float(score_ms_i.mean() * 1e3) if score_ms_i is not None else None,
        "ms_per_step_separate_inputs": wall_f / steps * 1e3,
        "score_paged_hist_us_mean": score_us_f,
        "score_paged_hist_algorithmic_GBps": s.score_hist_bytes / (score_us_f / 1e6) / 1e9,
        # bounded logits: the same step with scoring + selection in row tiles
        "tile_rows": s.tile_rows, "tiles": s.tiles,
        "ms_per_step_tiled": wall_t / steps * 1e3,
        "score_topk_tiled_us_mean": float(tiled_ms.mean() * 1e3),
        "logits_bytes_tiled": s.tile_rows * s.wl.width * 4,
        "logits_bytes_untiled": s.wl.num_rows * s.wl.width * 4,
        "ms_per_step_unfused": wall_u / steps * 1e3,
        "step_pairs_per_s_unfused": s.pairs / (wall_u / steps),
        "score_paged_us_mean_unfused": score_us_u,
        "score_paged_algorithmic_GBps_unfused": s.score_bytes / (score_us_u / 1e6) / 1e9,
        "score_TFLOPs": s.score_flops / (score_us / 1e6) / 1e12,
        # the contraction's matrix-core peak: scaled FP4 MFMA for MXFP4; FP8 keys and queries
        # are widened exactly to BF16 and contracted on the BF16 MFMA
        "mfma_peak_TFLOPs": MFMA_PEAK_TFLOPS[s.wl.fmt],
        "score_mfma_frac_of_peak": s.score_flops / (score_us / 1e6) / 1e12 / MFMA_PEAK_TFLOPS[s.wl.fmt],
        "store_keys_bulk_fill": s.bulk_fill,
        "cache_replicas": len(s.caches),
        "kernel_us_alone": {k: v * 1e3 for k, v in kernel_times(s).items()},
    }
    ref = read_reference(s)
    # the scoring launch's time over a plain read of its key sections in the same grid
    ref["score_time_over_paged_read"] = score_us / ref["paged_us_mean"]
    res["read_reference"] = ref
    res["score_key_frac_of_peak"] = res["score_key_GBps"] / HBM_PEAK_GBPS
    if cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(s, cpu_budget)
    del s
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from sparse_attention_indexer_quant_amd.workloads import CONFIG_NAMES

    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        del src, dst
    main_res = run_config(args.config, args, args.steps, args.warmup,
                          0.0 if args.no_cpu_baseline else args.cpu_seconds)
    print(f"[bench] {args.config}: {main_res['ms_per_step']:.4f} ms/step, score "
          f"{main_res['score_us_mean']:.2f} us", file=sys.stderr, flush=True)
    others = []
    if args.configs == "all":
        others = [c for c in CONFIG_NAMES if c != args.config]
    elif args.configs not in ("none", ""):
        others = [c for c in args.configs.split(",") if c != args.config]
    per_config = {args.config: main_res}
    for name in others:
        per_config[name] = run_config(name, args, max(20, args.steps // 2), min(args.warmup, 10),
                                      0.0 if args.no_cpu_baseline else 2.0)
        print(f"[bench] {name}: {per_config[name]['ms_per_step']:.4f} ms/step, score "
              f"{per_config[name]['score_us_mean']:.2f} us", file=sys.stderr, flush=True)

    m = main_res
    ceiling = stream_ceiling(m["score_key_bytes"])
    print(f"[bench] read ceiling: " + ", ".join(f"{c['bytes'] / 1e6:.0f} MB {c['GBps']:.0f} GB/s"
                                                 for c in ceiling), file=sys.stderr, flush=True)
    traffic = measured_traffic(m["score_kernel"], args.config)
    achieved = m["score_algorithmic_GBps"]
    line = {
        "metric": METRIC,
        "value": m["step_pairs_per_s"],
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["fmt"],
        "data": "synthetic",
        "config": {"workload": args.config, "heads": m["heads"], "rows": m["rows"],
                   "requests": m["requests"], "topk": m["topk"], "page_stride": m["page_stride"],
                   "scored_pairs": m["scored_pairs"], "parallelism": "none (1 GPU)"},
        "key_cache_GBps": m["score_key_GBps"],
        "key_cache_frac_of_peak": m["score_key_frac_of_peak"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": m["score_kernel"],
                     "bytes_per_launch": m["score_algorithmic_bytes"],
                     "launch_us_mean": m["score_us_mean"],
                     "launches_timed": m["score_launches_timed"],
                     # the same launch repeated back to back outside the step (no other kernel
                     # between the launches): the kernel's own rate without the step around it
                     "launch_us_alone": m["kernel_us_alone"][m["score_kernel"]],
                     "frac_alone": m["score_algorithmic_bytes"] / m["kernel_us_alone"][m["score_kernel"]]
                                   / 1e3 / HBM_PEAK_GBPS,
                     "read_reference_GBps": m["read_reference"]["paged_GBps"],
                     "read_reference_contiguous_GBps": m["read_reference"]["contiguous_GBps"],
                     # a plain contiguous read of the scorer's key bytes at its best grid: the
                     # device's measured read rate at this size, and the scorer against it
                     "stream_read_ceiling_GBps": ceiling[0]["GBps"],
                     "frac_of_stream_read_ceiling": achieved / ceiling[0]["GBps"]},
        "stream_read_ceiling": ceiling,
        "cpu_baseline": m.get("cpu_baseline"),
        "per_config": per_config,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
