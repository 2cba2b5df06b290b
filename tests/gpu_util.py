"""Helpers of the GPU parity tests: upload seeded workloads, run the HIP path through the
binding (which calls the C-ABI), run the oracle on the same host arrays, compare."""
import numpy as np
import torch

import oracle
import sparse_attention_indexer_quant_amd as dsa

DEV = "cuda"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(DEV)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def logit_tolerance(ref_row: np.ndarray) -> float:
    """|delta| <= 1e-5 * max |oracle logit| over the row's valid keys."""
    return 1e-5 * float(np.max(np.abs(ref_row))) if ref_row.size else 0.0


def assert_logits_close(got: np.ndarray, ref: np.ndarray, ends, rows, what=""):
    for r in rows:
        n = int(ends[r])
        if n <= 0:
            continue
        tol = logit_tolerance(ref[r, :n])
        err = np.abs(got[r, :n].astype(np.float64) - ref[r, :n].astype(np.float64))
        worst = int(np.argmax(err))
        assert err[worst] <= tol, f"{what} row {r}: |delta| {err[worst]:.3e} at key {worst} > tol {tol:.3e}"


def assert_topk_sets(got: np.ndarray, want: np.ndarray, rows, what=""):
    for r in rows:
        g, w = np.sort(got[r]), np.sort(want[r])
        assert np.array_equal(g, w), f"{what} row {r}: top-k sets differ ({np.setdiff1d(g, w)[:8]} vs {np.setdiff1d(w, g)[:8]})"


class DeviceWorkload:
    """A Workload's arrays on the GPU plus its cache buffer (filled with `filler`)."""

    def __init__(self, wl, filler=0xA5):
        self.wl = wl
        self.cache = torch.full((wl.cache_bytes,), filler, dtype=torch.uint8, device=DEV)
        self.gamma = dev(wl.gamma)
        self.beta = dev(wl.beta)
        self.block_table = dev(wl.block_table)
        self.seq_lens = dev(wl.seq_lens)
        self.query_lens = dev(wl.query_lens)
        self.q = bf16_dev(wl.q_bits)
        self.wv = bf16_dev(wl.wv_bits)

    def fill_cache(self, chunk=1 << 21):
        wl = self.wl
        for s in range(0, wl.total_keys, chunk):
            e = min(wl.total_keys, s + chunk)
            dsa.store_keys(bf16_dev(wl.key_bits[s:e]), self.gamma, self.beta, wl.eps,
                           dev(wl.key_slots[s:e]), self.cache, wl.num_pages, wl.page_stride,
                           wl.fmt, wl.section_offset)

    def quantize(self):
        return dsa.quantize_queries(self.q, self.wv, self.wl.fmt)

    def layout(self):
        return dsa.decode_layout(self.seq_lens, self.query_lens, self.wl.num_rows)

    def score(self, q_rows, w, starts, ends):
        wl = self.wl
        return dsa.score_paged(q_rows, wl.heads, w, self.cache, wl.num_pages, wl.page_stride,
                               self.block_table, starts, ends, wl.max_query_len, wl.fmt,
                               wl.section_offset)


def oracle_cache(wl, filler=0xA5):
    cache = np.full(wl.cache_bytes, filler, dtype=np.uint8)
    oracle.store_keys(wl.key_bits, wl.gamma, wl.beta, wl.eps, wl.key_slots, cache, wl.num_pages,
                      wl.page_stride, wl.section_offset, wl.fmt)
    return cache
