"""Seeded synthetic inputs for the indexer hot path.

One module serves the HIP path, the oracle, the tests and the benchmark alike.
It holds no step of the method itself: only random draws (NumPy PCG64),
their rounding to BF16 as input values, sequence and query lengths, page
permutations, block tables and slots.

The five named workloads follow the workload descriptions that come with the
pages' indexer path (tiny MXFP4, FP8 decode, MXFP4 decode, MXFP4 speculative
verify, long-context MXFP4); ``make_workload`` builds any other shape.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE_TOKENS = 64
MXFP4_SECTION = 64 * 64 + 64 * 4    # 4352 B: [64 x 64 B E2M1 | 64 x 4 B UE8M0]
FP8_SECTION = 64 * 128 + 64 * 4     # 8448 B: [64 x 128 B E4M3 | 64 x 4 B FP32 scale]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to BF16 (nearest, ties to even); return the raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    fmt: str                    # "mxfp4", "fp8" or "fp8_mx" (FP8 keys, UE8M0 scale bytes)
    heads: int
    topk: int
    seed: int
    seq_lens: np.ndarray        # int32 [R]: keys per request, the step's new tokens included
    query_lens: np.ndarray      # int32 [R]: query rows per request
    num_rows: int               # query rows, graph padding included
    q_bits: np.ndarray          # uint16 BF16 [num_rows, heads, 128]; padding rows zero
    wv_bits: np.ndarray         # uint16 BF16 [num_rows, heads]: raw head weights
    key_bits: np.ndarray        # uint16 BF16 [total_keys, 128]: pre-norm keys of every position
    key_offsets: np.ndarray     # int64 [R + 1]: request q's keys are key_bits[off[q]:off[q+1]]
    key_slots: np.ndarray       # int64 [total_keys]: physical slot = page * 64 + offset
    gamma: np.ndarray           # float32 [128], BF16-representable
    beta: np.ndarray            # float32 [128], BF16-representable
    eps: float
    block_table: np.ndarray     # int32 [R, max_blocks]; unused entries -1
    num_pages: int
    page_stride: int            # bytes between page sections
    section_offset: int         # byte offset of page 0's section in the cache buffer
    recipe: dict = field(default_factory=dict)

    @property
    def num_requests(self) -> int:
        return int(self.seq_lens.size)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def width(self) -> int:
        return self.max_blocks * PAGE_TOKENS

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.query_lens.size else 1

    @property
    def section_bytes(self) -> int:
        return MXFP4_SECTION if self.fmt == "mxfp4" else FP8_SECTION

    @property
    def cache_bytes(self) -> int:
        """Bytes of the cache buffer: the last section ends the buffer."""
        return self.section_offset + max(self.num_pages - 1, 0) * self.page_stride + self.section_bytes

    @property
    def total_keys(self) -> int:
        return int(self.key_offsets[-1])

    def step_key_index(self) -> np.ndarray:
        """Positions in key_bits of the step's new tokens: the last query_len keys of each request."""
        idx = [np.arange(self.key_offsets[q + 1] - self.query_lens[q], self.key_offsets[q + 1])
               for q in range(self.num_requests)]
        return np.concatenate(idx).astype(np.int64) if idx else np.zeros(0, np.int64)

    def scored_pairs(self, row_ends: np.ndarray) -> int:
        return int(np.minimum(np.asarray(row_ends, dtype=np.int64), self.width).sum())

    def key_bytes(self) -> int:
        """Unique key-cache bytes one scoring pass must read (68 or 132 B per key)."""
        per = 68 if self.fmt == "mxfp4" else 132
        return int(self.seq_lens.astype(np.int64).sum()) * per


def make_workload(name: str, *, fmt: str, heads: int, seq_lens, query_lens, num_rows: int | None = None,
                  topk: int, seed: int, page_stride: int | None = None, section_offset: int = 0,
                  permute_pages: bool = True, outlier_frac: float = 0.0, outlier_gain: float = 1.0,
                  head_log2_scale: float = 0.0, extra_pages: int = 0, eps: float = 1e-6,
                  max_blocks: int | None = None, key_chunk: int = 1 << 20) -> Workload:
    """Build a seeded workload. Draw order: page permutation, gamma, beta,
    query (then outlier mask, then per-head log2 scales), head weights, keys."""
    rng = np.random.default_rng(seed)
    seq = np.asarray(seq_lens, dtype=np.int32)
    ql = np.asarray(query_lens, dtype=np.int32)
    R = int(seq.size)
    live_rows = int(ql.sum())
    num_rows = live_rows if num_rows is None else int(num_rows)
    assert num_rows >= live_rows
    section = MXFP4_SECTION if fmt == "mxfp4" else FP8_SECTION
    page_stride = section if page_stride is None else int(page_stride)
    assert page_stride >= section and section_offset + section <= page_stride

    blocks = (seq.astype(np.int64) + PAGE_TOKENS - 1) // PAGE_TOKENS
    need_pages = int(blocks.sum())
    num_pages = need_pages + int(extra_pages)
    perm = rng.permutation(num_pages)  # always drawn, so placement options leave later draws alone
    if not permute_pages:
        perm = np.arange(num_pages)
    mb = int(blocks.max()) if R else 1
    mb = max(mb, 1) if max_blocks is None else int(max_blocks)
    block_table = np.full((R, mb), -1, dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(blocks)]).astype(np.int64)
    for q in range(R):
        block_table[q, :blocks[q]] = perm[first[q]:first[q + 1]]

    gamma = bf16_to_f32(bf16_bits(1.0 + 0.1 * rng.standard_normal(128, dtype=np.float32)))
    beta = bf16_to_f32(bf16_bits(0.1 * rng.standard_normal(128, dtype=np.float32)))

    qf = rng.standard_normal((live_rows, heads, 128), dtype=np.float32)
    if outlier_frac > 0:
        mask = rng.random((live_rows, heads, 128)) < outlier_frac
        qf = np.where(mask, qf * np.float32(outlier_gain), qf)
    if head_log2_scale > 0:
        u = rng.uniform(-head_log2_scale, head_log2_scale, size=heads).astype(np.float32)
        qf = qf * np.exp2(u)[None, :, None].astype(np.float32)
    q_bits = np.zeros((num_rows, heads, 128), dtype=np.uint16)
    q_bits[:live_rows] = bf16_bits(qf)
    del qf
    wv_bits = np.zeros((num_rows, heads), dtype=np.uint16)
    wv_bits[:live_rows] = bf16_bits(rng.standard_normal((live_rows, heads), dtype=np.float32))

    key_offsets = np.concatenate([[0], np.cumsum(seq.astype(np.int64))]).astype(np.int64)
    total = int(key_offsets[-1])
    key_bits = np.empty((total, 128), dtype=np.uint16)
    for s in range(0, total, key_chunk):
        e = min(total, s + key_chunk)
        key_bits[s:e] = bf16_bits(rng.standard_normal((e - s, 128), dtype=np.float32))
    key_slots = np.empty(total, dtype=np.int64)
    for q in range(R):
        pos = np.arange(int(seq[q]), dtype=np.int64)
        key_slots[key_offsets[q]:key_offsets[q + 1]] = (
            block_table[q, pos // PAGE_TOKENS].astype(np.int64) * PAGE_TOKENS + pos % PAGE_TOKENS)

    recipe = dict(fmt=fmt, heads=heads, requests=R, rows=num_rows, live_rows=live_rows, seed=seed,
                  page_stride=page_stride, section_offset=section_offset, topk=topk,
                  permute_pages=permute_pages, outlier_frac=outlier_frac, outlier_gain=outlier_gain,
                  head_log2_scale=head_log2_scale, eps=eps)
    return Workload(name=name, fmt=fmt, heads=heads, topk=topk, seed=seed, seq_lens=seq,
                    query_lens=ql, num_rows=num_rows, q_bits=q_bits, wv_bits=wv_bits,
                    key_bits=key_bits, key_offsets=key_offsets, key_slots=key_slots, gamma=gamma,
                    beta=beta, eps=eps, block_table=block_table, num_pages=num_pages,
                    page_stride=page_stride, section_offset=section_offset, recipe=recipe)


CONFIG_NAMES = ("tiny_mxfp4", "fp8_decode", "mxfp4_decode", "mxfp4_verify", "long_mxfp4")


def config(name: str) -> Workload:
    """The five named workloads (seeds 0, 2, 3, 4, 5)."""
    if name == "tiny_mxfp4":
        # 1 request, 1 decode row, 256 keys (4 pages), 32 heads, top-64.
        return make_workload(name, fmt="mxfp4", heads=32, seq_lens=[256], query_lens=[1],
                             topk=64, seed=0)
    if name == "fp8_decode":
        # 16 decode rows, keys U{1024..8192}, queries with 1% outliers x20, FP8 cache, top-2048.
        rng = np.random.default_rng(2)
        seq = rng.integers(1024, 8193, size=16)
        return make_workload(name, fmt="fp8", heads=32, seq_lens=seq, query_lens=[1] * 16,
                             topk=2048, seed=2 + 1000, outlier_frac=0.01, outlier_gain=20.0)
    if name == "mxfp4_decode":
        # 64 decode rows x 32768 keys, page stride 4352, permuted pages, top-2048.
        return make_workload(name, fmt="mxfp4", heads=32, seq_lens=[32768] * 64,
                             query_lens=[1] * 64, topk=2048, seed=3)
    if name == "mxfp4_verify":
        # 128 requests, 1..4 verify rows each, keys U{4096..65536}, rows padded to 512.
        rng = np.random.default_rng(4)
        ql = rng.integers(1, 5, size=128)
        seq = rng.integers(4096, 65537, size=128)
        return make_workload(name, fmt="mxfp4", heads=32, seq_lens=seq, query_lens=ql,
                             num_rows=512, topk=2048, seed=4 + 1000)
    if name == "long_mxfp4":
        # 64 heads, 8 rows x 131072 keys, 8192-B merged pages with the 4352-B index
        # section at their end, queries scaled per head by 2^U(-4, 4), top-2048.
        return make_workload(name, fmt="mxfp4", heads=64, seq_lens=[131072] * 8,
                             query_lens=[1] * 8, topk=2048, seed=5, page_stride=8192,
                             section_offset=8192 - MXFP4_SECTION, head_log2_scale=4.0)
    raise KeyError(name)
