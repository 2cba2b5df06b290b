"""CPU oracle of the DSA lightning-indexer hot path (numpy front end of the C oracle).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. The product package
never imports it; the two share no code.

Every function takes and returns numpy arrays holding raw bits: BF16 as
``uint16``, quantized bytes as ``uint8``. The arithmetic lives in
``dsaidx_oracle.c`` (plain C, built with gcc and no floating-point contraction).

Parity is pinned for every function here by the tests under ``tests/`` marked
``not gpu``. The LayerNorm follows the summation order the page shows (running
totals of 8 consecutive columns per lane, pinned by a hand-worked key whose
other orders give other bytes); three points of it stay unpinned because the
page hides them: the lane combine (read as a butterfly over offsets 8, 4, 2, 1),
whether the squares and the affine step are contracted to fused multiply-adds
(read as not), and the rounding of the page's rsqrt (read as IEEE square root
then IEEE divide).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsaidx_oracle.c")
_LIB = os.path.join(_HERE, "libdsaidx_oracle.so")

MXFP4, FP8, FP8_MX = 0, 1, 2
FORMATS = {"mxfp4": MXFP4, "fp8": FP8, "fp8_mx": FP8_MX}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
             "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        sig = {
            "orc_e2m1_value": (ctypes.c_double, [I32]),
            "orc_e2m1_encode": (I32, [F32]),
            "orc_e4m3_value": (ctypes.c_double, [I32]),
            "orc_e4m3_encode": (I32, [F32]),
            "orc_bf16_round": (F32, [F32]),
            "orc_ue8m0_exponent": (I32, [F32]),
            "orc_ue8m0_byte": (I32, [F32]),
            "orc_pow2_ceil": (F32, [F32]),
            "orc_head_weight_scale": (F32, [I32]),
            "orc_ln_sum128": (F32, [P]),
            "orc_layernorm128": (None, [P, P, P, F32, P]),
            "orc_quantize_queries": (I32, [I32, P, I64, I32, I64, I64, P, I64, P, I64, P, I64]),
            "orc_store_keys": (I32, [I32, P, I64, I64, P, P, F32, P, P, I64, I64]),
            "orc_decode_layout": (I32, [P, P, I64, I64, I32, I32, I32, P, P]),
            "orc_score_paged": (I32, [I32, P, I64, I32, P, I64, P, I64, I64, P, I64, I64, P, P,
                                      I64, P, I64, P, I64]),
            "orc_topk": (I32, [P, I64, I64, I64, P, I32, P, I64]),
            "orc_num_threads": (I32, []),
            "orc_decode_tile_size": (I64, [I64, I64, I32, I32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _check(status: int, what: str):
    if status != 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {status})")


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


# ---- scalar formats ---------------------------------------------------------

def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e2m1_encode(x: float) -> int:
    return _load().orc_e2m1_encode(float(x))


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e4m3_encode(x: float) -> int:
    return _load().orc_e4m3_encode(float(x))


def bf16_round(x: float) -> float:
    return _load().orc_bf16_round(float(x))


def ue8m0_exponent(amax: float) -> int:
    return _load().orc_ue8m0_exponent(float(amax))


def ue8m0_byte(amax: float) -> int:
    return _load().orc_ue8m0_byte(float(amax))


def pow2_ceil(x: float) -> float:
    return _load().orc_pow2_ceil(float(x))


def head_weight_scale(heads: int) -> float:
    return _load().orc_head_weight_scale(int(heads))


def ln_sum128(z: np.ndarray) -> float:
    """The LayerNorm's sum of 128 FP32 values in the order page "...cutedsl.dsa.index",
    insert_key, shows (per-lane running totals of 8 columns, then the half-warp combine)."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    return _load().orc_ln_sum128(_ptr(z))


def layernorm128(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    b = np.ascontiguousarray(beta, dtype=np.float32)
    out = np.empty(128, dtype=np.float32)
    _load().orc_layernorm128(_ptr(x), _ptr(g), _ptr(b), float(eps), _ptr(out))
    return out


# ---- hot-path stages --------------------------------------------------------

def row_bytes(fmt, heads: int) -> int:
    """Bytes of one quantized query row: heads x 68 (MXFP4) or heads x 128 (FP8)."""
    return heads * 68 if _fmt(fmt) == MXFP4 else heads * 128


def quantize_queries(q_bits: np.ndarray, wv_bits: np.ndarray | None, fmt="mxfp4"):
    """q_bits: uint16 BF16 [rows, heads, 128]; wv_bits: uint16 BF16 [rows, heads].

    Returns (q_out uint8 [rows, row_bytes], w_out uint16 BF16 [rows, heads] or None)."""
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    rows, heads, dim = q.shape
    assert dim == 128
    out = np.zeros((rows, row_bytes(fmt, heads)), dtype=np.uint8)
    wv = None if wv_bits is None else np.ascontiguousarray(wv_bits, dtype=np.uint16)
    w_out = None if wv is None else np.zeros((rows, heads), dtype=np.uint16)
    st = _load().orc_quantize_queries(
        _fmt(fmt), _ptr(q), rows, heads, heads * 128, 128, _ptr(wv), heads, _ptr(out),
        out.shape[1], _ptr(w_out), heads)
    _check(st, "quantize_queries")
    return out, w_out


def store_keys(key_bits: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float,
               slots: np.ndarray, cache: np.ndarray, num_pages: int, page_stride: int,
               section_offset: int = 0, fmt="mxfp4") -> None:
    """Insert LayerNorm'd, quantized keys into ``cache`` (flat uint8, modified in place).

    Section p starts at byte section_offset + p * page_stride of ``cache``."""
    k = np.ascontiguousarray(key_bits, dtype=np.uint16)
    tokens = k.shape[0]
    assert k.shape[1] == 128 and cache.dtype == np.uint8 and cache.flags.c_contiguous
    s = np.ascontiguousarray(slots, dtype=np.int64)
    assert s.shape == (tokens,)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    b = np.ascontiguousarray(beta, dtype=np.float32)
    base = cache.ctypes.data + int(section_offset)
    st = _load().orc_store_keys(_fmt(fmt), _ptr(k), tokens, 128, _ptr(g), _ptr(b), float(eps),
                                _ptr(s), base, int(num_pages), int(page_stride))
    _check(st, "store_keys")


def index_inputs(projected_bits: np.ndarray, key_col: int, weight_col: int, q_bits: np.ndarray,
                 gamma: np.ndarray, beta: np.ndarray, eps: float, slots: np.ndarray,
                 cache: np.ndarray, num_pages: int, page_stride: int, section_offset: int = 0,
                 fmt="mxfp4"):
    """The indexer inputs of one step, per token (page
    "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index", DsaIndex): the token's
    query ``q_bits[t]`` (uint16 BF16 [tokens, heads, 128]) quantized as ``quantize_queries``
    does, with the raw head weights read from the packed projection row ``projected_bits[t]``
    (uint16 BF16 [tokens, >= cols]) at columns [weight_col, weight_col + heads), and the key
    at columns [key_col, key_col + 128) of the same row inserted at ``slots[t]`` as
    ``store_keys`` does. Returns (q_out, w_out); ``cache`` is modified in place."""
    proj = np.ascontiguousarray(projected_bits, dtype=np.uint16)
    heads = q_bits.shape[1]
    q_out, w_out = quantize_queries(q_bits, proj[:, weight_col:weight_col + heads], fmt)
    store_keys(proj[:, key_col:key_col + 128], gamma, beta, eps, slots, cache, num_pages,
               page_stride, section_offset, fmt)
    return q_out, w_out


def decode_layout(seq_lens, query_lens, num_rows: int, dcp_rank: int = 0,
                  dcp_world_size: int = 1, interleave: int = 1):
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ql = np.ascontiguousarray(query_lens, dtype=np.int32)
    if seq.ndim != 1 or ql.ndim != 1 or seq.size < ql.size:
        raise ValueError("oracle decode_layout: bad length arrays")
    starts = np.zeros(ql.size + 1, dtype=np.int32)
    ends = np.zeros(num_rows, dtype=np.int32) if num_rows >= 0 else None
    st = _load().orc_decode_layout(_ptr(seq), _ptr(ql), ql.size, int(num_rows), int(dcp_rank),
                                   int(dcp_world_size), int(interleave), _ptr(starts), _ptr(ends))
    _check(st, "decode_layout")
    return starts, ends


def score_paged(q_rows: np.ndarray, heads: int, w_bits: np.ndarray, cache: np.ndarray,
                num_pages: int, page_stride: int, block_table: np.ndarray,
                query_starts: np.ndarray, row_ends: np.ndarray, fmt="mxfp4",
                section_offset: int = 0, rows_subset=None, logits: np.ndarray | None = None):
    """Exact scoring. Returns FP32 logits [num_rows, max_blocks * 64]; entries
    that are not scored hold NaN (or keep the values of ``logits`` if given)."""
    q = np.ascontiguousarray(q_rows, dtype=np.uint8)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    qs = np.ascontiguousarray(query_starts, dtype=np.int32)
    re = np.ascontiguousarray(row_ends, dtype=np.int32)
    num_rows = re.shape[0]
    num_requests, max_blocks = bt.shape
    width = max_blocks * 64
    if logits is None:
        logits = np.full((num_rows, width), np.nan, dtype=np.float32)
    subset = None if rows_subset is None else np.ascontiguousarray(rows_subset, dtype=np.int64)
    st = _load().orc_score_paged(
        _fmt(fmt), _ptr(q), q.shape[1], int(heads), _ptr(w), w.shape[1],
        cache.ctypes.data + int(section_offset), int(num_pages), int(page_stride), _ptr(bt),
        num_requests, max_blocks, _ptr(qs), _ptr(re), num_rows, _ptr(logits), logits.shape[1],
        _ptr(subset), 0 if subset is None else subset.size)
    _check(st, "score_paged")
    return logits


def topk(logits: np.ndarray, row_ends: np.ndarray, k: int) -> np.ndarray:
    """Per-row top-k key positions (logit descending, ties to the lower index), -1 padded."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    re = np.ascontiguousarray(row_ends, dtype=np.int32)
    rows, width = lg.shape
    out = np.empty((rows, k), dtype=np.int32)
    st = _load().orc_topk(_ptr(lg), rows, width, width, _ptr(re), int(k), _ptr(out), k)
    _check(st, "topk")
    return out


# ---- decode context parallelism: rank-local keys and the top-k merge -------------------------
# Page "vllm.models.kimi_k3.amd.ops.fp4_indexer", decode_layout: keys are dealt to the ranks in
# runs of `interleave`; page "...cutedsl.dsa.overlap", module text: under DCP the indexer path
# ends in a top-k merge and the local slots.

def dcp_owner(position, world: int, interleave: int):
    """(rank, rank-local position) of global key position(s): run j = position // interleave
    goes to rank j % world as that rank's run j // world."""
    g = np.asarray(position, dtype=np.int64)
    run = g // interleave
    return run % world, (run // world) * interleave + g % interleave


def dcp_global_position(local, rank: int, world: int, interleave: int):
    """Global key position of rank-local position(s) on `rank` (inverse of dcp_owner)."""
    l = np.asarray(local, dtype=np.int64)
    return (l // interleave) * (world * interleave) + rank * interleave + l % interleave


def dcp_candidates(logits: np.ndarray, indices: np.ndarray, rank: int, world: int,
                   interleave: int):
    """One rank's merge candidates from its local top-k: (values FP32 [rows, k], global
    positions int64 [rows, k]); an index of -1 gives value -inf and position -1."""
    idx = np.asarray(indices, dtype=np.int64)
    lg = np.asarray(logits, dtype=np.float32)
    rows = np.arange(idx.shape[0])[:, None]
    ok = idx >= 0
    vals = np.where(ok, lg[rows, np.where(ok, idx, 0)], -np.inf).astype(np.float32)
    pos = np.where(ok, dcp_global_position(np.where(ok, idx, 0), rank, world, interleave), -1)
    return vals, pos


def dcp_merge(values: np.ndarray, positions: np.ndarray, k: int):
    """Global top-k of every row from all ranks' candidates (values / global positions
    [world, rows, kc], position -1 = none): the k largest values, ties to the lower global
    position (-0 equals +0), -1 padded. Returns int32 [rows, k] global positions."""
    v = np.asarray(values, dtype=np.float32)
    p = np.asarray(positions, dtype=np.int64)
    world, rows, kc = v.shape
    out = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        vv = v[:, r, :].reshape(-1).astype(np.float64)
        pp = p[:, r, :].reshape(-1)
        keep = pp >= 0
        vv, pp = vv[keep] + 0.0, pp[keep]          # + 0.0 turns -0 into +0
        order = np.lexsort((pp, -vv))               # value descending, then position ascending
        sel = pp[order[:k]]
        out[r, :sel.size] = sel
    return out


def dcp_local_slots(merged: np.ndarray, rank: int, world: int, interleave: int):
    """The rank-local positions of the merged global top-k that `rank` owns, in the merged
    order, -1 padded: int32 [rows, k]."""
    m = np.asarray(merged, dtype=np.int64)
    out = np.full(m.shape, -1, np.int32)
    for r in range(m.shape[0]):
        g = m[r][m[r] >= 0]
        owner, local = dcp_owner(g, world, interleave)
        mine = local[owner == rank]
        out[r, :mine.size] = mine
    return out


def decode_tile_size(max_model_len: int, width: int, topk: int, heads: int) -> int:
    """Rows per verify tile (page "vllm.models.kimi_k3.amd.ops.fp4_indexer", decode_tile_size)."""
    return int(_load().orc_decode_tile_size(int(max_model_len), int(width), int(topk), int(heads)))


def num_threads() -> int:
    return _load().orc_num_threads()
