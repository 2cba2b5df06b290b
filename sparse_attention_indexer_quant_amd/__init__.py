"""MI355X-native DSA lightning-indexer hot path: thin Python binding over libdsaidx.so.

Every call marshals torch tensors into the C-ABI declared in ``include/dsaidx.h``
and enqueues the HIP kernels on the current torch stream; no step of the path
runs in Python. The library is loaded on first use and a missing build raises
``RuntimeError`` -- there is no CPU fallback.

Calls (names follow the pages' problem statement: page
"vllm.models.kimi_k3.amd.ops.fp4_indexer" quantize_queries / store_keys /
score_paged / decode_layout, plus the per-row top-k and the fused per-token inputs of
page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index", DsaIndex):

  quantize_queries(q, wv, fmt)            -> (q_rows uint8, w_out bf16)
  index_inputs(projected, key_col, weight_col, q, gamma, beta, eps, slots, cache, ...)
                                          -> (q_rows uint8, w_out bf16); keys inserted
  store_keys(keys, gamma, beta, eps, slots, cache, num_pages, page_stride, fmt)
  decode_layout(seq_lens, query_lens, num_rows, dcp_rank, dcp_world_size, interleave)
  score_paged(q_rows, heads, weights, cache, ..., block_table, query_starts, row_ends, max_query_len)
  topk(logits, row_ends, k)
  score_topk(...)  = score_paged + topk with the scorer writing the selection's histograms
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libdsaidx.so")

MXFP4, FP8, FP8_MX = 0, 1, 2
_FORMATS = {"mxfp4": MXFP4, "fp8": FP8, "fp8_mx": FP8_MX}
SECTION_BYTES = {MXFP4: 4352, FP8: 8448, FP8_MX: 8448}
PAGE_TOKENS = 64

_lib = None


class DsaidxError(RuntimeError):
    """A non-zero status from the C-ABI (argument, layout or HIP launch error)."""

    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"dsaidx_{call}: {message} (status {status})")
        self.status = status


def library():
    """The loaded C-ABI library; raises RuntimeError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is not built: run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
        lib = ctypes.CDLL(LIBRARY)
        P, I64, I32, F32, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                ctypes.c_size_t)
        sig = {
            "dsaidx_status_string": (ctypes.c_char_p, [I32]),
            "dsaidx_query_row_bytes": (I64, [I32, I32]),
            "dsaidx_quantize_queries": (I32, [I32, P, I64, I32, I64, I64, P, I64, P, I64, P, I64, P]),
            "dsaidx_store_keys": (I32, [I32, P, I64, I64, P, P, F32, P, P, I64, I64, P]),
            "dsaidx_index_inputs": (I32, [I32, P, I64, I64, I64, I64, P, I32, I64, I64, P, P, F32,
                                          P, P, I64, I64, P, I64, P, I64, P]),
            "dsaidx_index_inputs_layout": (I32, [I32, P, I64, I64, I64, I64, P, I32, I64, I64, P, P,
                                                 F32, P, P, I64, I64, P, I64, P, I64, P, P, I64,
                                                 I64, I32, I32, I32, P, P, P]),
            "dsaidx_decode_layout": (I32, [P, P, I64, I64, I32, I32, I32, P, P, P]),
            "dsaidx_score_paged": (I32, [I32, P, I64, I32, P, I64, P, I64, I64, P, I64, I64, P, P,
                                         I64, I32, P, I64, P]),
            "dsaidx_topk_workspace_bytes": (SZ, [I64, I64, I32]),
            "dsaidx_score_topk_workspace_bytes": (SZ, [I64, I64, I64]),
            "dsaidx_score_segment_keys": (I64, [I64, I64]),
            "dsaidx_read_sections_words": (I64, [I64, I64]),
            "dsaidx_read_sections": (I32, [I32, P, I64, I64, P, I64, I64, P, P, I64, P]),
            "dsaidx_read_stream": (I32, [P, I64, I32, P, I64, P]),
            "dsaidx_score_paged_hist": (I32, [I32, P, I64, I32, P, I64, P, I64, I64, P, I64, I64,
                                              P, P, I64, I32, P, I64, P, SZ, P]),
            "dsaidx_index_score_hist": (I32, [I32, P, I64, I64, I64, P, I32, I64, I64, P, P, F32,
                                              P, P, I64, I64, I32, P, I64, I64, P, I64, P, P, P,
                                              I64, P, SZ, P]),
            "dsaidx_index_score_topk": (I32, [I32, P, I64, I64, I64, P, I32, I64, I64, P, P, F32,
                                              P, P, I64, I64, I32, P, I64, I64, P, I64, P, P, P,
                                              I64, I32, P, I64, P, SZ, P]),
            "dsaidx_topk_scored": (I32, [P, I64, I64, P, I32, P, I64, I64, I64, P, SZ, P]),
            "dsaidx_topk": (I32, [P, I64, I64, I64, P, I32, P, I64, P, SZ, P]),
            "dsaidx_topk_noalloc": (I32, [P, I64, I64, I64, P, I32, P, I64, P]),
            "dsaidx_decode_tile_size": (I64, [I64, I64, I32, I32]),
            "dsaidx_score_topk_tiled_workspace_bytes": (SZ, [I64, I64, I64, I32]),
            "dsaidx_score_topk_tiled": (I32, [I32, P, I64, I32, P, I64, P, I64, I64, P, I64, I64,
                                              P, P, I64, I32, I32, P, I64, I64, P, I64, P, SZ, P]),
            "dsaidx_dcp_candidates": (I32, [P, I64, I64, I64, P, I32, I64, I32, I32, I32, P, P, P]),
            "dsaidx_dcp_merge": (I32, [P, P, I32, I64, I32, I32, P, I64, I32, I32, P, I64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _fmt(fmt) -> int:
    return _FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _check(call: str, status: int):
    if status != 0:
        msg = library().dsaidx_status_string(status).decode()
        raise DsaidxError(call, status, msg)


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def query_row_bytes(fmt, heads: int) -> int:
    """Bytes of one quantized query row: [H x 64 E2M1 | H x 4 UE8M0] or [H x 128 E4M3]."""
    return int(library().dsaidx_query_row_bytes(_fmt(fmt), int(heads)))


def quantize_queries(q, wv=None, fmt="mxfp4", out=None, w_out=None):
    """q: bf16 [rows, heads, 128] (128-element heads contiguous); wv: bf16 [rows, heads] raw
    head weights or None. Returns (q_rows uint8 [rows, row_bytes], w_out bf16 [rows, heads])."""
    import torch
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != 128 or q.stride(2) != 1:
        raise ValueError("quantize_queries: q must be [rows, heads, 128] with contiguous heads")
    rows, heads = q.shape[0], q.shape[1]
    f = _fmt(fmt)
    rb = query_row_bytes(f, heads) if heads in (16, 32, 64) else heads * 128
    if out is None:
        out = torch.empty((rows, rb), dtype=torch.uint8, device=q.device)
    _dev(out, "out", torch.uint8)
    if wv is not None:
        _dev(wv, "wv", torch.bfloat16)
        if wv.dim() != 2 or wv.stride(1) != 1:
            raise ValueError("quantize_queries: wv must be [rows, heads] with unit head stride")
        if w_out is None:
            w_out = torch.empty((rows, heads), dtype=torch.bfloat16, device=q.device)
        _dev(w_out, "w_out", torch.bfloat16)
    st = library().dsaidx_quantize_queries(
        f, q.data_ptr(), rows, heads, q.stride(0), q.stride(1),
        None if wv is None else wv.data_ptr(), 0 if wv is None else wv.stride(0),
        out.data_ptr(), out.stride(0),
        None if wv is None else w_out.data_ptr(), 0 if wv is None else w_out.stride(0),
        _stream(q))
    _check("quantize_queries", st)
    return out, w_out


def store_keys(keys, gamma, beta, eps, slots, cache, num_pages, page_stride, fmt="mxfp4",
               section_offset=0):
    """LayerNorm + quantize + insert keys [T, 128] bf16 into the paged cache.

    cache: flat uint8 tensor; section p starts at byte section_offset + p * page_stride.
    slots: int64 [T]; negative slots are padding."""
    import torch
    _dev(keys, "keys", torch.bfloat16)
    if keys.dim() != 2 or keys.shape[1] != 128 or keys.stride(1) != 1:
        raise ValueError("store_keys: keys must be [T, 128] with contiguous rows")
    _dev(slots, "slots", torch.int64)
    if slots.dim() != 1 or slots.numel() != keys.shape[0] or slots.stride(0) != 1:
        raise ValueError("store_keys: one contiguous slot per key")
    _dev(gamma, "gamma", torch.float32)
    _dev(beta, "beta", torch.float32)
    _dev(cache, "cache", torch.uint8)
    st = library().dsaidx_store_keys(
        _fmt(fmt), keys.data_ptr(), keys.shape[0], keys.stride(0), gamma.data_ptr(),
        beta.data_ptr(), float(eps), slots.data_ptr(), cache.data_ptr() + int(section_offset),
        int(num_pages), int(page_stride), _stream(keys))
    _check("store_keys", st)


def index_inputs(projected, key_col, weight_col, q, gamma, beta, eps, slots, cache, num_pages,
                 page_stride, fmt="mxfp4", section_offset=0, out=None, w_out=None):
    """The indexer inputs of one step in one launch, one workgroup per token: the query
    q [tokens, heads, 128] (bf16) quantized with the raw head weights read from the packed
    projection rows projected [tokens, >= cols] (bf16) at columns weight_col.., and the key
    at columns key_col..key_col+128 of the same rows inserted at slots (int64 [tokens]).
    Returns (q_rows uint8 [tokens, row_bytes], w_out bf16 [tokens, heads])."""
    import torch
    _dev(projected, "projected", torch.bfloat16)
    if projected.dim() != 2 or projected.stride(1) != 1:
        raise ValueError("index_inputs: projected must be [tokens, cols] with unit column stride")
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != 128 or q.stride(2) != 1 or q.shape[0] != projected.shape[0]:
        raise ValueError("index_inputs: q must be [tokens, heads, 128] with contiguous heads")
    _dev(slots, "slots", torch.int64)
    if slots.dim() != 1 or slots.numel() != q.shape[0] or slots.stride(0) != 1:
        raise ValueError("index_inputs: one contiguous slot per token")
    _dev(gamma, "gamma", torch.float32)
    _dev(beta, "beta", torch.float32)
    _dev(cache, "cache", torch.uint8)
    tokens, heads = q.shape[0], q.shape[1]
    f = _fmt(fmt)
    if out is None:
        out = torch.empty((tokens, query_row_bytes(f, heads) or heads * 128), dtype=torch.uint8,
                          device=q.device)
    if w_out is None:
        w_out = torch.empty((tokens, heads), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", torch.uint8)
    _dev(w_out, "w_out", torch.bfloat16)
    st = library().dsaidx_index_inputs(
        f, projected.data_ptr(), tokens, projected.stride(0), int(key_col), int(weight_col),
        q.data_ptr(), heads, q.stride(0), q.stride(1), gamma.data_ptr(), beta.data_ptr(),
        float(eps), slots.data_ptr(), cache.data_ptr() + int(section_offset), int(num_pages),
        int(page_stride), out.data_ptr(), out.stride(0), w_out.data_ptr(), w_out.stride(0),
        _stream(q))
    _check("index_inputs", st)
    return out, w_out


def index_inputs_layout(projected, key_col, weight_col, q, gamma, beta, eps, slots, cache,
                        num_pages, page_stride, seq_lens, query_lens, num_rows, fmt="mxfp4",
                        section_offset=0, dcp_rank=0, dcp_world_size=1, interleave=1):
    """index_inputs and decode_layout in one launch. Returns (q_rows, w_out, query_starts,
    row_ends)."""
    import torch
    _dev(projected, "projected", torch.bfloat16)
    _dev(q, "q", torch.bfloat16)
    _dev(slots, "slots", torch.int64)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(query_lens, "query_lens", torch.int32)
    if projected.dim() != 2 or projected.stride(1) != 1 or q.dim() != 3 or q.stride(2) != 1 \
            or q.shape[0] != projected.shape[0] or slots.numel() != q.shape[0]:
        raise ValueError("index_inputs_layout: projected [tokens, cols], q [tokens, heads, 128], "
                         "one slot per token")
    tokens, heads = q.shape[0], q.shape[1]
    f = _fmt(fmt)
    out = torch.empty((tokens, query_row_bytes(f, heads)), dtype=torch.uint8, device=q.device)
    w_out = torch.empty((tokens, heads), dtype=torch.bfloat16, device=q.device)
    R = query_lens.numel()
    starts = torch.empty(R + 1, dtype=torch.int32, device=q.device)
    ends = torch.empty(max(int(num_rows), 0), dtype=torch.int32, device=q.device)
    st = library().dsaidx_index_inputs_layout(
        f, projected.data_ptr(), tokens, projected.stride(0), int(key_col), int(weight_col),
        q.data_ptr(), heads, q.stride(0), q.stride(1), gamma.data_ptr(), beta.data_ptr(),
        float(eps), slots.data_ptr(), cache.data_ptr() + int(section_offset), int(num_pages),
        int(page_stride), out.data_ptr(), out.stride(0), w_out.data_ptr(), w_out.stride(0),
        seq_lens.contiguous().data_ptr(), query_lens.contiguous().data_ptr(), R, int(num_rows),
        int(dcp_rank), int(dcp_world_size), int(interleave), starts.data_ptr(), ends.data_ptr(),
        _stream(q))
    _check("index_inputs_layout", st)
    return out, w_out, starts, ends


def decode_layout(seq_lens, query_lens, num_rows, dcp_rank=0, dcp_world_size=1, interleave=1,
                  starts=None, row_ends=None):
    """Device-side row grouping: returns (query_starts int32 [R+1], row_ends int32 [num_rows])."""
    import torch
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(query_lens, "query_lens", torch.int32)
    if seq_lens.dim() != 1 or query_lens.dim() != 1:
        raise ValueError("decode_layout: sequence and query lengths must be one-dimensional")
    if seq_lens.numel() < query_lens.numel():
        raise ValueError("decode_layout: each decode request requires a global sequence length")
    R = query_lens.numel()
    dev = query_lens.device
    if starts is None:
        starts = torch.empty(R + 1, dtype=torch.int32, device=dev)
    if row_ends is None:
        row_ends = torch.empty(max(int(num_rows), 0), dtype=torch.int32, device=dev)
    st = library().dsaidx_decode_layout(
        seq_lens.contiguous().data_ptr(), query_lens.contiguous().data_ptr(), R, int(num_rows),
        int(dcp_rank), int(dcp_world_size), int(interleave), starts.data_ptr(),
        row_ends.data_ptr(), _stream(query_lens))
    _check("decode_layout", st)
    return starts, row_ends


def score_paged(q_rows, heads, weights, cache, num_pages, page_stride, block_table, query_starts,
                row_ends, max_query_len, fmt="mxfp4", section_offset=0, out=None):
    """Score every query row against its request's paged keys.

    Returns FP32 logits [num_rows, max_blocks * 64]; entries at or past a row's bound are
    not written."""
    import torch
    _dev(q_rows, "q_rows", torch.uint8)
    _dev(weights, "weights", torch.bfloat16)
    _dev(cache, "cache", torch.uint8)
    _dev(block_table, "block_table", torch.int32)
    _dev(query_starts, "query_starts", torch.int32)
    _dev(row_ends, "row_ends", torch.int32)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("score_paged: block_table must be [requests, max_blocks], row-major")
    num_rows = row_ends.numel()
    R, mb = block_table.shape
    if out is None:
        out = torch.empty((num_rows, mb * PAGE_TOKENS), dtype=torch.float32, device=q_rows.device)
    _dev(out, "out", torch.float32)
    st = library().dsaidx_score_paged(
        _fmt(fmt), q_rows.data_ptr(), q_rows.stride(0), int(heads), weights.data_ptr(),
        weights.stride(0), cache.data_ptr() + int(section_offset), int(num_pages),
        int(page_stride), block_table.data_ptr(), R, block_table.stride(0),
        query_starts.data_ptr(), row_ends.data_ptr(), num_rows, int(max_query_len),
        out.data_ptr(), out.stride(0), _stream(q_rows))
    _check("score_paged", st)
    return out


def score_topk_workspace_bytes(num_requests, max_blocks, num_rows) -> int:
    return int(library().dsaidx_score_topk_workspace_bytes(int(num_requests), int(max_blocks),
                                                           int(num_rows)))


def score_segment_keys(num_requests, max_blocks) -> int:
    """Keys per top-k histogram segment (one scoring workgroup's keys) for these sizes."""
    return int(library().dsaidx_score_segment_keys(int(num_requests), int(max_blocks)))


def read_sections(cache, num_pages, page_stride, block_table, seq_lens, fmt="mxfp4",
                  section_offset=0, out=None):
    """A plain read of the cache sections score_paged reads (a bandwidth reference, not a step
    of the path). Returns uint32 [words]: one XOR word per wavefront; their XOR is the XOR of
    every 32-bit word of every section read."""
    import torch
    _dev(cache, "cache", torch.uint8)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [num_requests, max_blocks] tensor")
    nreq, max_blocks = block_table.shape
    if seq_lens.shape != (nreq,):
        raise ValueError("seq_lens must be [num_requests]")
    lib = library()
    words = int(lib.dsaidx_read_sections_words(int(nreq), int(max_blocks)))
    if out is None:
        out = torch.zeros(max(words, 1), dtype=torch.int32, device=cache.device)
    _check("read_sections", lib.dsaidx_read_sections(
        _fmt(fmt), cache.data_ptr() + section_offset, num_pages, page_stride,
        block_table.data_ptr(), nreq, max_blocks, seq_lens.data_ptr(), out.data_ptr(),
        out.numel(), _stream(cache)))
    return out


def read_stream(buf, workgroups, nbytes=None, out=None):
    """A plain contiguous read of the first `nbytes` (default: all) bytes of the uint8 device
    tensor `buf` by `workgroups` workgroups (a bandwidth reference, not a step of the path).
    Returns uint32 [4 * workgroups] XOR words, one per wavefront."""
    import torch
    _dev(buf, "buf", torch.uint8)
    nbytes = buf.numel() if nbytes is None else int(nbytes)
    if nbytes > buf.numel() or not buf.is_contiguous():
        raise ValueError("read_stream: nbytes beyond a contiguous buffer")
    if out is None:
        out = torch.zeros(4 * int(workgroups), dtype=torch.int32, device=buf.device)
    _check("read_stream", library().dsaidx_read_stream(buf.data_ptr(), nbytes, int(workgroups),
                                                       out.data_ptr(), out.numel(), _stream(buf)))
    return out


def score_topk(q_rows, heads, weights, cache, num_pages, page_stride, block_table, query_starts,
               row_ends, max_query_len, k, fmt="mxfp4", section_offset=0, out=None, indices=None,
               workspace=None):
    """score_paged followed by topk with one pass fewer over the logits: the scorer writes the
    selection's histograms. Returns (logits FP32 [rows, max_blocks*64], indices int32 [rows, k])."""
    import torch
    _dev(q_rows, "q_rows", torch.uint8)
    _dev(weights, "weights", torch.bfloat16)
    _dev(cache, "cache", torch.uint8)
    _dev(block_table, "block_table", torch.int32)
    _dev(query_starts, "query_starts", torch.int32)
    _dev(row_ends, "row_ends", torch.int32)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("score_topk: block_table must be [requests, max_blocks], row-major")
    num_rows = row_ends.numel()
    R, mb = block_table.shape
    if out is None:
        out = torch.empty((num_rows, mb * PAGE_TOKENS), dtype=torch.float32, device=q_rows.device)
    if indices is None:
        indices = torch.empty((num_rows, int(k)), dtype=torch.int32, device=q_rows.device)
    _dev(out, "out", torch.float32)
    _dev(indices, "indices", torch.int32)
    need = score_topk_workspace_bytes(R, mb, num_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_rows.device)
    lib = library()
    st = lib.dsaidx_score_paged_hist(
        _fmt(fmt), q_rows.data_ptr(), q_rows.stride(0), int(heads), weights.data_ptr(),
        weights.stride(0), cache.data_ptr() + int(section_offset), int(num_pages),
        int(page_stride), block_table.data_ptr(), R, block_table.stride(0),
        query_starts.data_ptr(), row_ends.data_ptr(), num_rows, int(max_query_len),
        out.data_ptr(), out.stride(0), workspace.data_ptr(), workspace.numel(), _stream(q_rows))
    _check("score_paged_hist", st)
    st = lib.dsaidx_topk_scored(out.data_ptr(), num_rows, out.stride(0), row_ends.data_ptr(),
                                int(k), indices.data_ptr(), indices.stride(0), R, mb,
                                workspace.data_ptr(), workspace.numel(), _stream(q_rows))
    _check("topk_scored", st)
    return out, indices


def decode_tile_size(max_model_len, width, topk, heads) -> int:
    """Rows per tile that bound logits, selection scratch and queries (page
    "vllm.models.kimi_k3.amd.ops.fp4_indexer", decode_tile_size)."""
    return int(library().dsaidx_decode_tile_size(int(max_model_len), int(width), int(topk),
                                                 int(heads)))


def score_topk_tiled(q_rows, heads, weights, cache, num_pages, page_stride, block_table,
                     query_starts, row_ends, max_query_len, k, tile_rows, fmt="mxfp4",
                     section_offset=0, indices=None, logits_tile=None, workspace=None):
    """score_topk over row tiles of `tile_rows` rows: only one tile's logits and selection
    scratch exist at a time. Returns (indices int32 [rows, k], logits_tile FP32
    [tile_rows, max_blocks*64] holding the last tile's logits)."""
    import torch
    _dev(q_rows, "q_rows", torch.uint8)
    _dev(weights, "weights", torch.bfloat16)
    _dev(cache, "cache", torch.uint8)
    _dev(block_table, "block_table", torch.int32)
    _dev(query_starts, "query_starts", torch.int32)
    _dev(row_ends, "row_ends", torch.int32)
    if block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [num_requests, max_blocks] tensor")
    nreq, max_blocks = block_table.shape
    rows = q_rows.shape[0]
    width = max_blocks * 64
    dev_ = q_rows.device
    if indices is None:
        indices = torch.empty((rows, k), dtype=torch.int32, device=dev_)
    if logits_tile is None:
        logits_tile = torch.empty((int(tile_rows), width), dtype=torch.float32, device=dev_)
    lib = library()
    need = int(lib.dsaidx_score_topk_tiled_workspace_bytes(nreq, max_blocks, int(tile_rows),
                                                           int(max_query_len)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev_)
    _check("score_topk_tiled", lib.dsaidx_score_topk_tiled(
        _fmt(fmt), q_rows.data_ptr(), q_rows.stride(0), heads, weights.data_ptr(),
        weights.stride(0), cache.data_ptr() + section_offset, num_pages, page_stride,
        block_table.data_ptr(), nreq, max_blocks, query_starts.data_ptr(), row_ends.data_ptr(),
        rows, max_query_len, k, indices.data_ptr(), indices.stride(0), int(tile_rows),
        logits_tile.data_ptr(), logits_tile.stride(0), workspace.data_ptr(), workspace.numel(),
        _stream(q_rows)))
    return indices, logits_tile


def index_score_topk(projected, key_col, weight_col, q, gamma, beta, eps, seq_lens, query_lens,
                     num_rows, cache, num_pages, page_stride, block_table, max_query_len, k,
                     fmt="mxfp4", section_offset=0, out=None, indices=None, workspace=None):
    """One step with its selection (dsaidx_index_score_topk): the step's inputs made inside the
    scorer (query quantization, key insert at the block table's positions, row layout, logits),
    then every row's top-k -- in the scoring launch itself where every request has one row that
    one scoring workgroup covers, else on the scorer's histograms (topk_scored). Returns
    (query_starts, row_ends, logits, indices)."""
    import torch
    _dev(projected, "projected", torch.bfloat16)
    _dev(q, "q", torch.bfloat16)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(query_lens, "query_lens", torch.int32)
    _dev(cache, "cache", torch.uint8)
    _dev(block_table, "block_table", torch.int32)
    if projected.dim() != 2 or projected.stride(1) != 1 or q.dim() != 3 or q.stride(2) != 1 \
            or q.shape[0] < int(num_rows) or projected.shape[0] < int(num_rows):
        raise ValueError("index_score_topk: projected [rows, cols], q [rows, heads, 128]")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("index_score_topk: block_table must be [requests, max_blocks], row-major")
    dev = q.device
    R, mb = block_table.shape
    num_rows = int(num_rows)
    starts = torch.empty(R + 1, dtype=torch.int32, device=dev)
    ends = torch.empty(max(num_rows, 0), dtype=torch.int32, device=dev)
    logits = out
    if logits is None:
        logits = torch.empty((num_rows, mb * PAGE_TOKENS), dtype=torch.float32, device=dev)
    if indices is None:
        indices = torch.empty((num_rows, int(k)), dtype=torch.int32, device=dev)
    _dev(logits, "out", torch.float32)
    _dev(indices, "indices", torch.int32)
    if workspace is None:
        need = score_topk_workspace_bytes(R, mb, num_rows)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    lib = library()
    st = lib.dsaidx_index_score_topk(
        _fmt(fmt), projected.data_ptr(), projected.stride(0), int(key_col), int(weight_col),
        q.data_ptr(), q.shape[1], q.stride(0), q.stride(1), gamma.data_ptr(), beta.data_ptr(),
        float(eps), seq_lens.contiguous().data_ptr(), query_lens.contiguous().data_ptr(), R,
        num_rows, int(max_query_len), cache.data_ptr() + int(section_offset), int(num_pages),
        int(page_stride), block_table.data_ptr(), mb, starts.data_ptr(), ends.data_ptr(),
        logits.data_ptr(), logits.stride(0), int(k), indices.data_ptr(), indices.stride(0),
        workspace.data_ptr(), workspace.numel(), _stream(q))
    _check("index_score_topk", st)
    return starts, ends, logits, indices


def topk_workspace_bytes(rows, width, k) -> int:
    return int(library().dsaidx_topk_workspace_bytes(int(rows), int(width), int(k)))


def topk(logits, row_ends, k, width=None, out=None, workspace=None):
    """Per-row top-k key positions of logits [rows, >= width] over [0, row_ends[r]).

    Returns int32 [rows, k]; the order within a row is unspecified; unused entries are -1."""
    import torch
    _dev(logits, "logits", torch.float32)
    _dev(row_ends, "row_ends", torch.int32)
    rows = logits.shape[0]
    width = logits.shape[1] if width is None else int(width)
    if out is None:
        out = torch.empty((rows, int(k)), dtype=torch.int32, device=logits.device)
    _dev(out, "out", torch.int32)
    need = topk_workspace_bytes(rows, width, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    st = library().dsaidx_topk(
        logits.data_ptr(), rows, width, logits.stride(0), row_ends.data_ptr(), int(k),
        out.data_ptr(), out.stride(0), None if workspace is None else workspace.data_ptr(),
        0 if workspace is None else workspace.numel(), _stream(logits))
    _check("topk", st)
    return out


def dcp_candidates(logits, indices, rank, world, interleave, width=None, values=None,
                   positions=None):
    """One DCP rank's merge candidates from its local top-k: (values FP32 [rows, k], global
    positions int32 [rows, k]); pass slices of the gathered [world, rows, k] buffers as
    values / positions to write in place."""
    import torch
    _dev(logits, "logits", torch.float32)
    _dev(indices, "indices", torch.int32)
    rows, k = indices.shape
    width = logits.shape[1] if width is None else int(width)
    if values is None:
        values = torch.empty((rows, k), dtype=torch.float32, device=logits.device)
    if positions is None:
        positions = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    if not (values.is_contiguous() and positions.is_contiguous()):
        raise ValueError("dcp_candidates: values and positions must be contiguous [rows, k]")
    st = library().dsaidx_dcp_candidates(
        logits.data_ptr(), rows, width, logits.stride(0), indices.data_ptr(), k,
        indices.stride(0), int(rank), int(world), int(interleave), values.data_ptr(),
        positions.data_ptr(), _stream(logits))
    _check("dcp_candidates", st)
    return values, positions


def dcp_merge(values, positions, k, rank=None, interleave=1):
    """Global top-k of every row from all ranks' candidates (values / positions
    [world, rows, kc]). Returns merged global positions int32 [rows, k], and with `rank` also
    that rank's local slots int32 [rows, k]."""
    import torch
    _dev(values, "values", torch.float32)
    _dev(positions, "positions", torch.int32)
    if values.dim() != 3 or values.shape != positions.shape or not values.is_contiguous() \
            or not positions.is_contiguous():
        raise ValueError("dcp_merge: values and positions must be contiguous [world, rows, kc]")
    world, rows, kc = values.shape
    merged = torch.empty((rows, int(k)), dtype=torch.int32, device=values.device)
    local = None if rank is None else torch.empty_like(merged)
    st = library().dsaidx_dcp_merge(
        values.data_ptr(), positions.data_ptr(), world, rows, kc, int(k), merged.data_ptr(),
        merged.stride(0), -1 if rank is None else int(rank), int(interleave),
        None if local is None else local.data_ptr(), 0 if local is None else local.stride(0),
        _stream(values))
    _check("dcp_merge", st)
    return merged if local is None else (merged, local)
