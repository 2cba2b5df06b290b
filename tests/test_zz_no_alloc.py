"""The allocation-free top-k (dsaidx_topk_noalloc, for callers that cannot allocate) against
dsaidx_topk with a caller workspace, through the C-ABI: the same index sets on two calls in a
row, the second with a smaller input, both also against the oracle's top-k; sizes beyond the
static scratch rejected with nothing written."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_quant_amd as dsa
from gpu_util import assert_topk_sets, dev

pytestmark = pytest.mark.gpu

ESCRATCH = 5


def _logits(rows, width, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((rows, width)).astype(np.float32)
    lg[0, ::7] = 0.5                               # ties across the boundary
    lg[-1] = np.round(lg[-1] * 2) / 2              # heavy ties
    ends = rng.integers(0, width + 1, size=rows).astype(np.int32)
    ends[0] = width
    ends[1 % rows] = 0                             # an empty row
    return lg, ends


def _both(lib, lg_t, ends_t, width, k):
    rows = lg_t.shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = torch.empty(max(int(lib.dsaidx_topk_workspace_bytes(rows, width, k)), 1),
                     dtype=torch.uint8, device="cuda")
    a = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    b = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    st = lib.dsaidx_topk(lg_t.data_ptr(), rows, width, lg_t.stride(0), ends_t.data_ptr(), k,
                         a.data_ptr(), a.stride(0), ws.data_ptr(), ws.numel(), stream)
    assert st == 0, st
    st = lib.dsaidx_topk_noalloc(lg_t.data_ptr(), rows, width, lg_t.stride(0), ends_t.data_ptr(),
                                 k, b.data_ptr(), b.stride(0), stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_topk_noalloc_matches_topk_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = dsa.library()
    # first the verify workload's selection size (512 rows x 65536 keys, the segmented
    # kernels), then a smaller one (16 rows x 8192 keys, one workgroup per row)
    for rows, width, k, seed in [(512, 65536, 2048, 31), (16, 8192, 2048, 32)]:
        print(f"[noalloc] rows={rows} width={width} k={k}", flush=True)
        lg, ends = _logits(rows, width, seed)
        ref, got = _both(lib, dev(lg), dev(ends), width, k)
        assert_topk_sets(got, ref, range(rows), f"noalloc vs topk {rows}x{width}")
        want = oracle.topk(lg, ends, k)
        assert_topk_sets(got, want, range(rows), f"noalloc vs oracle {rows}x{width}")


def test_topk_noalloc_rejects_sizes_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = dsa.library()
    rows, width, k = 2048, 65536, 2048
    assert lib.dsaidx_topk_workspace_bytes(rows, width, k) > (64 << 20)
    lg = torch.zeros((rows, width), dtype=torch.float32, device="cuda")
    ends = torch.full((rows,), width, dtype=torch.int32, device="cuda")
    out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    st = lib.dsaidx_topk_noalloc(lg.data_ptr(), rows, width, width, ends.data_ptr(), k,
                                 out.data_ptr(), k, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == ESCRATCH
    assert torch.all(out == -7)
