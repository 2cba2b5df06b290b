"""GPU decode context parallelism on one device: every rank's shard scored at its real shape
(rank-local block tables and bounds), each rank's local top-k turned into merge candidates,
and the merge, checked against the oracle's global top-k of the whole row; plus the merge
alone on crafted candidates (ties, signed zeros, empty and short rows) against the oracle
merge."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_quant_amd as dsa
from gpu_util import DeviceWorkload, assert_topk_sets, dev
from sparse_attention_indexer_quant_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


@pytest.mark.parametrize("world,k", [(4, 256), (2, 2048), (8, 64)])
def test_rank_local_scoring_and_merge_give_global_topk(world, k):
    # interleave 64 = one page per run: rank r owns pages r, r + W, ... of every request, so its
    # block table is every W-th column of the global one, over the same cache
    il = 64
    wl = make_workload("dcp", fmt="mxfp4", heads=32, seq_lens=[5000, 1500, 700, 65],
                       query_lens=[1, 1, 1, 1], topk=k, seed=60 + world)
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    q_rows, w = dw.quantize()
    starts, gends = dw.layout()
    glog = dw.score(q_rows, w, starts, gends)                  # global logits (reference input)
    R, rows = wl.num_requests, wl.num_rows
    vals = torch.empty((world, rows, k), dtype=torch.float32, device="cuda")
    poss = torch.empty((world, rows, k), dtype=torch.int32, device="cuda")
    local_idx = []
    for r in range(world):
        bt = wl.block_table[:, r::world]
        bt = np.ascontiguousarray(bt) if bt.shape[1] else np.full((R, 1), -1, np.int32)
        _, lends = dsa.decode_layout(dw.seq_lens, dw.query_lens, rows, r, world, il)
        llog = dsa.score_paged(q_rows, wl.heads, w, dw.cache, wl.num_pages, wl.page_stride,
                               dev(bt), starts, lends, wl.max_query_len, wl.fmt)
        lidx = dsa.topk(llog, lends, k)
        dsa.dcp_candidates(llog, lidx, r, world, il, values=vals[r], positions=poss[r])
        local_idx.append((llog, lidx, lends))
    ge = gends.cpu().numpy()
    want = oracle.topk(np.nan_to_num(glog.cpu().numpy(), nan=0.0), ge, k)
    for r in range(world):
        merged, slots = dsa.dcp_merge(vals, poss, k, rank=r, interleave=il)
        got = merged.cpu().numpy()
        assert_topk_sets(got, want, range(rows), f"world {world} rank {r}")
        # the rank's local slots are exactly the merged keys it owns, as local positions
        sl = slots.cpu().numpy()
        for row in range(rows):
            g = got[row][got[row] >= 0]
            owner, local = oracle.dcp_owner(g, world, il)
            assert sorted(sl[row][sl[row] >= 0].tolist()) == sorted(local[owner == r].tolist())
    # the candidates equal the oracle's from the same local results
    for r, (llog, lidx, lends) in enumerate(local_idx):
        ov, op = oracle.dcp_candidates(llog.cpu().numpy(), lidx.cpu().numpy(), r, world, il)
        assert np.array_equal(poss[r].cpu().numpy(), op)
        assert np.array_equal(vals[r].cpu().numpy(), ov)


@pytest.mark.parametrize("world,kc,k", [(3, 50, 40), (2, 7, 20), (8, 2048, 2048)])
def test_merge_matches_oracle_on_crafted_candidates(world, kc, k):
    rng = np.random.default_rng(world * 7 + kc)
    rows = 6
    v = rng.standard_normal((world, rows, kc)).astype(np.float32)
    v[:, 1] = 1.5                                     # all equal: lower global positions win
    v[:, 2] = np.round(v[:, 2])                       # heavy ties
    v[:, 3, ::2], v[:, 3, 1::2] = -0.0, 0.0           # signed zeros are equal
    perm = rng.permutation(world * kc * 4)[:world * kc].reshape(world, kc)
    p = np.broadcast_to(perm[:, None, :], (world, rows, kc)).copy().astype(np.int64)
    p[:, 4, kc // 3:] = -1                            # some ranks short of candidates
    p[:, 5] = -1                                      # a row with none
    v = np.where(p < 0, -np.inf, v).astype(np.float32)
    want = oracle.dcp_merge(v, p, k)
    got = dsa.dcp_merge(dev(v), dev(p.astype(np.int32)), k).cpu().numpy()
    for r in range(rows):
        assert sorted(got[r].tolist()) == sorted(want[r].tolist()), r
