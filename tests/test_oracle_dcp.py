"""Oracle pins for decode context parallelism (DCP): the interleaved key ownership agrees with
decode_layout's rank-local bounds (page "vllm.models.kimi_k3.amd.ops.fp4_indexer",
decode_layout), and merging every rank's local top-k gives the global top-k of the whole row
(page "...cutedsl.dsa.overlap", module text: the top-k merge and the local slots)."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("world,interleave", [(2, 1), (3, 64), (4, 16), (8, 64)])
def test_owner_round_trip_and_layout_counts(world, interleave):
    g = np.arange(5000)
    rank, local = oracle.dcp_owner(g, world, interleave)
    for r in range(world):
        mine = g[rank == r]
        # rank-local positions are 0, 1, 2, ... in global order, and map back exactly
        assert np.array_equal(local[rank == r], np.arange(mine.size))
        assert np.array_equal(oracle.dcp_global_position(np.arange(mine.size), r, world, interleave), mine)
    # decode_layout's rank-local bound = the number of the rank's keys below the global bound
    seq = np.array([1, 63, 64, 65, 777, 4096, 4999], np.int32)
    ql = np.ones(seq.size, np.int32)
    for r in range(world):
        _, ends = oracle.decode_layout(seq, ql, seq.size, r, world, interleave)
        want = [int(np.sum(rank[:n] == r)) for n in seq]
        assert list(ends) == want


def _split_and_merge(lg, ends, k, world, interleave):
    """Each rank's local rows (its keys in global order), its local top-k, the candidates,
    the merge, and every rank's local slots."""
    rows, width = lg.shape
    vals, poss, per_rank = [], [], []
    for r in range(world):
        mine = np.nonzero(oracle.dcp_owner(np.arange(width), world, interleave)[0] == r)[0]
        local = lg[:, mine] if mine.size else np.zeros((rows, 1), np.float32)
        lend = np.array([int(np.sum(mine < e)) for e in ends], np.int32)
        idx = oracle.topk(local, lend, k)
        v, p = oracle.dcp_candidates(local, idx, r, world, interleave)
        vals.append(v)
        poss.append(p)
        per_rank.append(mine)
    merged = oracle.dcp_merge(np.stack(vals), np.stack(poss), k)
    return merged


@pytest.mark.parametrize("world,interleave", [(2, 1), (4, 64), (3, 7)])
@pytest.mark.parametrize("k", [1, 50, 300])
def test_merge_of_local_topk_is_global_topk(world, interleave, k):
    rng = np.random.default_rng(world * 100 + k)
    rows, width = 7, 1000
    lg = rng.standard_normal((rows, width)).astype(np.float32)
    lg[1] = 0.5                                   # all equal: ties to the lower global position
    lg[2] = np.round(lg[2] * 2) / 2               # heavy ties across ranks
    lg[3, ::2], lg[3, 1::2] = -0.0, 0.0           # signed zeros are equal
    lg[4, 200:] = -1e30
    ends = np.array([1000, 1000, 999, 1000, 150, 0, 40], np.int32)
    merged = _split_and_merge(lg, ends, k, world, interleave)
    want = oracle.topk(lg, ends, k)
    for r in range(rows):
        assert sorted(merged[r].tolist()) == sorted(want[r].tolist()), r


def test_local_slots_partition_the_merge():
    rng = np.random.default_rng(5)
    world, interleave, k = 4, 8, 64
    lg = rng.standard_normal((3, 700)).astype(np.float32)
    ends = np.array([700, 333, 5], np.int32)
    merged = _split_and_merge(lg, ends, k, world, interleave)
    back = [[] for _ in range(3)]
    for rank in range(world):
        slots = oracle.dcp_local_slots(merged, rank, world, interleave)
        for r in range(3):
            loc = slots[r][slots[r] >= 0]
            assert np.all(oracle.dcp_owner(oracle.dcp_global_position(loc, rank, world, interleave),
                                           world, interleave)[0] == rank)
            back[r] += oracle.dcp_global_position(loc, rank, world, interleave).tolist()
    for r in range(3):
        assert sorted(back[r]) == sorted(merged[r][merged[r] >= 0].tolist())
