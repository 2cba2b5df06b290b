"""Pins of the oracle's hot-path stages: closed forms, lossless layouts decoded by an
independent NumPy decoder, hand-worked row bounds and top-k sets, and brute-force FP64
scores on tiny inputs. No GPU needed."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import npdecode
from goldens import byte_list, f32, int_list, layernorm_order_key, rows
from sparse_attention_indexer_quant_amd.workloads import bf16_bits, bf16_to_f32, make_workload

E2M1_GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


# ---- LayerNorm (page "...cutedsl.dsa.index", insert_key) ----------------------------------

def test_layernorm_constant_key_gives_beta():
    rng = np.random.default_rng(1)
    gamma = bf16_to_f32(bf16_bits(1 + 0.1 * rng.standard_normal(128).astype(np.float32)))
    beta = bf16_to_f32(bf16_bits(0.1 * rng.standard_normal(128).astype(np.float32)))
    for c in (0.0, 1.0, -3.5, 1e-3, 250.0):
        out = oracle.layernorm128(np.full(128, c, np.float32), gamma, beta, 1e-6)
        assert np.array_equal(out, beta), c


def test_layernorm_alternating_closed_form():
    # x = +1, -1, ... : mean 0 and variance 1 exactly, so with eps = 0, y = +-gamma + beta.
    rng = np.random.default_rng(2)
    gamma = bf16_to_f32(bf16_bits(1 + 0.1 * rng.standard_normal(128).astype(np.float32)))
    beta = bf16_to_f32(bf16_bits(0.1 * rng.standard_normal(128).astype(np.float32)))
    x = np.tile(np.array([1.0, -1.0], np.float32), 64)
    out = oracle.layernorm128(x, gamma, beta, 0.0)
    want = torch.from_numpy(x * gamma + beta).to(torch.bfloat16).float().numpy()
    assert np.array_equal(out, want)


def test_layernorm_within_one_bf16_step_of_exact():
    rng = np.random.default_rng(3)
    gamma = bf16_to_f32(bf16_bits(1 + 0.1 * rng.standard_normal(128).astype(np.float32)))
    beta = bf16_to_f32(bf16_bits(0.1 * rng.standard_normal(128).astype(np.float32)))
    for t in range(300):
        scale = 10.0 ** rng.uniform(-3, 3)
        x = bf16_to_f32(bf16_bits((rng.standard_normal(128) * scale + rng.standard_normal()).astype(np.float32)))
        out = oracle.layernorm128(x, gamma, beta, 1e-6)
        exact = F.layer_norm(torch.from_numpy(x.astype(np.float64)), (128,),
                             torch.from_numpy(gamma.astype(np.float64)),
                             torch.from_numpy(beta.astype(np.float64)), eps=1e-6).numpy()
        step = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
        assert np.all(np.abs(out - exact) <= step * 1.0001 + 1e-30), t


def test_layernorm_page_summation_order_golden():
    # tests/golden/layernorm_order.txt: a key whose sums, BF16 outputs and MXFP4 bytes differ
    # between the page's per-lane running totals and other summation orders, worked by hand.
    x, gamma, beta = layernorm_order_key()
    gold = {}
    for line in rows("layernorm_order.txt"):
        kind, *vals = line.split()
        gold.setdefault(kind, []).append(vals)
    assert oracle.ln_sum128(x) == float(gold["sum"][0][0])
    # a different order of the same values is not what the oracle computes
    assert float(gold["mean_alternative_order_sum"][0][0]) != oracle.ln_sum128(x)
    out = oracle.layernorm128(x, gamma, beta, 1e-6)
    for col, val in gold["normed"]:
        assert out[int(col)] == f32(val), col
    cache = np.zeros(4352, np.uint8)
    oracle.store_keys(bf16_bits(x).reshape(1, 128), gamma, beta, 1e-6, np.array([5]), cache, 1, 4352)
    assert list(cache[5 * 64:6 * 64]) == byte_list(gold["mxfp4_payload"][0][0])
    assert list(cache[4096 + 20:4096 + 24]) == byte_list(gold["mxfp4_scales"][0][0])
    # every other byte of the section untouched
    rest = np.delete(cache, np.r_[5 * 64:6 * 64, 4096 + 20:4096 + 24])
    assert not rest.any()


def test_ln_sum_running_totals_then_butterfly():
    # Structure of the page's order on values where each step is exact except where stated:
    # a lane's total absorbs ones into a leading 2^24 (ties to even), but ones summed before
    # they meet 2^24 survive. Columns 0..7 = [1, 1, 1, 1, 1, 1, 1, 2^24]: the running total
    # reaches 7 before adding 2^24, and 2^24 + 7 rounds to 2^24 + 8 (spacing 2, tie 7 -> 8).
    z = np.zeros(128, np.float32)
    z[:7] = 1.0
    z[7] = 2.0 ** 24
    assert oracle.ln_sum128(z) == 2.0 ** 24 + 8
    # the same values in the other order (2^24 first) lose every one: 2^24
    z2 = np.zeros(128, np.float32)
    z2[0] = 2.0 ** 24
    z2[1:8] = 1.0
    assert oracle.ln_sum128(z2) == 2.0 ** 24
    # ones in lanes that meet 2^24 only in the combine: lane j = 8 holds 2^24 alone, lanes
    # 0..7 hold 8 ones each (total 8); offset 8 pairs lane 0 with lane 8: 8 + 2^24 (exact),
    # then offsets 4, 2, 1 add 8 + 8, 16 + 16, 32 + ... -> 2^24 + 64 exactly.
    z3 = np.zeros(128, np.float32)
    z3[:64] = 1.0
    z3[64] = 2.0 ** 24
    assert oracle.ln_sum128(z3) == 2.0 ** 24 + 64


# ---- quantize_queries layouts (page "...cutedsl.dsa.index", quantize_fp4_query, fp8_query) --

def _lossless_fp4_queries(rows_, heads, seed):
    # every 32-column block holds all 16 E2M1 grid values twice, times 2^k: amax = 6 * 2^k, so the
    # block scale is exactly 2^k and every value is representable.
    rng = np.random.default_rng(seed)
    q = np.zeros((rows_, heads, 128), np.float32)
    for r in range(rows_):
        for h in range(heads):
            for g in range(4):
                k = int(rng.integers(-20, 20))
                q[r, h, 32 * g:32 * g + 32] = rng.permutation(np.concatenate([E2M1_GRID, E2M1_GRID])) * 2.0 ** k
    return q


@pytest.mark.parametrize("heads", [16, 32, 64])
def test_quantize_fp4_lossless_layout(heads):
    q = _lossless_fp4_queries(3, heads, heads)
    wv = np.random.default_rng(7).standard_normal((3, heads)).astype(np.float32)
    out, w_out = oracle.quantize_queries(bf16_bits(q), bf16_bits(wv), "mxfp4")
    assert out.shape == (3, heads * 68)
    deq = npdecode.mxfp4_query_rows(out, heads)
    assert np.array_equal(deq, q.astype(np.float64))
    # signed zeros survive with their sign (code 8)
    assert np.array_equal(np.signbit(deq), np.signbit(q))
    # MXFP4 head weights only carry c_H: BF16(wv * c_H)
    c = np.float32(oracle.head_weight_scale(heads))
    want = torch.from_numpy(bf16_to_f32(bf16_bits(wv)) * c).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bf16_to_f32(w_out), want)


def test_quantize_fp4_error_bound_random():
    # random N(0,1) queries: each block's scale is the smallest 2^e with amax <= 6 * 2^e, and every
    # dequantized value is within half a grid step (or saturates at the block's 6 * 2^e).
    rng = np.random.default_rng(8)
    q = bf16_to_f32(bf16_bits(rng.standard_normal((4, 32, 128)).astype(np.float32) * 3))
    out, _ = oracle.quantize_queries(bf16_bits(q), None, "mxfp4")
    deq = npdecode.mxfp4_query_rows(out, 32)
    sc = out[:, 32 * 64:].reshape(4, 32, 4).astype(np.int64) - 127
    amax = np.abs(q).reshape(4, 32, 4, 32).max(-1)
    assert np.all(amax <= 6.0 * np.exp2(sc)) and np.all(amax > 3.0 * np.exp2(sc))
    step = np.repeat(np.exp2(sc), 32, axis=-1)  # largest grid spacing (2) x half x scale
    assert np.all(np.abs(deq - q) <= step + 1e-30)


def test_quantize_fp8_lossless_layout():
    # heads of E4M3 values times 2^k with one element at 448 * 2^k: s = 2^k exactly, lossless.
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 0x7F, size=(2, 32, 128))
    codes = np.where(rng.random((2, 32, 128)) < 0.5, codes, codes | 0x80)
    vals = npdecode.e4m3(codes)
    ks = rng.integers(-10, 10, size=(2, 32))
    vals[:, :, 3] = 448.0
    q = (vals * np.exp2(ks)[:, :, None]).astype(np.float32)
    wv = np.ones((2, 32), np.float32)
    out, w_out = oracle.quantize_queries(bf16_bits(q), bf16_bits(wv), "fp8")
    assert out.shape == (2, 32 * 128)
    deq = npdecode.fp8_query_rows(out, 32) * np.exp2(ks)[:, :, None]
    assert np.array_equal(deq, q.astype(np.float64))
    assert np.array_equal(bf16_to_f32(w_out), np.exp2(ks - 6.0).astype(np.float32))


# ---- store_keys (page "...cutedsl.dsa.index", insert_key / insert_fp4_key;
#      page "...amd.ops.fp4_indexer", store_keys, cache_views) --------------------------------

def _lossless_beta(fmt, rng):
    if fmt == "mxfp4":
        return np.concatenate([rng.permutation(np.concatenate([E2M1_GRID, E2M1_GRID])) * 2.0 ** int(rng.integers(-8, 8))
                               for _ in range(4)]).astype(np.float32)
    v = npdecode.e4m3(rng.integers(0, 0xFF, size=128) & 0xF7)  # finite codes
    v[5] = 448.0
    return (v * 2.0 ** int(rng.integers(-8, 8))).astype(np.float32)


@pytest.mark.parametrize("fmt,stride,offset", [("mxfp4", 4352, 0), ("mxfp4", 8192, 3840),
                                               ("mxfp4", 8192, 0), ("fp8", 8448, 0),
                                               ("fp8", 9216, 512)])
def test_store_keys_layout_padding_and_filler(fmt, stride, offset):
    # A constant pre-norm key normalizes to exactly beta; a beta that quantizes losslessly pins
    # where every byte goes. Negative and out-of-range slots write nothing; bytes outside the
    # index sections keep their 0xA5 filler.
    rng = np.random.default_rng(10)
    pages = 3
    section = 4352 if fmt == "mxfp4" else 8448
    nbytes = offset + (pages - 1) * stride + section
    cache = np.full(nbytes, 0xA5, np.uint8)
    gamma = np.ones(128, np.float32)
    slots = np.array([0, 130, -1, 63, 64 * pages, 77], np.int64)
    betas = [_lossless_beta(fmt, rng) for _ in slots]
    touched = np.zeros(nbytes, bool)
    for i, s in enumerate(slots):
        keys = bf16_bits(np.full((1, 128), float(i) - 2.0, np.float32))
        oracle.store_keys(keys, gamma, betas[i], 1e-6, np.array([s]), cache, pages, stride, offset, fmt)
        if 0 <= s < 64 * pages:
            page, off = divmod(int(s), 64)
            if fmt == "mxfp4":
                got = npdecode.mxfp4_key(cache, page, off, stride, offset)
                base = offset + page * stride
                touched[base + off * 64: base + off * 64 + 64] = True
                touched[base + 4096 + off * 4: base + 4096 + off * 4 + 4] = True
                assert np.array_equal(got, betas[i].astype(np.float64))
            else:
                got, scale = npdecode.fp8_key(cache, page, off, stride, offset)
                base = offset + page * stride
                touched[base + off * 128: base + off * 128 + 128] = True
                touched[base + 8192 + off * 4: base + 8192 + off * 4 + 4] = True
                assert np.array_equal(got, betas[i].astype(np.float64))
                assert scale == np.abs(betas[i]).max() / 448.0
    assert np.all(cache[~touched] == 0xA5)


@pytest.mark.parametrize("k", [-10, 0, 7])
def test_store_keys_fp8_mx_scale_bytes(k):
    # the mx variant ([idx] module text and insert_key, mx): a key normalizing to E4M3 values
    # with amax 448 * 2^k has scale 2^k, stored as four equal UE8M0 bytes k + 127, and the
    # same payload bytes as the FP32-scale variant
    rng = np.random.default_rng(40 + k)
    v = npdecode.e4m3(rng.integers(0, 0xFF, size=128) & 0xF7)
    v[9] = -448.0
    beta = (v * 2.0 ** k).astype(np.float32)
    key = bf16_bits(np.full((1, 128), 3.0, np.float32))        # normalizes to beta exactly
    caches = {}
    for fmt in ("fp8", "fp8_mx"):
        c = np.full(8448 * 2, 0xA5, np.uint8)
        oracle.store_keys(key, np.ones(128, np.float32), beta, 1e-6, np.array([64 + 5]), c, 2,
                          8448, 0, fmt)
        caches[fmt] = c
    vals, scale, sb = npdecode.fp8_mx_key(caches["fp8_mx"], 1, 5, 8448)
    assert np.all(sb == k + 127) and scale == 2.0 ** k
    assert np.array_equal(vals, beta.astype(np.float64))
    payload = slice(8448 + 5 * 128, 8448 + 6 * 128)
    assert np.array_equal(caches["fp8"][payload], caches["fp8_mx"][payload])
    # nothing else differs between the two layouts
    diff = np.nonzero(caches["fp8"] != caches["fp8_mx"])[0]
    assert np.all((diff >= 8448 + 8192 + 5 * 4) & (diff < 8448 + 8192 + 6 * 4))


def test_store_keys_fp8_mx_zero_key_scale_floor():
    # an all-zero normalized key: amax floored at FP32(1e-10), scale 2^-42, bytes 85
    cache = np.zeros(8448, np.uint8)
    oracle.store_keys(bf16_bits(np.ones((1, 128), np.float32)), np.ones(128, np.float32),
                      np.zeros(128, np.float32), 1e-6, np.array([9]), cache, 1, 8448, 0, "fp8_mx")
    vals, scale, sb = npdecode.fp8_mx_key(cache, 0, 9, 8448)
    assert scale == 2.0 ** -42 and np.all(sb == 85) and np.all(vals == 0)


def test_store_keys_fp8_zero_key_scale_floor():
    # an all-zero normalized key: amax floored at FP32(1e-10) gives s = 2^-42 and zero codes
    cache = np.zeros(8448, np.uint8)
    oracle.store_keys(bf16_bits(np.ones((1, 128), np.float32)), np.ones(128, np.float32),
                      np.zeros(128, np.float32), 1e-6, np.array([9]), cache, 1, 8448, 0, "fp8")
    vals, scale = npdecode.fp8_key(cache, 0, 9, 8448)
    assert scale == 2.0 ** -42 and np.all(vals == 0)


# ---- index_inputs (page "...cutedsl.dsa.index", DsaIndex: per token, query quant + head
#      weights from the packed projection row + key LayerNorm and insert) ------------------

def _packed_rows(tokens, cols, key_col, weight_col, keys, wv, rng):
    # filler columns hold NaN/Inf and huge BF16 patterns: nothing outside the key and weight
    # columns may reach any output
    filler = rng.choice(np.array([0x7FC0, 0xFF80, 0x7F80, 0x7F7F, 0xFF7F], np.uint16),
                        size=(tokens, cols))
    proj = filler.copy()
    proj[:, key_col:key_col + 128] = bf16_bits(keys)
    proj[:, weight_col:weight_col + wv.shape[1]] = bf16_bits(wv)
    return proj


@pytest.mark.parametrize("fmt,heads,key_col,weight_col,stride,offset",
                         [("mxfp4", 32, 4096, 4224, 4352, 0), ("mxfp4", 64, 0, 200, 8192, 3840),
                          ("fp8", 32, 130, 2, 8448, 0)])
def test_index_inputs_columns_and_layout(fmt, heads, key_col, weight_col, stride, offset):
    # Lossless queries, constant pre-norm keys (normalize to beta exactly) with lossless betas,
    # and head weights that scale exactly: every output decodes back to its input, and only
    # the key and weight columns of the packed row are read.
    rng = np.random.default_rng(21)
    tokens, pages = 4, 3
    if fmt == "mxfp4":
        q = _lossless_fp4_queries(tokens, heads, 22)
    else:
        codes = rng.integers(0, 0x7F, size=(tokens, heads, 128))
        q = npdecode.e4m3(codes)
        q[:, :, 7] = 448.0
        q = q.astype(np.float32)
    beta = _lossless_beta(fmt, rng)
    keys = np.repeat(np.arange(tokens, dtype=np.float32)[:, None] - 1.5, 128, axis=1)
    wv = (2.0 ** rng.integers(-4, 4, size=(tokens, heads))).astype(np.float32)
    cols = max(key_col + 128, weight_col + heads) + 7
    proj = _packed_rows(tokens, cols, key_col, weight_col, keys, wv, rng)
    slots = np.array([5, -1, 64 * 2 + 17, 64], np.int64)
    section = 4352 if fmt == "mxfp4" else 8448
    cache = np.full(offset + (pages - 1) * stride + section, 0xA5, np.uint8)
    q_out, w_out = oracle.index_inputs(proj, key_col, weight_col, bf16_bits(q), np.ones(128, np.float32),
                                       beta, 1e-6, slots, cache, pages, stride, offset, fmt)
    # head weights: BF16(wv * c_H) (FP8: times s = 1, since every head's amax is 448)
    c = np.float32(oracle.head_weight_scale(heads))
    want_w = torch.from_numpy(wv * c).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bf16_to_f32(w_out), want_w)
    if fmt == "mxfp4":
        assert np.array_equal(npdecode.mxfp4_query_rows(q_out, heads), q.astype(np.float64))
    else:
        assert np.array_equal(npdecode.fp8_query_rows(q_out, heads), q.astype(np.float64))
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        page, off = divmod(int(sl), 64)
        if fmt == "mxfp4":
            got = npdecode.mxfp4_key(cache, page, off, stride, offset)
        else:
            got, _ = npdecode.fp8_key(cache, page, off, stride, offset)
        assert np.array_equal(got, beta.astype(np.float64)), (t, sl)
    # padding token 1 wrote nothing: its would-be slot region still holds filler elsewhere
    untouched = np.ones(cache.size, bool)
    for sl in slots[slots >= 0]:
        page, off = divmod(int(sl), 64)
        base = offset + page * stride
        w = 64 if fmt == "mxfp4" else 128
        untouched[base + off * w: base + off * w + w] = False
        sb = base + (4096 if fmt == "mxfp4" else 8192) + off * 4
        untouched[sb:sb + 4] = False
    assert np.all(cache[untouched] == 0xA5)


# ---- decode_layout (page "...amd.ops.fp4_indexer", decode_layout) -------------------------

def _parse_layout(line):
    lhs, rhs = line.split("->")
    kv = dict(t.split("=", 1) for t in lhs.split())
    out = dict(t.split("=", 1) for t in rhs.split())
    dcp = (0, 1, 1)
    if "dcp" in kv:
        dcp = tuple(int(v) for v in kv["dcp"].split("/"))
    return (int_list(kv["seq"]), int_list(kv["qlen"]), int(kv["rows"]), dcp,
            int_list(out["starts"]), int_list(out["ends"]))


def test_decode_layout_golden():
    n = 0
    for line in rows("decode_layout.txt"):
        seq, ql, nr, (rank, world, il), starts, ends = _parse_layout(line)
        s, e = oracle.decode_layout(seq, ql, nr, rank, world, il)
        assert s.tolist() == starts and e.tolist() == ends, line
        n += 1
    assert n == 10


def test_decode_tile_size_golden():
    # tests/golden/decode_tile_size.txt, worked by hand from page "...amd.ops.fp4_indexer"
    n = 0
    for line in rows("decode_tile_size.txt"):
        mml, width, topk, heads, want = (int(v) for v in line.split())
        assert oracle.decode_tile_size(mml, width, topk, heads) == want, line
        n += 1
    assert n == 7


def test_decode_layout_dcp_shares_sum_to_global():
    rng = np.random.default_rng(14)
    for _ in range(50):
        R = int(rng.integers(1, 6))
        ql = rng.integers(1, 5, R)
        seq = ql + rng.integers(0, 300, R)
        nr = int(ql.sum()) + 3
        world, il = int(rng.integers(2, 5)), int(rng.integers(1, 9))
        _, full = oracle.decode_layout(seq, ql, nr)
        parts = sum(oracle.decode_layout(seq, ql, nr, r, world, il)[1].astype(np.int64) for r in range(world))
        assert np.array_equal(parts, full)


def test_decode_layout_rejects_bad_geometry():
    with pytest.raises(ValueError):
        oracle.decode_layout([5], [1], 1, 2, 2, 1)
    with pytest.raises(ValueError):
        oracle.decode_layout([5], [1], 1, 0, 1, 0)
    with pytest.raises(ValueError):
        oracle.decode_layout([5], [1, 1], 2)


# ---- top-k ----------------------------------------------------------------------------------

def test_topk_golden():
    for line in rows("topk.txt"):
        lhs, rhs = line.split("->")
        vals, re, k = [t.strip() for t in lhs.split(";")]
        lg = np.array([[float(v) for v in vals.split(",")]], np.float32)
        got = oracle.topk(lg, np.array([int(re)], np.int32), int(k))[0]
        assert sorted(got.tolist()) == sorted(int_list(rhs)), line


def test_topk_matches_stable_sort():
    rng = np.random.default_rng(15)
    lg = rng.standard_normal((6, 500)).astype(np.float32)
    lg[:, ::7] = np.round(lg[:, ::7])  # plenty of ties
    lg[2] = 0.0
    lg[3, :250] = -0.0
    re = np.array([500, 0, 500, 311, 37, 499], np.int32)
    for k in (1, 16, 37, 64, 499, 600):
        got = oracle.topk(lg, re, k)
        for r in range(6):
            n = min(re[r], 500)
            order = np.argsort(-lg[r, :n].astype(np.float64), kind="stable")[:k]
            want = np.full(k, -1)
            want[:order.size] = order
            assert np.array_equal(got[r], want), (r, k)


# ---- score_paged ---------------------------------------------------------------------------

def _bf16w(x):
    return bf16_bits(np.asarray(x, np.float32))


def test_score_one_hot_closed_form():
    # 16 heads, weight e0; head 0 of the query is 1.0 in one column of block g (block scale byte
    # 125 = 2^-2, code 6 = 4.0); the key holds code c with scale byte b in that column:
    # logit = 4 * 2^-2 * E2M1(c) * 2^(b - 127), ReLU'd.
    heads = 16
    for g, col, c, b in [(0, 3, 6, 127), (1, 40, 5, 130), (3, 127, 13, 127), (2, 64, 2, 100)]:
        q = np.zeros((1, heads, 128), np.float32)
        q[0, 0, col] = 1.0
        qrows, _ = oracle.quantize_queries(bf16_bits(q), None, "mxfp4")
        assert qrows[0, heads * 64 + g] == 125 and npdecode.unpack_nibbles(qrows[0, :64])[col] == 6
        cache = np.zeros(4352, np.uint8)
        token = 5
        nib = np.zeros(128, np.uint8)
        nib[col] = c
        cache[token * 64: token * 64 + 64] = nib[0::2] | (nib[1::2] << 4)
        cache[4096 + token * 4: 4096 + token * 4 + 4] = 127
        cache[4096 + token * 4 + g] = b
        w = np.zeros((1, heads), np.float32)
        w[0, 0] = 1.0
        lg = oracle.score_paged(qrows, heads, _bf16w(w), cache, 1, 4352, np.array([[0]], np.int32),
                                np.array([0, 1], np.int32), np.array([64], np.int32))
        val = 4 * 2.0 ** -2 * E2M1_GRID[c] * 2.0 ** (b - 127)
        assert lg[0, token] == np.float32(max(val, 0.0)), (g, col, c, b)
        assert np.all(lg[0, :64][np.arange(64) != token] == 0)


def _brute_force(wl, qrows, w_bits, cache, starts, ends):
    """FP64 sum_h w * relu(q_h . k) from the NumPy field decoders (no oracle code)."""
    H = wl.heads
    if wl.fmt == "mxfp4":
        qv = npdecode.mxfp4_query_rows(qrows, H)
    else:
        qv = npdecode.fp8_query_rows(qrows, H)
    w = bf16_to_f32(w_bits).astype(np.float64)
    out = np.full((wl.num_rows, wl.width), np.nan)
    for q in range(wl.num_requests):
        for r in range(starts[q], starts[q + 1]):
            n = min(ends[r], wl.width)
            keys = np.zeros((n, 128))
            for p in range(n):
                page = wl.block_table[q, p // 64]
                if wl.fmt == "mxfp4":
                    keys[p] = npdecode.mxfp4_key(cache, page, p % 64, wl.page_stride, wl.section_offset)
                elif wl.fmt == "fp8_mx":
                    keys[p] = npdecode.fp8_mx_key(cache, page, p % 64, wl.page_stride, wl.section_offset)[0]
                else:
                    keys[p] = npdecode.fp8_key(cache, page, p % 64, wl.page_stride, wl.section_offset)[0]
            dots = qv[r] @ keys.T  # [H, n]
            out[r, :n] = (w[r][:, None] * np.maximum(dots, 0.0)).sum(0)
    return out


@pytest.mark.parametrize("fmt,heads,stride,offset", [("mxfp4", 32, 4352, 0), ("mxfp4", 16, 8192, 3840),
                                                     ("mxfp4", 64, 4352, 0), ("fp8", 32, 8448, 0),
                                                     ("fp8_mx", 32, 9216, 512)])
def test_score_matches_fp64_brute_force(fmt, heads, stride, offset):
    wl = make_workload("tiny", fmt=fmt, heads=heads, seq_lens=[70, 200, 3], query_lens=[1, 3, 2],
                       num_rows=8, topk=8, seed=heads, page_stride=stride, section_offset=offset,
                       extra_pages=2)
    cache = np.full(wl.cache_bytes, 0xA5, np.uint8)
    oracle.store_keys(wl.key_bits, wl.gamma, wl.beta, wl.eps, wl.key_slots, cache, wl.num_pages,
                      wl.page_stride, wl.section_offset, fmt)
    qrows, w_out = oracle.quantize_queries(wl.q_bits, wl.wv_bits, fmt)
    starts, ends = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
    lg = oracle.score_paged(qrows, heads, w_out, cache, wl.num_pages, wl.page_stride, wl.block_table,
                            starts, ends, fmt, wl.section_offset)
    ref = _brute_force(wl, qrows, w_out, cache, starts, ends)
    valid = ~np.isnan(ref)
    assert np.array_equal(np.isnan(lg), ~valid)
    assert valid.sum() == sum(ends)
    # the oracle rounds the exact FP64 value once to FP32; numpy's summation order may differ by
    # a few FP64 ulps, which can move the FP32 result by at most one ulp at a tie
    got, want = lg[valid].astype(np.float64), ref[valid].astype(np.float32).astype(np.float64)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp)
    # ReLU actually clips: some head dots are negative in this workload
    assert (lg[valid] > 0).any() and (lg[valid] < 0).any()


def test_score_fp8_mx_equals_fp8():
    # the key scale is a power of two either way: storing it as UE8M0 bytes changes no logit
    wls = {f: make_workload("mx", fmt=f, heads=32, seq_lens=[300, 65], query_lens=[2, 1], topk=8,
                            seed=12, outlier_frac=0.01, outlier_gain=20.0) for f in ("fp8", "fp8_mx")}
    out = {}
    for f, wl in wls.items():
        cache = np.full(wl.cache_bytes, 0xA5, np.uint8)
        oracle.store_keys(wl.key_bits, wl.gamma, wl.beta, wl.eps, wl.key_slots, cache,
                          wl.num_pages, wl.page_stride, 0, f)
        qrows, w_out = oracle.quantize_queries(wl.q_bits, wl.wv_bits, f)
        starts, ends = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
        out[f] = oracle.score_paged(qrows, 32, w_out, cache, wl.num_pages, wl.page_stride,
                                    wl.block_table, starts, ends, f, 0)
    assert np.array_equal(out["fp8"], out["fp8_mx"], equal_nan=True)


def test_score_invariant_to_page_placement():
    base = dict(fmt="mxfp4", heads=32, seq_lens=[130, 64], query_lens=[2, 1], topk=8, seed=21)
    res = []
    for permute, stride, offset in [(False, 4352, 0), (True, 4352, 0), (True, 8192, 3840)]:
        wl = make_workload("p", permute_pages=permute, page_stride=stride, section_offset=offset,
                           extra_pages=1, **base)
        cache = np.zeros(wl.cache_bytes, np.uint8)
        oracle.store_keys(wl.key_bits, wl.gamma, wl.beta, wl.eps, wl.key_slots, cache, wl.num_pages,
                          wl.page_stride, wl.section_offset)
        qrows, w_out = oracle.quantize_queries(wl.q_bits, wl.wv_bits)
        starts, ends = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
        res.append(oracle.score_paged(qrows, 32, w_out, cache, wl.num_pages, wl.page_stride,
                                      wl.block_table, starts, ends, "mxfp4", wl.section_offset))
    assert np.array_equal(res[0], res[1], equal_nan=True)
    assert np.array_equal(res[0], res[2], equal_nan=True)
