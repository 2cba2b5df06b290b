"""The C-ABI library on the host: it loads, exports every entry point include/dsaidx.h
declares, and every argument check fails before anything is enqueued (no GPU needed; the
pointers passed here are never dereferenced because each call returns at its check)."""
import ctypes
import os
import re

import pytest
import torch

import sparse_attention_indexer_quant_amd as dsa
from goldens import rows

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsaidx.h")

OK, EINVAL, ELAYOUT, EUNSUP, ESCRATCH = 0, 1, 2, 3, 5
P = 0x10000  # a 64 KiB-aligned stand-in pointer: every check below fails before any use
MX, FP8 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIBRARY):
        pytest.skip("libdsaidx.so not built (run __graft_entry__.build())")
    return dsa.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsaidx_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dsaidx_quantize_queries", "dsaidx_store_keys", "dsaidx_score_paged", "dsaidx_topk",
              "dsaidx_decode_layout", "dsaidx_topk_workspace_bytes", "dsaidx_status_string",
              "dsaidx_query_row_bytes", "dsaidx_index_inputs", "dsaidx_score_paged_hist",
              "dsaidx_topk_scored", "dsaidx_score_topk_workspace_bytes", "dsaidx_dcp_candidates",
              "dsaidx_dcp_merge", "dsaidx_index_inputs_layout", "dsaidx_score_segment_keys",
              "dsaidx_read_sections", "dsaidx_read_sections_words", "dsaidx_read_stream",
              "dsaidx_topk_noalloc", "dsaidx_decode_tile_size", "dsaidx_score_topk_tiled",
              "dsaidx_score_topk_tiled_workspace_bytes", "dsaidx_index_score_hist",
              "dsaidx_index_score_topk"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(dsa.LIBRARY)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings_and_row_bytes(lib):
    assert lib.dsaidx_status_string(0) == b"ok"
    assert lib.dsaidx_status_string(99) == b"unknown status"
    assert lib.dsaidx_query_row_bytes(MX, 32) == 2176
    assert lib.dsaidx_query_row_bytes(MX, 64) == 4352
    assert lib.dsaidx_query_row_bytes(FP8, 32) == 4096
    assert lib.dsaidx_query_row_bytes(MX, 48) == 0
    assert lib.dsaidx_query_row_bytes(7, 32) == 0


def quant(lib, **kw):
    a = dict(fmt=MX, q=P, rows=4, heads=32, rs=32 * 128, hs=128, wv=P, wvs=32, out=P, outs=2176,
             wo=P, wos=32)
    a.update(kw)
    return lib.dsaidx_quantize_queries(a["fmt"], a["q"], a["rows"], a["heads"], a["rs"], a["hs"],
                                       a["wv"], a["wvs"], a["out"], a["outs"], a["wo"], a["wos"], None)


def test_quantize_queries_checks(lib):
    assert quant(lib, fmt=5) == EINVAL
    assert quant(lib, rows=-1) == EINVAL
    assert quant(lib, heads=48) == EUNSUP            # fp4_indexer quantize_queries: 16, 32 or 64
    assert quant(lib, rows=0, q=None, out=None) == OK  # empty: nothing enqueued
    assert quant(lib, q=None) == EINVAL
    assert quant(lib, wo=None) == EINVAL             # weights without an output
    assert quant(lib, hs=64) == ELAYOUT              # heads overlap
    assert quant(lib, rs=31 * 128) == ELAYOUT        # rows overlap
    assert quant(lib, q=P + 2) == ELAYOUT            # 16-byte loads
    assert quant(lib, hs=132, rs=32 * 132) == ELAYOUT
    assert quant(lib, outs=2160) == ELAYOUT          # stride below the row size
    assert quant(lib, outs=2184) == ELAYOUT          # stride not a multiple of 16
    assert quant(lib, fmt=FP8, outs=2176) == ELAYOUT  # FP8 rows are 4096 B
    assert quant(lib, wvs=16) == ELAYOUT


def store(lib, **kw):
    a = dict(fmt=MX, keys=P, t=8, ks=128, g=P, b=P, eps=1e-6, slots=P, cache=P, pages=4, ps=4352)
    a.update(kw)
    return lib.dsaidx_store_keys(a["fmt"], a["keys"], a["t"], a["ks"], a["g"], a["b"], a["eps"],
                                 a["slots"], a["cache"], a["pages"], a["ps"], None)


def test_store_keys_checks(lib):
    assert store(lib, fmt=-1) == EINVAL
    assert store(lib, t=-2) == EINVAL
    assert store(lib, eps=float("nan")) == EINVAL
    assert store(lib, eps=-1.0) == EINVAL
    assert store(lib, t=0, keys=None) == OK
    assert store(lib, slots=None) == EINVAL
    assert store(lib, ks=127) == ELAYOUT            # contiguous 128-element rows
    assert store(lib, ks=129) == ELAYOUT
    assert store(lib, ps=4351) == ELAYOUT           # cache_views: stride >= 4352
    assert store(lib, ps=4360) == ELAYOUT           # 16-byte aligned sections
    assert store(lib, fmt=FP8, ps=4352) == ELAYOUT  # FP8 sections are 8448 B
    assert store(lib, fmt=2, ps=4352) == ELAYOUT    # so are FP8 sections with UE8M0 scales
    assert store(lib, fmt=3) == EINVAL
    assert store(lib, cache=P + 8) == ELAYOUT
    assert store(lib, g=P + 4) == ELAYOUT


def inputs(lib, **kw):
    a = dict(fmt=MX, proj=P, t=4, ps=4352, kc=4096, wc=4224, q=P, h=32, qs=4096, qh=128, g=P,
             b=P, eps=1e-6, slots=P, cache=P, pages=4, cs=4352, qo=P, qos=2176, wo=P, wos=32)
    a.update(kw)
    return lib.dsaidx_index_inputs(a["fmt"], a["proj"], a["t"], a["ps"], a["kc"], a["wc"], a["q"],
                                   a["h"], a["qs"], a["qh"], a["g"], a["b"], a["eps"], a["slots"],
                                   a["cache"], a["pages"], a["cs"], a["qo"], a["qos"], a["wo"],
                                   a["wos"], None)


def test_index_inputs_checks(lib):
    assert inputs(lib, fmt=3) == EINVAL
    assert inputs(lib, t=-1) == EINVAL
    assert inputs(lib, kc=-2) == EINVAL
    assert inputs(lib, wc=-1) == EINVAL
    assert inputs(lib, eps=float("inf")) == EINVAL
    assert inputs(lib, h=48) == EUNSUP
    assert inputs(lib, t=0, proj=None, q=None) == OK
    assert inputs(lib, wo=None) == EINVAL               # head weights are always written
    assert inputs(lib, slots=None) == EINVAL
    assert inputs(lib, ps=4223) == ELAYOUT              # key columns outside the row
    assert inputs(lib, ps=4240) == ELAYOUT              # weight columns outside the row
    assert inputs(lib, kc=4095) == ELAYOUT              # key read as column pairs
    assert inputs(lib, ps=4353) == ELAYOUT
    assert inputs(lib, proj=P + 2) == ELAYOUT
    assert inputs(lib, qh=127) == ELAYOUT               # contiguous 128-element heads
    assert inputs(lib, q=P + 8) == ELAYOUT
    assert inputs(lib, qos=2175) == ELAYOUT
    assert inputs(lib, cs=4351) == ELAYOUT              # cache_views: stride >= 4352
    assert inputs(lib, fmt=FP8, qos=4096, cs=4352) == ELAYOUT


def layout(lib, **kw):
    a = dict(seq=P, ql=P, r=4, rows=8, rank=0, world=1, il=1, starts=P, ends=P)
    a.update(kw)
    return lib.dsaidx_decode_layout(a["seq"], a["ql"], a["r"], a["rows"], a["rank"], a["world"],
                                    a["il"], a["starts"], a["ends"], None)


def test_decode_layout_checks(lib):
    # fp4_indexer decode_layout: invalid DCP geometry or query row count
    assert layout(lib, rank=1, world=1) == EINVAL
    assert layout(lib, rank=-1) == EINVAL
    assert layout(lib, il=0) == EINVAL
    assert layout(lib, rows=-1) == EINVAL
    assert layout(lib, r=-1) == EINVAL
    assert layout(lib, starts=None) == EINVAL
    assert layout(lib, ends=None) == EINVAL
    assert layout(lib, seq=None) == EINVAL
    assert layout(lib, starts=P + 2) == ELAYOUT


def score(lib, **kw):
    a = dict(fmt=MX, q=P, qs=2176, heads=32, w=P, ws=32, cache=P, pages=8, ps=4352, bt=P, r=2,
             mb=4, starts=P, ends=P, rows=2, mql=1, out=P, os=256)
    a.update(kw)
    return lib.dsaidx_score_paged(a["fmt"], a["q"], a["qs"], a["heads"], a["w"], a["ws"], a["cache"],
                                  a["pages"], a["ps"], a["bt"], a["r"], a["mb"], a["starts"],
                                  a["ends"], a["rows"], a["mql"], a["out"], a["os"], None)


def test_score_paged_checks(lib):
    assert score(lib, fmt=3) == EINVAL
    assert score(lib, rows=-1) == EINVAL
    assert score(lib, heads=8) == EUNSUP
    assert score(lib, mql=0) == EUNSUP
    assert score(lib, mql=17) == EUNSUP
    assert score(lib, rows=0, q=None) == OK          # fp4_indexer score_paged: empty output
    assert score(lib, r=0, q=None) == OK
    assert score(lib, mb=0, q=None) == OK
    assert score(lib, bt=None) == EINVAL
    assert score(lib, qs=2160) == ELAYOUT
    assert score(lib, q=P + 4) == ELAYOUT
    assert score(lib, ws=30) == ELAYOUT
    assert score(lib, ps=4000) == ELAYOUT
    assert score(lib, fmt=FP8, qs=4096, ps=4352) == ELAYOUT
    assert score(lib, os=255) == ELAYOUT


def topk(lib, **kw):
    a = dict(lg=P, rows=2, width=256, ls=256, ends=P, k=16, out=P, os=16, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.dsaidx_topk(a["lg"], a["rows"], a["width"], a["ls"], a["ends"], a["k"], a["out"],
                           a["os"], a["ws"], a["wsb"], None)


def test_topk_checks(lib):
    assert topk(lib, k=0) == EINVAL
    assert topk(lib, rows=-1) == EINVAL
    assert topk(lib, width=-1) == EINVAL
    assert topk(lib, rows=0, lg=None) == OK
    assert topk(lib, ends=None) == EINVAL
    assert topk(lib, ls=255) == ELAYOUT
    assert topk(lib, os=15) == ELAYOUT
    assert topk(lib, lg=P + 2) == ELAYOUT
    assert lib.dsaidx_topk_workspace_bytes(4, 1024, 0) == 0
    # rows hold at most 2^25 keys
    assert topk(lib, width=(1 << 25) + 1, ls=(1 << 25) + 1) == EUNSUP
    assert lib.dsaidx_topk_workspace_bytes(1, (1 << 25) + 1, 8) == 0
    assert lib.dsaidx_topk_workspace_bytes(1, 1 << 25, 8) > 0


def topk_noalloc(lib, **kw):
    a = dict(lg=P, rows=2, width=256, ls=256, ends=P, k=16, out=P, os=16)
    a.update(kw)
    return lib.dsaidx_topk_noalloc(a["lg"], a["rows"], a["width"], a["ls"], a["ends"], a["k"],
                                   a["out"], a["os"], None)


def test_topk_noalloc_checks(lib):
    # the same checks as topk, and sizes beyond the static scratch rejected before any HIP call
    assert topk_noalloc(lib, k=0) == EINVAL
    assert topk_noalloc(lib, rows=-1) == EINVAL
    assert topk_noalloc(lib, rows=0, lg=None) == OK
    assert topk_noalloc(lib, ends=None) == EINVAL
    assert topk_noalloc(lib, ls=255) == ELAYOUT
    assert topk_noalloc(lib, os=15) == ELAYOUT
    assert topk_noalloc(lib, width=(1 << 25) + 1, ls=(1 << 25) + 1) == EUNSUP
    limit = 64 << 20
    assert lib.dsaidx_topk_workspace_bytes(512, 65536, 2048) <= limit     # the verify workload fits
    assert lib.dsaidx_topk_workspace_bytes(2048, 65536, 2048) > limit
    assert topk_noalloc(lib, rows=2048, width=65536, ls=65536, k=2048, os=2048) == ESCRATCH
    assert lib.dsaidx_status_string(ESCRATCH) != lib.dsaidx_status_string(99)


def score_hist(lib, **kw):
    a = dict(fmt=MX, q=P, qs=2176, h=32, w=P, ws=32, cache=P, pages=8, ps=4352, bt=P, r=2, mb=4,
             starts=P, ends=P, rows=2, mq=1, lg=P, ls=256, wk=P, wkb=1 << 30)
    a.update(kw)
    return lib.dsaidx_score_paged_hist(a["fmt"], a["q"], a["qs"], a["h"], a["w"], a["ws"],
                                       a["cache"], a["pages"], a["ps"], a["bt"], a["r"], a["mb"],
                                       a["starts"], a["ends"], a["rows"], a["mq"], a["lg"],
                                       a["ls"], a["wk"], a["wkb"], None)


def test_score_paged_hist_checks(lib):
    assert score_hist(lib, fmt=3) == EINVAL
    assert score_hist(lib, h=20) == EUNSUP
    assert score_hist(lib, mq=17) == EUNSUP
    assert score_hist(lib, rows=0, q=None) == OK
    assert score_hist(lib, wk=None) == EINVAL
    assert score_hist(lib, wkb=16) == EINVAL
    assert score_hist(lib, wk=P + 16) == ELAYOUT
    assert score_hist(lib, ls=255) == ELAYOUT
    assert score_hist(lib, ps=4350) == ELAYOUT
    assert lib.dsaidx_score_topk_workspace_bytes(0, 4, 2) == 0
    assert lib.dsaidx_score_topk_workspace_bytes(2, 4, 2) > 0
    # more than 1024 scoring workgroups per row (> 4M keys) is refused
    assert lib.dsaidx_score_topk_workspace_bytes(1, 70000, 1) == 0
    assert score_hist(lib, r=1, mb=70000, ls=70000 * 64) == EUNSUP
    # segment = one scoring workgroup: 4 wavefronts x pages per wavefront x 64 keys, pages per
    # wavefront 1..16 (a multiple of 4 above 4) sized for one wavefront per SIMD (256 compute
    # units assumed where no GPU is visible)
    lib.dsaidx_score_segment_keys.restype = ctypes.c_int64
    assert lib.dsaidx_score_segment_keys(0, 4) == 0
    assert lib.dsaidx_score_segment_keys(2, 4) == 4 * 1 * 64
    if not torch.cuda.is_available():
        assert lib.dsaidx_score_segment_keys(8, 2048) == 4 * 16 * 64
        assert lib.dsaidx_score_segment_keys(16, 128) == 4 * 2 * 64
        assert lib.dsaidx_score_segment_keys(24, 128) == 4 * 3 * 64
        assert lib.dsaidx_score_segment_keys(40, 128) == 4 * 8 * 64
        assert lib.dsaidx_score_segment_keys(64, 128) == 4 * 8 * 64


def read_sections(lib, **kw):
    a = dict(fmt=MX, cache=P, np_=8, ps=4352, bt=P, r=2, mb=4, seq=P, out=P, ow=1 << 20)
    a.update(kw)
    return lib.dsaidx_read_sections(a["fmt"], a["cache"], a["np_"], a["ps"], a["bt"], a["r"],
                                    a["mb"], a["seq"], a["out"], a["ow"], None)


def test_decode_tile_size_matches_golden(lib):
    # a host function of the library: the hand-worked values of tests/golden/decode_tile_size.txt
    for line in rows("decode_tile_size.txt"):
        mml, width, topk, heads, want = (int(v) for v in line.split())
        assert lib.dsaidx_decode_tile_size(mml, width, topk, heads) == want, line
    assert lib.dsaidx_decode_tile_size(-1, 64, 8, 32) == 0
    assert lib.dsaidx_decode_tile_size(64, 64, 0, 32) == 0
    assert lib.dsaidx_decode_tile_size(64, 64, 8, 0) == 0


def tiled(lib, **kw):
    a = dict(fmt=0, q=P, qs=2176, h=32, w=P, ws_=32, cache=P, np_=10, ps=4352, bt=P, r=2, mb=4,
             st=P, ends=P, rows=8, mql=4, k=16, out=P, os=16, tile=4, lt=P, lts=256, wsp=P,
             wsb=1 << 30)
    a.update(kw)
    return lib.dsaidx_score_topk_tiled(a["fmt"], a["q"], a["qs"], a["h"], a["w"], a["ws_"],
                                       a["cache"], a["np_"], a["ps"], a["bt"], a["r"], a["mb"],
                                       a["st"], a["ends"], a["rows"], a["mql"], a["k"], a["out"],
                                       a["os"], a["tile"], a["lt"], a["lts"], a["wsp"], a["wsb"],
                                       None)


def test_score_topk_tiled_checks(lib):
    assert tiled(lib, tile=0) == EINVAL
    assert tiled(lib, k=0) == EINVAL
    assert tiled(lib, fmt=7) == EINVAL
    assert tiled(lib, h=24) == EUNSUP
    assert tiled(lib, mql=17) == EUNSUP
    assert tiled(lib, rows=0, q=None) == OK
    assert tiled(lib, r=0) == EINVAL            # rows to select for, nothing to score with
    assert tiled(lib, lt=None) == EINVAL
    assert tiled(lib, wsp=None) == EINVAL
    assert tiled(lib, wsb=16) == EINVAL
    assert tiled(lib, lts=255) == ELAYOUT       # a tile row narrower than max_blocks * 64
    assert tiled(lib, os=15) == ELAYOUT
    assert tiled(lib, ps=4096) == ELAYOUT
    assert tiled(lib, wsp=P + 16) == ELAYOUT
    # the workspace holds one tile: it grows with tile_rows, not with the rows
    one = lib.dsaidx_score_topk_tiled_workspace_bytes(128, 1024, 32, 4)
    assert 0 < one < lib.dsaidx_score_topk_tiled_workspace_bytes(128, 1024, 64, 4)
    assert lib.dsaidx_score_topk_tiled_workspace_bytes(128, 1024, 0, 4) == 0
    assert lib.dsaidx_score_topk_tiled_workspace_bytes(128, 1024, 32, 0) == 0


def test_read_stream_checks(lib):
    buf, out = 1 << 12, 1 << 16  # host-side stand-ins: every call below fails its checks first
    f = lib.dsaidx_read_stream
    assert f(buf, 17, 4, out, 16, None) == EINVAL          # not a multiple of 16
    assert f(buf, -16, 4, out, 16, None) == EINVAL
    assert f(buf, 64, 0, out, 16, None) == EINVAL          # no workgroups
    assert f(buf, 64, (1 << 20) + 1, out, 1 << 23, None) == EINVAL
    assert f(buf, 64, 4, out, 15, None) == EINVAL          # out shorter than 4 per workgroup
    assert f(None, 64, 4, out, 16, None) == EINVAL
    assert f(buf + 8, 64, 4, out, 16, None) == EINVAL      # unaligned
    assert f(buf, 0, 4, out, 16, None) == OK               # nothing to read: nothing enqueued


def test_read_sections_checks(lib):
    assert read_sections(lib, fmt=5) == EINVAL
    assert read_sections(lib, r=-1) == EINVAL
    assert read_sections(lib, ow=-1) == EINVAL
    assert read_sections(lib, r=0, cache=None) == OK
    assert read_sections(lib, np_=0, cache=None) == OK
    assert read_sections(lib, seq=None) == EINVAL
    assert read_sections(lib, ps=4350) == ELAYOUT
    assert read_sections(lib, fmt=FP8, ps=4352) == ELAYOUT
    assert read_sections(lib, cache=P + 8) == ELAYOUT
    assert read_sections(lib, out=P + 2) == ELAYOUT
    assert read_sections(lib, ow=1) == EINVAL  # shorter than one word per wavefront
    # one word per wavefront of the scorer's grid: 4 per workgroup, chunks x requests workgroups
    assert lib.dsaidx_read_sections_words(0, 4) == 0
    assert lib.dsaidx_read_sections_words(2, 4) == 4 * 2 * 1
    if not torch.cuda.is_available():
        assert lib.dsaidx_read_sections_words(8, 2048) == 4 * 8 * 32


def topk_scored(lib, **kw):
    a = dict(lg=P, rows=2, ls=256, ends=P, k=8, out=P, os=8, r=2, mb=4, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.dsaidx_topk_scored(a["lg"], a["rows"], a["ls"], a["ends"], a["k"], a["out"],
                                  a["os"], a["r"], a["mb"], a["ws"], a["wsb"], None)


def test_topk_scored_checks(lib):
    assert topk_scored(lib, k=0) == EINVAL
    assert topk_scored(lib, rows=-1) == EINVAL
    assert topk_scored(lib, rows=0, lg=None) == OK
    assert topk_scored(lib, r=0) == EINVAL
    assert topk_scored(lib, ws=None) == EINVAL
    assert topk_scored(lib, wsb=8) == EINVAL
    assert topk_scored(lib, ls=255) == ELAYOUT
    assert topk_scored(lib, os=7) == ELAYOUT
    assert topk_scored(lib, ws=P + 8) == ELAYOUT


def index_step(lib, call, **kw):
    """dsaidx_index_score_hist (call "hist") or dsaidx_index_score_topk (call "topk")."""
    a = dict(fmt=MX, proj=P, ps_=256, kc=0, wc=128, q=P, h=32, qs=32 * 128, qh=128, g=P, b=P,
             eps=1e-6, seq=P, ql=P, r=2, rows=2, mq=1, cache=P, pages=8, ps=4352, bt=P, mb=4,
             starts=P, ends=P, lg=P, ls=256, k=8, idx=P, istr=8, wk=P, wkb=1 << 30)
    a.update(kw)
    head = [a["fmt"], a["proj"], a["ps_"], a["kc"], a["wc"], a["q"], a["h"], a["qs"], a["qh"],
            a["g"], a["b"], ctypes.c_float(a["eps"]), a["seq"], a["ql"], a["r"], a["rows"], a["mq"],
            a["cache"], a["pages"], a["ps"], a["bt"], a["mb"], a["starts"], a["ends"], a["lg"],
            a["ls"]]
    if call == "hist":
        return lib.dsaidx_index_score_hist(*head, a["wk"], a["wkb"], None)
    return lib.dsaidx_index_score_topk(*head, a["k"], a["idx"], a["istr"], a["wk"], a["wkb"], None)


@pytest.mark.parametrize("call", ["hist", "topk"])
def test_index_step_checks(lib, call):
    # the checks both step calls share (every case returns before any launch)
    assert index_step(lib, call, fmt=3) == EINVAL
    assert index_step(lib, call, eps=-1.0) == EINVAL
    assert index_step(lib, call, h=20) == EUNSUP
    assert index_step(lib, call, mq=5) == EUNSUP
    assert index_step(lib, call, fmt=FP8, mq=3) == EUNSUP
    assert index_step(lib, call, starts=None) == EINVAL
    assert index_step(lib, call, proj=None) == EINVAL
    assert index_step(lib, call, ps_=130) == ELAYOUT  # the key's 128 columns do not fit
    assert index_step(lib, call, q=P + 8) == ELAYOUT
    assert index_step(lib, call, ps=4350) == ELAYOUT
    assert index_step(lib, call, ls=255) == ELAYOUT
    assert index_step(lib, call, wk=None) == EINVAL
    assert index_step(lib, call, wkb=16) == EINVAL
    assert index_step(lib, call, wk=P + 16) == ELAYOUT


def test_index_score_topk_checks(lib):
    # the selection's own checks
    assert index_step(lib, "topk", k=0) == EINVAL
    assert index_step(lib, "topk", k=0, rows=0) == EINVAL
    assert index_step(lib, "topk", idx=None) == EINVAL
    assert index_step(lib, "topk", istr=7) == ELAYOUT
    assert index_step(lib, "topk", idx=P + 2) == ELAYOUT


def cand(lib, **kw):
    a = dict(lg=P, rows=4, width=1000, ls=1000, idx=P, k=64, istr=64, rank=1, world=4, il=64,
             v=P, p=P)
    a.update(kw)
    return lib.dsaidx_dcp_candidates(a["lg"], a["rows"], a["width"], a["ls"], a["idx"], a["k"],
                                     a["istr"], a["rank"], a["world"], a["il"], a["v"], a["p"], None)


def merge(lib, **kw):
    a = dict(v=P, p=P, world=4, rows=4, kc=64, k=64, out=P, os=64, rank=0, il=64, loc=None, lstr=0)
    a.update(kw)
    return lib.dsaidx_dcp_merge(a["v"], a["p"], a["world"], a["rows"], a["kc"], a["k"], a["out"],
                                a["os"], a["rank"], a["il"], a["loc"], a["lstr"], None)


def test_dcp_checks(lib):
    assert cand(lib, k=0) == EINVAL
    assert cand(lib, rank=4) == EINVAL
    assert cand(lib, rank=-1) == EINVAL
    assert cand(lib, il=0) == EINVAL
    assert cand(lib, rows=0, lg=None) == OK
    assert cand(lib, width=1 << 30, ls=1 << 30) == EUNSUP   # global positions past INT32_MAX
    assert cand(lib, istr=63) == ELAYOUT
    assert cand(lib, v=P + 2) == ELAYOUT
    assert merge(lib, kc=0) == EINVAL
    assert merge(lib, k=0) == EINVAL
    assert merge(lib, loc=P, lstr=64, rank=4) == EINVAL
    assert merge(lib, world=8, kc=4096) == EUNSUP           # 32768 candidates per row
    assert merge(lib, rows=0, v=None) == OK
    assert merge(lib, out=None) == EINVAL
    assert merge(lib, os=63) == ELAYOUT
    assert merge(lib, loc=P, lstr=10) == ELAYOUT


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        dsa.quantize_queries(torch.zeros((1, 32, 128), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        dsa.topk(torch.zeros((1, 8)), torch.zeros(1, dtype=torch.int32), 2)


def test_build_reads_kernel_resource_remarks():
    # the build rejects kernels that spill to scratch; its parser of hipcc's remarks
    from sparse_attention_indexer_quant_amd import build as b
    text = "\n".join([
        "a.hip:9:1: remark: Function Name: k1 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs: 27 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:20:1: remark: Function Name: k2 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:20:1: remark:     ScratchSize [bytes/lane]: 64 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:20:1: warning: unrelated",
    ])
    res = b.kernel_resources(text)
    assert res["k1"]["VGPRs"] == "27"
    assert res["k1"]["ScratchSize [bytes/lane]"] == "0"
    assert res["k2"]["ScratchSize [bytes/lane]"] == "64"
