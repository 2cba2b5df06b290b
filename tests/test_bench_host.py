"""Host-side logic of bench.py (no GPU): the one-GPU guard, the step's packed projection rows,
and the HBM byte counters read from a committed rocprofv3 summary only while the scorer
sources they were taken on are unchanged."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_attention_indexer_quant_amd.workloads import config  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_packed_rows_hold_the_step_keys_and_weights():
    wl = config("tiny_mxfp4")
    proj, slots = bench.packed_rows(wl)
    sk = wl.step_key_index()
    assert proj.shape == (wl.num_rows, 128 + wl.heads)
    assert np.array_equal(proj[:sk.size, :128], wl.key_bits[sk])
    assert np.array_equal(proj[:, 128:], wl.wv_bits)
    assert np.array_equal(slots[:sk.size], wl.key_slots[sk])
    assert np.all(slots[sk.size:] == -1)


def test_traffic_only_for_the_profiled_sources(tmp_path, monkeypatch):
    text = open(bench.PROFILE_PMC.format(kernel="index_score_hist", workload="long_mxfp4")).read()
    got = bench.measured_traffic("index_score_hist", "long_mxfp4")
    vals = dict(l.split(" = ", 1) for l in text.splitlines() if " = " in l and not l.startswith("#"))
    if vals["scorer_sources_sha256_16"] == bench.scorer_source_hash():
        assert got == float(vals["hbm_bytes_per_launch"])
    else:
        assert got is None
    # a summary taken on other sources gives no traffic
    stale = text.replace(vals["scorer_sources_sha256_16"], "0" * 16)
    (tmp_path / "index_score_hist_long_mxfp4_pmc.txt").write_text(stale)
    monkeypatch.setattr(bench, "PROFILE_PMC", str(tmp_path / "{kernel}_{workload}_pmc.txt"))
    assert bench.measured_traffic("index_score_hist", "long_mxfp4") is None


def test_histogram_bytes_count_the_coarse_bins_reached():
    # order keys: 1.0 -> coarse 47, 2.0 -> 48, -1.0 -> 16, -0.0 and 0.0 -> 32
    lg = np.array([[1.0, 2.0, -1.0, -0.0, 0.0, 7.0, 7.0, 7.0]], np.float32)
    assert bench.histogram_bytes(lg, np.array([5]), 8, 8) == 128 + 4 * 128
    assert bench.histogram_bytes(lg, np.array([5]), 2, 8) == (128 + 256) * 2 + (128 + 128)
    assert bench.histogram_bytes(lg, np.array([0]), 2, 8) == 0
    # bound clamped to the width; 7.0 shares coarse bin 48 with 2.0
    assert bench.histogram_bytes(lg, np.array([99]), 8, 8) == 128 + 4 * 128


def test_prepared_call_converts_arguments_once():
    # the bench's pre-marshalled calls: arguments converted to their C types when prepared,
    # a nonzero status raised (here the step call's own check of k, before any launch)
    import ctypes
    import pytest
    import sparse_attention_indexer_quant_amd as dsa
    if not os.path.exists(dsa.LIBRARY):
        pytest.skip("libdsaidx.so not built")
    lib = dsa.library()
    P = 0x10000
    args = [0, P, 256, 0, 128, P, 32, 4096, 128, P, P, ctypes.c_float(1e-6), P, P, 1, 1, 1, P, 8,
            4352, P, 4, P, P, P, 256, 0, P, 64, P, 1 << 20, None]
    call = bench.Prepared(lib.dsaidx_index_score_topk, *args)
    assert all(a is None or isinstance(a, ctypes._SimpleCData) for a in call.args)
    assert isinstance(call.args[11], ctypes.c_float) and call.args[11].value == np.float32(1e-6)
    assert call.args[26].value == 0  # k, as c_int32
    with pytest.raises(RuntimeError, match="status 1"):
        call()
    with pytest.raises(AssertionError):
        bench.Prepared(lib.dsaidx_index_score_topk, *args[:-1])
