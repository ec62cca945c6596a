"""bench.py's host side on the CPU: it refuses more than one GPU, and it reports
HBM traffic from a committed rocprofv3 summary only while that summary was
taken of the current kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rank_gemm_page_amd.profiling import kernel_source_hash  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], cwd=ROOT,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=300)
    assert r.returncode == 3, r.stderr
    assert "one GPU only" in r.stderr and r.stdout == ""


def write_traffic(root, source_hash):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    rec = {"kernel_source_hash": source_hash,
           "kernels": {"fused_kernel": {"fetch_bytes": 1000, "write_bytes": 24, "trace_avg_us": 20.5},
                       "scatter_pages_kernel": {"fetch_bytes": 7, "write_bytes": 7, "trace_avg_us": 4.0}}}
    with open(os.path.join(root, "profiles", "traffic_decode7b.json"), "w") as f:
        json.dump(rec, f)


def test_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("decode7b", "fused_kernel") == (None, None)        # no summary
    write_traffic(str(tmp_path), kernel_source_hash("fused"))
    assert bench.load_traffic("decode7b", "fused_kernel") == (1024, 20.5)        # that kernel only
    assert bench.load_traffic("decode7b", "expand_kernel") == (None, None)
    write_traffic(str(tmp_path), "0" * 16)                                        # other sources
    assert bench.load_traffic("decode7b", "fused_kernel") == (None, None)


def test_committed_profiles_match_the_sources():
    """The summaries under profiles/ were taken of the kernels as committed."""
    for cfg in ("decode7b", "prefill7b", "mixed13b", "mlp70b"):
        b, us = bench.load_traffic(cfg, "fused_kernel")
        assert b is not None and us is not None, cfg
    for cfg in ("decode7b", "prefill7b", "mixed13b", "mlp70b"):
        b, us = bench.load_traffic(cfg, "forward_kernel", kind="forward")
        assert b is not None and us is not None, cfg


@pytest.mark.parametrize("pad", [16, 32, 64, 128])
def test_rank_padding_keeps_the_batch(pad):
    """bench.py --rank-pad: ranks rounded up to a multiple of pad (at most 256),
    the tokens, their adapters, x and y unchanged."""
    import numpy as np

    w0, w1 = bench.workload("decode7b", 0), bench.workload("decode7b", 0, pad)
    assert np.array_equal(w0.ids, w1.ids)
    assert all(np.array_equal(a, b) for a, b in zip(w0.x, w1.x))
    assert all(np.array_equal(a, b) for a, b in zip(w0.y, w1.y))
    want = np.minimum(256, -(-w0.ranks // pad) * pad)
    assert np.array_equal(w1.ranks, want) and (w1.ranks % pad == 0).all()
    assert (w1.ranks >= w0.ranks).all()


def test_mfma_util_follows_the_kernel_sources(tmp_path, monkeypatch):
    """The committed counter runs are read back while they match the sources."""
    for cfg in ("prefill7b", "mixed13b"):
        u = bench.load_mfma_util(cfg)
        assert u is not None and 0 < u["mfma_util_percent"] < 100, cfg
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_mfma_util("prefill7b") is None
    os.makedirs(os.path.join(str(tmp_path), "profiles"))
    with open(os.path.join(str(tmp_path), "profiles", "mfma_prefill7b.json"), "w") as f:
        json.dump({"kernel_source_hash": "0" * 16, "mfma_util_percent": 5.0,
                   "mfma_flops_f16_per_launch": 1.0, "counters": "x"}, f)
    assert bench.load_mfma_util("prefill7b") is None
