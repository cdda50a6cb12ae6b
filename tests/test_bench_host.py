"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic byte count that the HBM roofline divides by, and that every
committed traffic profile was taken on the current kernel sources (the bench
reports `roofline.traffic` only while they match)."""
import glob
import json
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_alg_bytes_of_the_tiny_workload_by_hand():
    """tiny_fp32: B 4, L = 1, 17, 64, 130, 8 / 8 heads, D 64, P 16, fp32
    throughout.  Decode reads every cached K and V element once (4 bytes
    each), q and writes out, one page id per used page and the lengths; the
    append reads the new K and V rows and writes them into the pools."""
    wl = configs.tiny_fp32()
    assert list(wl.seq_lens) == [1, 17, 64, 130] and (wl.Hq, wl.Hkv, wl.D, wl.P) == (8, 8, 64, 16)
    dec, app, kv = bench.alg_bytes(wl, wl.seq_lens)
    tokens = 1 + 17 + 64 + 130
    assert kv == tokens * 8 * 64 * 4 * 2
    pages = 1 + 2 + 4 + 9
    assert dec == kv + 4 * 8 * 64 * (4 + 4) + pages * 4 + 4 * 4
    assert app == 2 * (4 * 8 * 64 * 4 * 2) + 4 * 8


def test_alg_bytes_scaled_cache_counts_page_scales():
    """An fp8 cache adds a K and a V scale (4 bytes each) per used page and kv
    head, and its elements are one byte."""
    wl = configs.tiny_fp32()
    wl.kv_dtype, wl.q_dtype, wl.out_dtype = "fp8", "bf16", "bf16"
    dec, _, kv = bench.alg_bytes(wl, wl.seq_lens)
    pages = 1 + 2 + 4 + 9
    assert kv == 212 * 8 * 64 * 1 * 2
    assert dec == kv + 4 * 8 * 64 * (2 + 2) + pages * 4 + 4 * 4 + pages * 8 * 4 * 2


def test_committed_traffic_profiles_match_the_kernel_sources():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")))
    assert files, "no traffic profiles committed"
    for f in files:
        t = json.load(open(f))
        srcs = bench.PREFILL_SRCS if os.path.basename(f).startswith("prefill_") else bench.DECODE_SRCS
        assert t["kernel_source_sha256_16"] == bench.kernel_hash(srcs), \
            f"{os.path.basename(f)} was taken on other kernel sources: profile again"
        assert t["workload"] in bench.WORKLOADS


def test_every_bench_workload_has_a_generator():
    names = set(configs.CONFIGS) | set(configs.PREFILL_CONFIGS)
    assert set(bench.WORKLOADS) <= names
