"""Host-side parts of bench.py, on the CPU: the algorithmic work each stage's
roofline divides by, against closed forms worked out by hand for two of the
measured workloads; the traffic figures, which must be dropped once a
kernel's source no longer matches the one that was profiled; the labels of
the timed kernels; and the one-GPU guard."""

import json
import os
import subprocess
import sys

import pytest

import bench
from sparse_attention_long_fp8_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_32k_work():
    # 32 decodes over 32768 keys each; FP8 keys of 128 bytes + a 4-byte scale,
    # a 4-byte score written per key; per query 64 x 128 FP8 + scale + 64 weights
    wl = synth.WORKLOADS["decode_32k"]
    w = bench.stage_work(wl, synth.make_layout(wl))
    pairs = 32 * 32768
    assert w["pairs"] == pairs and w["selected"] == 32 * 2048
    assert w["indexer"]["bytes"] == pairs * 136 + 32 * (64 * 128 + 4 + 4 * 64)
    assert abs(w["indexer"]["bytes"] / 1e6 - 142.9) < 0.05
    # gathered latent rows (2048 x 576 bf16 a query), q and o (128 heads), lse, indices
    mla = 32 * 2048 * 1152 + 32 * 128 * (576 + 512) * 2 + 32 * 128 * 4 + 32 * 2048 * 4
    assert w["mla"]["bytes"] == mla and abs(mla / 1e6 - 84.7) < 0.05
    assert abs(w["indexer"]["flops"] / 1e9 - 17.2) < 0.05        # 2 x 64 x 128 per pair
    assert abs(w["mla"]["flops"] / 1e9 - 18.3) < 0.05            # 2 x 128 x (576 + 512) per selected pair
    assert w["topk"]["bytes"] == pairs * 4 + 32 * 2048 * 4


def test_prefill_16k_work():
    # causal pairs sum_{t<L} (t+1); selected pairs sum_t min(k, t+1)
    wl = synth.WORKLOADS["prefill_16k"]
    w = bench.stage_work(wl, synth.make_layout(wl))
    L, k = 16384, 2048
    pairs = L * (L + 1) // 2
    sel = k * (k + 1) // 2 + (L - k) * k
    assert w["pairs"] == pairs and w["selected"] == sel and w["queries"] == L
    assert abs(w["indexer"]["flops"] / 2.199e12 - 1) < 1e-3
    assert abs(w["mla"]["flops"] / 8.762e12 - 1) < 1e-3


def test_traffic_needs_the_profiled_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_of("mla", "decode_32k") is None          # no summary
    rec = {"mla": {"source_sha256_16": bench.source_hash("mla"), "hbm_bytes_per_launch": 123.0},
           "topk": {"source_sha256_16": "0" * 16, "hbm_bytes_per_launch": 7.0}}
    (tmp_path / "traffic_decode_32k.json").write_text(json.dumps(rec))
    assert bench.traffic_of("mla", "decode_32k") == 123.0
    assert bench.traffic_of("topk", "decode_32k") is None          # profiled on another source
    assert bench.traffic_of("indexer", "decode_32k") is None       # not profiled


def test_kernel_labels():
    lab = {n: bench.kernel_name("mla", synth.WORKLOADS[n], synth.make_layout(synth.WORKLOADS[n]))
           for n in ("decode_32k", "paged_decode", "prefill_16k", "tiny_prefill")}
    # few rows: the selections are split into ranges and merged
    assert lab["decode_32k"] == lab["paged_decode"] == "mla_bf16_kernel + mla_combine_kernel"
    assert lab["prefill_16k"] == "mla_bf16_kernel" and lab["tiny_prefill"] == "mla_f32_kernel"
    wl = synth.WORKLOADS["decode_32k"]
    assert bench.kernel_name("indexer", wl, synth.make_layout(wl)) == "indexer_fp8_staged_kernel"
    tk = {n: bench.kernel_name("topk", synth.WORKLOADS[n], synth.make_layout(synth.WORKLOADS[n]))
          for n in ("decode_32k", "paged_decode", "prefill_16k")}
    # decode rows in one pass load before their length is known; paged rows
    # past 32768 keys take the two passes, prefill rows the general form
    assert tk == {"decode_32k": "topk_kernel<true>", "paged_decode": "topk_kernel<false>",
                  "prefill_16k": "topk_kernel<false>"}


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout


def test_prefill_oracle_sample():
    # the fixed rows (ends and the k boundary) plus one seeded row per stratum,
    # deterministic and inside [0, L)
    fixed, strat = bench.prefill_sample_rows(65536, 2048, 256)
    assert fixed == [0, 1, 2046, 2047, 2048, 2049, 65535]
    assert len(strat) == 249 and all(0 <= r < 65536 for r in strat)
    edges = [int(x) for x in __import__("numpy").linspace(0, 65536, 250)]
    assert all(edges[i] <= r < edges[i + 1] for i, r in enumerate(strat))
    assert (fixed, strat) == bench.prefill_sample_rows(65536, 2048, 256)
    assert len(set(fixed) | set(strat)) >= 250


def test_headline_is_the_long_prefill():
    # the default line measures the largest single-GPU workload
    assert bench.HEADLINE == "prefill_64k"
    assert set(bench.ALL_WORKLOADS) == set(synth.WORKLOADS)
