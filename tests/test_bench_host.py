"""Host-side pieces of the benchmark (no GPU): the algorithmic byte counts
the roofline fractions divide by, the indexer-key byte report, the metric
strings, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from top_sparse_attention_ls_amd import synth  # noqa: E402


def test_headline_step_bytes():
    # 128K x 32: compact keys 268.4 MB + candidates' keys 33.6 MB + slot table
    # + 20% misses read and written + selected rows + q / out / lse + idx q, w
    wl = synth.WORKLOADS["decode-128k-b32"]
    ab = bench.algorithmic_bytes(wl, n_miss_total=32 * 410)
    assert ab["coarse_keys"] == 32 * 131072 * 64
    assert ab["refine_keys"] == 32 * 8192 * 128
    assert ab["miss_read"] == ab["miss_write"] == 32 * 410 * 1152
    assert ab["kv_rows"] == 32 * 2048 * 1152
    assert ab["total"] == 417_171_456


def test_indexer_key_bytes_near_1m_context():
    # coarse-only pass 243.2 MB + refinement 8.39 MB against 486.4 MB of
    # full-key scoring
    wl = synth.WORKLOADS["decode-950k-b4"]
    ab = bench.algorithmic_bytes(wl, n_miss_total=4 * 410)
    r = bench.indexer_key_bytes(wl, ab)
    assert r["coarse_pass"] == 243_200_000
    assert r["refine"] == 8_388_608
    assert r["full_key_scoring"] == 486_400_000
    assert r["coarse_to_fine_total"] == 251_588_608
    assert r["ratio"] == round(251_588_608 / 486_400_000, 4)


def test_mha_rows_count_k_and_v_of_every_head():
    wl = synth.WORKLOADS["tiny-4k"]
    ab = bench.algorithmic_bytes(wl, 0)
    assert ab["kv_rows"] == 256 * 8 * (64 + 64) * 2


def test_every_decode_workload_has_its_own_metric():
    names = [n for n, w in synth.WORKLOADS.items() if not w.n_query and not w.serve_drift]
    metrics = [bench.metric_for(synth.WORKLOADS[n]) for n in names]
    assert len(set(metrics)) == len(metrics)
    assert bench.metric_for(synth.WORKLOADS["decode-128k-b32"]) == bench.METRIC
    assert "16K (B=192)" in bench.metric_for(synth.WORKLOADS["decode-16k-b192"])
    assert "950K (B=4)" in bench.metric_for(synth.WORKLOADS["decode-950k-b4"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_gather_folded_only_for_device_pools_on_the_latent_path():
    # the library folds the miss gather into the attention's tile DMA when
    # the pool is in device memory and the rows are latent (MLA) rows; the
    # bench then books the gather's bytes to the attention stage
    import bench
    from top_sparse_attention_ls_amd import synth
    W = synth.WORKLOADS
    assert bench.gather_folded(W["decode-128k-b32"])
    assert bench.gather_folded(W["decode-950k-b4"])
    assert not bench.gather_folded(W["decode-16k-b192"])    # pool in pinned host memory
    assert not bench.gather_folded(W["tiny-4k"])            # no hot buffer, MHA rows
