"""The bench's host-side legs on tiny workloads (no GPU): the oracle baseline runs on host
copies of each workload kind's inputs and reports a positive rate."""
import dataclasses
import os
import sys

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from compressed_sparse_attention_gated_amd import workloads as W  # noqa: E402


def _small(cfg, **kw):
    return dataclasses.replace(W.WORKLOADS[cfg], **kw)


@pytest.mark.parametrize("cfg,kw,build", [
    (2, dict(B=2, L=300, k=32, window=16), "decode"),
    (5, dict(B=2, L=300, k=32, window=16), "decode"),
    (4, dict(B=2, L=512, k=32, window=16, n_keep_blocks=16), "hier"),
    (6, dict(B=2, L=128 * 40, window=16), "hca"),
])
def test_cpu_baseline_decode_kinds(cfg, kw, build):
    wl = _small(cfg, **kw)
    if build == "hier":
        d = W.hier_inputs(wl, 3, device="cpu")
    elif build == "hca":
        d = W.hca_inputs(wl, 3, device="cpu")
    else:
        d = W.decode_inputs(wl, 3, device="cpu")
    r = bench.cpu_baseline(torch, wl, d, 0.05)
    assert r["value"] > 0 and r["unit"] == "queries/s" and r["kind"] == "oracle" and r["cores"] >= 1
    assert r["nproc"] >= 1 and r["cpu_count"] >= r["nproc"] and "cpu_model" in r
    assert r["single_thread"]["value"] > 0 and r["single_thread"]["cores"] == 1


def test_cpu_baseline_prefill():
    wl = _small(3, n_tokens=256, k=16, window=16)
    d = W.prefill_inputs(wl, 3, device="cpu")
    r = bench.cpu_baseline(torch, wl, d, 0.05)
    assert r["value"] > 0 and r["unit"] == "tokens/s"
