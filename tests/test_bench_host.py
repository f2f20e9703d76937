"""bench.py's host-side definitions, checked on the CPU: the FLOP counts of
the metric against the per-workload figures worked out independently from
the shapes (2 N^2 d per N x N x d contraction, halved under causal masking,
two contractions forward and five backward; block-sparse counted per kept
128 x 128 block), the default run configuration, the refusal of more than
one GPU, and the counter-traffic lookup's source check."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_attention_110_amd import inputs as I  # noqa: E402


@pytest.mark.parametrize("name,fwd,total", [
    ("gpt2_small_bf16", 1.2885e10, 4.5097e10),        # 8 x 12 heads, N 1024, d 64, causal
    ("long_seq_bf16", 1.09951e12, 3.84829e12),        # 16 heads, N 16384, d 128, causal
    ("gqa_bf16", 2.19902e12, None),                   # 4 x 32 heads, N 8192, d 128, causal, forward only
    ("single_head_fp32", 3.3554e7, None),             # one head, N 512, d 32, not causal
])
def test_dense_flop_counts(name, fwd, total):
    w = I.WORKLOADS[name]
    assert bench.flops(w, False) == pytest.approx(fwd, rel=1e-4)
    if total is not None:
        assert bench.flops(w, True) == pytest.approx(total, rel=1e-4)
        assert bench.flops(w, True) / bench.flops(w, False) == pytest.approx(3.5)


def test_block_sparse_flop_count():
    """15,047 kept blocks x 8 heads x 2 * 128 * 128 * 64 per contraction."""
    w = I.WORKLOADS["block_sparse_fp16"]
    m = I.band_plus_random_mask(w.N, w.seed + 200)
    per = 2 * 128 * 128 * 64 * 8 * 15047
    assert bench.sparse_flops(w, m, False) == pytest.approx(2 * per)
    assert bench.sparse_flops(w, m, True) == pytest.approx(7 * per)
    assert bench.sparse_flops(w, m, False) == pytest.approx(5.049e11, rel=1e-3)
    with pytest.raises(ValueError):
        bench.flops(w)


def test_default_configuration(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.workload) == (1, 20, 3, "long_seq_bf16")
    assert a.dropout == 0.0 and not a.fp8 and a.window == 0 and not a.alibi


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_lookup_checks_the_sources(monkeypatch):
    """A kernel's counter traffic is reported only while its sources hash as
    they did when the counters were taken: a changed hash gives None."""
    monkeypatch.setitem(bench.KERNEL_SOURCES, "bwd_kv_kernel", ["bwd.hip", "common.hpp"])
    assert bench.measured_traffic("bwd_kv_kernel", "long_seq_bf16") is None
    assert bench.measured_traffic("no_such_kernel", "long_seq_bf16") is None


def test_committed_profiles_cover_the_current_sources():
    """The counter summaries under profiles/ were taken from the kernels as they
    are: every kernel of the long-sequence step has a traffic line whose source
    hash matches, so bench.py reports its counter bytes (after a change to a
    kernel source or the compiler flags, the profiles are taken again)."""
    for k in ("fwd64_kernel", "bwd_pre_kernel", "bwd_kv_kernel", "bwd_q_kernel"):
        t = bench.measured_traffic(k, "long_seq_bf16")
        assert t is not None and t > 0, k
