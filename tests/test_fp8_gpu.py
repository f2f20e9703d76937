"""GPU parity of the FP8 (E4M3) forward pass against the float64 oracle on the
decoded inputs: every output element within the per-element bound derived
from the kernel's arithmetic (the probabilities' rounding to E4M3 and the FP8
matrix instruction's measured summing precision), LSE within 1e-5 or, where
larger, the bound from that summing precision, over shapes that span several
tiles, ragged tails and grouped heads."""

import numpy as np
import pytest
import torch

import parity as PT
from exact_attention_110_amd import binding
from exact_attention_110_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_lib):
    yield


SHAPES = [
    # B, H, Hkv, N, d
    (1, 2, 1, 1, 64),
    (1, 2, 2, 17, 128),
    (2, 2, 1, 300, 64),
    (1, 4, 2, 513, 128),
    (1, 2, 2, 1000, 128),
]


@pytest.mark.parametrize("out", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_forward(shape, causal, out):
    B, H, Hkv, N, d = shape
    PT.run_fp8(B, H, Hkv, N, d, causal, seed=N + d + 3 * int(causal) + (7 if out == "fp16" else 0), out_dtype=out)


def test_fp8_descales_exact(gpu_lib):
    """q and k descales enter only through their product with the scale, the
    value descale only as an output factor: powers of two change nothing but
    that factor, bit for bit."""
    x = I.make_fp8(1, 4, 2, 700, 128, 11)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o1, l1 = binding.forward_fp8(q, k, v, 1.0, 1.0, 1.0, 0.1, True)
    o2, l2 = binding.forward_fp8(q, k, v, 4.0, 0.25, 2.0, 0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2)
    assert torch.equal(o2, 2 * o1)


def test_fp8_rejects(gpu_lib):
    x = I.make_fp8(1, 2, 1, 64, 64, 1)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(binding.FAError):
            binding.forward_fp8(q, k, v, bad, 1.0, 1.0)
    q32 = torch.zeros((1, 2, 64, 32), dtype=torch.uint8, device=dev)
    with pytest.raises(binding.FAError):
        binding.forward_fp8(q32, q32[:, :1], q32[:, :1], 1.0, 1.0, 1.0)


def test_fp8_large_sampled():
    """The throughput workload's shape (B 1, H 16, N 16384, d 128, causal) in
    FP8: two heads' sampled rows against the oracle and the derived bound."""
    rows = np.sort(np.random.default_rng(91).choice(16384, size=48, replace=False))
    PT.run_fp8(1, 16, 16, 16384, 128, True, seed=90, heads=[(0, 3), (0, 12)], rows=rows)


def test_fp8_summing_precision(gpu_lib):
    """The measurement behind the FP8 bars' summing term (FP8_SUM in
    tests/parity.py): 65536 rows that each see exactly one key (N = 1), so
    that the kernel's LSE is that row's single score, scale * q . k, with unit
    descales. Against the exact float64 dot product of the decoded codes, the
    error left after the float32 steps that follow the matrix instruction (the
    scale, log2 e and ln 2 products: at most 4 ulps of |LSE|) is the
    instruction's summing error; relative to sum_d |q_d k_d| it must stay
    within FP8_SUM, and the largest value found is printed."""
    import oracle.fp8 as F8
    B, H, d = 64, 1024, 128
    x = I.make_fp8(B, H, H, 1, d, seed=77)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    _, lse = binding.forward_fp8(q, k, v, 1.0, 1.0, 1.0, scale=1.0, causal=False)
    torch.cuda.synchronize()
    got = PT.np64(lse).reshape(-1)
    qd = F8.e4m3_decode(x["q"].numpy()).reshape(-1, d)
    kd = F8.e4m3_decode(x["k"].numpy()).reshape(-1, d)
    exact = (qd * kd).sum(axis=1)
    mag = np.abs(qd * kd).sum(axis=1)
    resid = np.maximum(np.abs(got - exact) - 4 * 2.0 ** -24 * np.abs(got), 0.0)
    rel = resid / np.maximum(mag, 1e-30)
    worst = float(rel.max())
    PT.say(f"FP8 summing error: max {worst / 2.0 ** -24:.0f} * 2^-24 * sum|products| over {rel.size} dot products "
           f"(bar FP8_SUM = 2^-11 = {PT.FP8_SUM / 2.0 ** -24:.0f} * 2^-24; ratio {worst / PT.FP8_SUM:.3f})")
    assert np.all(np.isfinite(got))
    assert worst <= PT.FP8_SUM
