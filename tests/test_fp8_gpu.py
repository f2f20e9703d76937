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
