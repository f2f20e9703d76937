"""The allocation-free backward entry point (fa_backward_noalloc) against
fa_backward: the same kernels, with the statistics in the library's per-GPU
scratch array instead of a caller's workspace, so the gradients must agree bit
for bit. Two calls in a row, the second smaller (the array keeps the first
call's contents), then a size beyond the array, which must be refused before
anything runs."""

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


def _case(B, H, Hkv, N, d, dtype, causal, seed, mask=None):
    where = f"noalloc B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} mask={mask is not None}"
    PT.say("case", where)
    x = I.make_small(B, H, Hkv, N, d, dtype, seed)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    mt = None if mask is None else torch.from_numpy(mask).to(dev)
    o, lse = binding.forward(q, k, v, None, causal, mt)
    ref = binding.backward(q, k, v, o, lse, do, None, causal, mt)
    got = binding.backward_noalloc(q, k, v, o, lse, do, None, causal, mt)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{where}: {name} differs from fa_backward"
    # and both against the oracle, to the parity bar
    import oracle
    qd, kd, vd, dod = (PT.np64(x[n]) for n in ("q", "k", "v", "do"))
    rq, rk, rv = oracle.backward(qd, kd, vd, dod, 1.0 / np.sqrt(d), causal, mask)
    for name, a, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
        PT.check_grad(PT.np64(a), r, f"{where} {name}")


def test_noalloc_matches_backward_twice():
    _case(2, 8, 2, 1500, 128, "bf16", True, seed=71)
    m = I.random_block_mask(300, 0.5, 5, keep_diagonal=True)
    _case(1, 2, 1, 300, 64, "fp16", False, seed=72, mask=m)


def test_noalloc_rejects_beyond_scratch():
    # 64 heads x 65536 rows x 8 bytes = 32 MiB of statistics > 16 MiB
    dev = torch.device("cuda", 0)
    q = torch.zeros((1, 64, 65536, 32), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 1, 65536, 32), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((1, 64, 65536), dtype=torch.float32, device=dev)
    with pytest.raises(binding.FAError) as e:
        binding.backward_noalloc(q, k, k, q, lse, q, None, True, None, grads=(q, k, k))
    assert e.value.status == -2
