"""Invariants of exact attention replayed on the GPU output.

* Causal-prefix locality: under causal masking row i depends only on keys
  j <= i (the "FlashAttention" lesson, Beginner tier, "What was broken
  before": a word looks only at earlier words). Keys and values after a row
  index i0 are replaced by strongly aligned ones and large values; O, LSE and dQ of rows
  0..i0 must come back bit for bit identical when every row of their waves is
  at most i0 (the kernels make no decision that couples rows of different
  waves), and for a row index inside a wave still within the parity bar of
  the unperturbed oracle.
* Permutation equivariance: with neither causal nor block masking the keys
  are a set (same lesson, Researcher tier, "The problem being solved": each
  row's softmax runs over all keys). Permuting the rows of K and V together
  leaves O and LSE unchanged and permutes dK and dV; permuting the rows of Q
  permutes O, LSE and dQ. The two runs differ only by the order of the
  floating-point sums, so they are held to a bar tighter than the parity bar.
"""

import numpy as np
import pytest
import torch

import oracle
import parity as PT
from exact_attention_110_amd import binding
from exact_attention_110_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_lib):
    yield


def _run(x, causal, rows_per_wave, backward=True):
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    d = q.shape[-1]
    o, lse = binding.forward(q, k, v, d ** -0.5, causal, None, rows_per_wave=rows_per_wave)
    grads = None
    if backward:
        grads = binding.backward(q, k, v, o, lse, x["do"].to(dev), d ** -0.5, causal, None)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), None if grads is None else tuple(g.cpu() for g in grads)


def _o_bar(o):
    """Two bf16 ulps of |O| plus 2^-10."""
    return 2.0 ** -6 * np.abs(PT.np64(o)) + 2.0 ** -10


def _perturb_after(x, i0):
    """Keys and values after row i0 replaced: key j becomes 3 q_j (so row j,
    and any row that could see key j, would weight it far above every other
    key) and every value 1000."""
    y = {n: t.clone() for n, t in x.items()}
    G = x["q"].shape[1] // x["k"].shape[1]
    y["k"][:, :, i0 + 1:] = (3.0 * x["q"][:, ::G, i0 + 1:].float()).to(x["k"].dtype)
    y["v"][:, :, i0 + 1:] = 1000.0
    return y


@pytest.mark.parametrize("rows", [64, 32])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_prefix_locality_bitwise(rows, d):
    # i0 + 1 = 576 is a multiple of both wave heights (64 and 32 rows) but not
    # of the workgroup heights (256, 128): rows 0..575 share workgroups, tiles
    # and diagonal masks with perturbed rows, but not waves
    B, H, Hkv, N, i0 = 1, 4, 2, 1000, 575
    x = I.make_small(B, H, Hkv, N, d, "bf16", seed=300 + d + rows)
    y = _perturb_after(x, i0)
    o1, l1, (dq1, _, _) = _run(x, True, rows)
    o2, l2, (dq2, _, _) = _run(y, True, rows)
    PT.say(f"locality rows_per_wave={rows} d={d}: rows 0..{i0} bitwise, perturbed from {i0 + 1}")
    assert torch.equal(o1[:, :, :i0 + 1], o2[:, :, :i0 + 1])
    assert torch.equal(l1[:, :, :i0 + 1], l2[:, :, :i0 + 1])
    assert torch.equal(dq1[:, :, :i0 + 1], dq2[:, :, :i0 + 1])
    # the perturbation reaches the later rows (the check above is not vacuous)
    assert (o2[:, :, i0 + 1:].float() - o1[:, :, i0 + 1:].float()).abs().max() > 100.0


@pytest.mark.parametrize("rows", [64, 32])
def test_causal_prefix_locality_inside_a_wave(rows):
    """Perturbation starting inside a wave: rows up to i0 still match the
    oracle on the unperturbed inputs to the parity bar."""
    B, H, Hkv, N, d, i0 = 1, 2, 1, 700, 128, 600
    x = I.make_small(B, H, Hkv, N, d, "bf16", seed=410 + rows)
    y = _perturb_after(x, i0)
    o, lse, (dq, _, _) = _run(y, True, rows)
    qd, kd, vd, dod = (PT.np64(x[n]) for n in ("q", "k", "v", "do"))
    r = np.arange(i0 + 1)
    oref, lref = oracle.forward(qd, kd, vd, d ** -0.5, True, rows=r)
    where = f"locality inside a wave rows_per_wave={rows}"
    PT.check_out(PT.np64(o[:, :, :i0 + 1]), oref, "bf16", where)
    PT.check_lse(PT.np64(lse[:, :, :i0 + 1]), lref, where)
    rq, _, _ = oracle.backward(qd, kd, vd, dod, d ** -0.5, True)
    PT.check_grad(PT.np64(dq[:, :, :i0 + 1]), rq[:, :, :i0 + 1], where + " dq")


@pytest.mark.parametrize("rows", [64, 32])
@pytest.mark.parametrize("N,d", [(777, 64), (1000, 128)])
def test_kv_permutation_equivariance(N, d, rows):
    B, H, Hkv = 1, 4, 2
    x = I.make_small(B, H, Hkv, N, d, "bf16", seed=500 + N + rows)
    perm = torch.from_numpy(np.random.default_rng(N + d).permutation(N))
    y = dict(x)
    y["k"] = x["k"][:, :, perm].contiguous()
    y["v"] = x["v"][:, :, perm].contiguous()
    o1, l1, (dq1, dk1, dv1) = _run(x, False, rows)
    o2, l2, (dq2, dk2, dv2) = _run(y, False, rows)
    where = f"K/V permutation N={N} d={d} rows_per_wave={rows}"
    PT.say(where)
    # the same sums in another order (and the running reference raised at
    # other tiles, which rounds the 16-bit probabilities differently): O
    # within 2 bf16 ulps plus 2^-10, a twentieth of the parity bar; LSE within
    # float32 rounding; gradients within a tenth of the parity bar
    assert np.all(np.abs(PT.np64(o2) - PT.np64(o1)) <= _o_bar(o1)), where
    assert PT.max_abs(PT.np64(l2), PT.np64(l1)) <= 2e-6, where
    assert PT.rel_frob(PT.np64(dq2), PT.np64(dq1)) <= 5e-3, where + " dq"
    assert PT.rel_frob(PT.np64(dk2), PT.np64(dk1[:, :, perm])) <= 5e-3, where + " dk"
    assert PT.rel_frob(PT.np64(dv2), PT.np64(dv1[:, :, perm])) <= 5e-3, where + " dv"


@pytest.mark.parametrize("rows", [64, 32])
def test_q_permutation_equivariance(rows):
    B, H, Hkv, N, d = 1, 2, 2, 900, 128
    x = I.make_small(B, H, Hkv, N, d, "bf16", seed=610 + rows)
    perm = torch.from_numpy(np.random.default_rng(7).permutation(N))
    y = dict(x)
    y["q"] = x["q"][:, :, perm].contiguous()
    y["do"] = x["do"][:, :, perm].contiguous()
    o1, l1, (dq1, dk1, dv1) = _run(x, False, rows)
    o2, l2, (dq2, dk2, dv2) = _run(y, False, rows)
    where = f"Q permutation rows_per_wave={rows}"
    PT.say(where)
    # a row's result depends on its wave-mates only through the wave-wide
    # decision to raise the running reference, which moves it by rounding:
    # the moved rows are held to the same bars as the permuted keys above
    assert np.all(np.abs(PT.np64(o2) - PT.np64(o1[:, :, perm])) <= _o_bar(o1[:, :, perm])), where
    assert PT.max_abs(PT.np64(l2), PT.np64(l1[:, :, perm])) <= 2e-6, where
    assert PT.rel_frob(PT.np64(dq2), PT.np64(dq1[:, :, perm])) <= 5e-3, where + " dq"
    assert PT.rel_frob(PT.np64(dk2), PT.np64(dk1)) <= 5e-3, where + " dk"
    assert PT.rel_frob(PT.np64(dv2), PT.np64(dv1)) <= 5e-3, where + " dv"
