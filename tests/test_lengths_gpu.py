"""GPU parity for unequal query and key lengths (causal masking aligned to the
last query) and for packed variable-length batches: every output element of
the HIP path against the float64 oracle, on seeded inputs that span several
tiles, ragged tails, empty sequences and rows that see no key."""

import math

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


CROSS_SHAPES = [
    # B, H, Hkv, Nq, Nk, d
    (1, 2, 1, 1, 300, 64),       # one query over a long cache
    (1, 2, 2, 17, 200, 128),
    (2, 2, 1, 100, 300, 64),
    (1, 4, 2, 300, 100, 32),     # more queries than keys: the first 200 see nothing
    (1, 2, 2, 129, 513, 128),
    (1, 1, 1, 513, 129, 64),
    (2, 3, 3, 64, 1000, 128),
    (1, 2, 1, 1000, 999, 64),
]


def _seed(*xs):
    return int(sum((i + 1) * 131 * x for i, x in enumerate(xs)) % 100003)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", CROSS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_cross_lengths(shape, causal, dtype):
    B, H, Hkv, Nq, Nk, d = shape
    PT.run_cross(B, H, Hkv, Nq, Nk, d, dtype, causal, seed=_seed(*shape, causal, dtype == "fp16"))


@pytest.mark.parametrize("rows", ["64", "32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", CROSS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_cross_lengths_forward_kernels(shape, causal, rows):
    """Both 16-bit forward kernels, forced through fa_forward_select."""
    B, H, Hkv, Nq, Nk, d = shape
    PT.run_cross(B, H, Hkv, Nq, Nk, d, "bf16", causal, seed=_seed(*shape, causal, 7), backward=False,
                 rows_per_wave=int(rows))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,d", [(1, 700, 32), (100, 37, 64), (300, 513, 128)])
def test_cross_lengths_fp32(Nq, Nk, d, causal):
    PT.run_cross(1, 2, 1, Nq, Nk, d, "fp32", causal, seed=_seed(Nq, Nk, d, causal), backward=False)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,density", [(300, 700, 0.5), (700, 300, 0.5), (129, 1100, 0.3)])
def test_cross_lengths_block_sparse(Nq, Nk, density, causal):
    mask = I.random_block_mask(Nq, density, _seed(Nq, Nk), n_keys=Nk)
    PT.run_cross(1, 2, 1, Nq, Nk, 64, "bf16", causal, mask=mask, seed=_seed(Nq, Nk, causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 100, 300, 64), (1, 2, 2, 300, 129, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_cross_lengths_dropout(shape, causal):
    B, H, Hkv, Nq, Nk, d = shape
    PT.run_cross(B, H, Hkv, Nq, Nk, d, "bf16", causal, seed=_seed(*shape), dropout_rate=0.25,
                 drop_seed=_seed(*shape, 3))


VARLEN = [
    # lens_q, lens_k, H, Hkv, d
    ([5, 130, 1, 257, 64], [5, 130, 1, 257, 64], 4, 2, 64),
    ([3, 200, 0, 77], [100, 200, 5, 0], 2, 1, 128),          # empty query run; keys-free sequence
    ([300, 31, 129], [40, 500, 129], 2, 2, 32),
    (I.length_mix(8, 150, 11), I.length_mix(8, 150, 11), 3, 1, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen(case, causal, dtype):
    lq, lk, H, Hkv, d = VARLEN[case]
    PT.run_varlen(lq, lk, H, Hkv, d, dtype, causal, seed=_seed(case, causal, dtype == "fp16", 9))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen_fp32(case, causal):
    lq, lk, H, Hkv, d = VARLEN[case]
    PT.run_varlen(lq, lk, H, Hkv, d, "fp32", causal, seed=_seed(case, causal, 21), backward=False)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_dropout(causal):
    lq, lk, H, Hkv, d = VARLEN[2]
    PT.run_varlen(lq, lk, H, Hkv, d, "bf16", causal, seed=31, dropout_rate=0.3, drop_seed=77)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_long_sequences(causal, dtype):
    """Packed sequences long enough (the longest 9000 keys at d = 128) that the
    library takes the 64-row forward kernel for the packed batch, with an empty
    and a short sequence between them: every element against the oracle."""
    lens = [9000, 0, 131, 8300]
    assert binding.forward_kernel_rows(len(lens), 2, 1, max(lens), max(lens), 128, causal) == 64
    PT.run_varlen(lens, lens, 2, 1, 128, dtype, causal, seed=_seed(7, causal, dtype == "fp16", 13))


def test_varlen_grid_larger_than_sequences():
    """max_seqlen above every length: the extra workgroups exit without writing."""
    PT.run_varlen([70, 5], [9, 300], 2, 1, 64, "bf16", True, seed=41, max_q=1000, max_k=1200)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_fixed_bitwise(causal):
    """A packed batch of equal lengths runs the same arithmetic per sequence as
    the fixed-length entry points: the results agree bit for bit."""
    B, H, Hkv, N, d = 3, 4, 2, 333, 128
    x = I.make_small(B, H, Hkv, N, d, "bf16", 51)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = binding.forward(q, k, v, None, causal)
    dq, dk, dv = binding.backward(q, k, v, o, lse, do, None, causal)

    def pack(t):
        return t.transpose(0, 1).reshape(t.shape[1], t.shape[0] * t.shape[2], t.shape[3]).contiguous()

    cu = torch.tensor([0, N, 2 * N, 3 * N], dtype=torch.int32, device=dev)
    ov, lv = binding.forward_varlen(pack(q), pack(k), pack(v), cu, cu, N, N, None, causal)
    dqv, dkv, dvv = binding.backward_varlen(pack(q), pack(k), pack(v), ov, lv, pack(do), cu, cu, N, N, None,
                                            causal)
    torch.cuda.synchronize()
    assert torch.equal(ov, pack(o))
    assert torch.equal(lv, lse.transpose(0, 1).reshape(H, B * N))
    assert torch.equal(dqv, pack(dq)) and torch.equal(dkv, pack(dk)) and torch.equal(dvv, pack(dv))


def test_cross_lengths_large_sampled():
    """A 2048-query chunk over 16384 cached keys (causal, bf16, 16 heads at the
    bench's head size): one head's sampled rows and its key gradients' rows
    against the oracle."""
    B, H, Hkv, Nq, Nk, d = 1, 16, 16, 2048, 16384, 128
    x = I.make_cross(B, H, Hkv, Nq, Nk, d, "bf16", 61)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = binding.forward(q, k, v, scale, True)
    dq, dk, dv = binding.backward(q, k, v, o, lse, do, scale, True)
    torch.cuda.synchronize()
    h = 5
    rows = np.sort(np.random.default_rng(62).choice(Nq, size=64, replace=False))
    qd, kd, vd = (PT.np64(x[n][:, h:h + 1]) for n in ("q", "k", "v"))
    oref, lref = oracle.forward(qd, kd, vd, scale, True, rows=rows)
    PT.check_out(PT.np64(o[:, h:h + 1, rows]), oref, "bf16", "large cross forward")
    PT.check_lse(PT.np64(lse[:, h:h + 1, rows]), lref, "large cross lse")
    rq, rk, rv = oracle.backward(qd, kd, vd, PT.np64(x["do"][:, h:h + 1]), scale, True)
    PT.check_grad(PT.np64(dq[:, h:h + 1]), rq, "large cross dq")
    PT.check_grad(PT.np64(dk[:, h:h + 1]), rk, "large cross dk")
    PT.check_grad(PT.np64(dv[:, h:h + 1]), rv, "large cross dv")
