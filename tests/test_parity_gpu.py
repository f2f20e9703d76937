"""GPU parity on small shapes: every output element of the HIP path against the
float64 oracle, on seeded inputs that span several tiles and ragged tails."""

import numpy as np
import pytest
import torch

import parity as PT
from exact_attention_110_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_lib):
    yield


SHAPES = [
    # B, H, Hkv, N, d
    (1, 1, 1, 1, 64),
    (1, 2, 1, 17, 32),
    (2, 2, 2, 64, 64),
    (1, 3, 1, 127, 128),
    (1, 2, 2, 128, 128),
    (1, 4, 2, 129, 64),
    (2, 4, 1, 300, 32),
    (1, 2, 2, 513, 128),
    (1, 8, 2, 1000, 64),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dense(shape, causal, dtype):
    B, H, Hkv, N, d = shape
    seed = 1000 * B + 100 * H + 10 * Hkv + N + 7 * d + 3 * int(causal) + (1 if dtype == "fp16" else 0)
    PT.run_small(B, H, Hkv, N, d, dtype, causal, seed=seed)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dense_64_rows_per_wave(shape, causal, dtype):
    """The 64-row forward kernel (chosen by the library at head size 128 for
    large enough grids and long enough rows) at every small shape, forced
    through fa_forward_select."""
    B, H, Hkv, N, d = shape
    PT.run_small(B, H, Hkv, N, d, dtype, causal, seed=5000 + N + d + int(causal) + (1 if dtype == "fp16" else 0),
                 backward=False, rows_per_wave=64)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N", [1, 100, 512, 700])
def test_fp32_forward(N, d, causal):
    PT.run_small(1, 2, 1, N, d, "fp32", causal, seed=N + d, backward=False)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,density,seed", [(300, 64, 0.5, 1), (700, 128, 0.3, 2), (1100, 32, 0.25, 3),
                                              (1024, 64, 0.6, 4)])
def test_block_sparse(N, d, density, seed, causal, dtype):
    m = I.random_block_mask(N, density, seed, keep_diagonal=True)
    PT.run_small(1, 4, 2, N, d, dtype, causal, mask=m, seed=seed)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_empty_rows(dtype):
    """A block row of zeros: those queries see no key -> O = 0, LSE = -inf, zero dq."""
    N = 400
    m = np.ones((4, 4), dtype=np.uint8)
    m[1, :] = 0
    m[3, 3] = 0
    m[3, 0] = 0
    res = PT.run_small(1, 2, 1, N, 64, dtype, False, mask=m, seed=9, backward=True)
    assert res["o"] <= (PT.TOL_F32 if dtype == "fp32" else PT.TOL_16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", ["64", "32"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_late_dominant_scores(dtype, causal, rows, d):
    """Keys far into the sequence whose scores exceed every earlier one by far
    more than the forward's fixed-reference range (keys 400..410: about 90 in
    log2 units above the first tile's maximum, forcing a restart with lazy
    rescaling) or its rescale slack (key 350: about 46 above). The large keys
    keep their random part: with identical key rows the exact dQ of every row
    that attends to them would be zero (the dS of a row sums to zero), and any
    rounding of dS would make the relative error meaningless. At d = 128 (the
    split-role forward with 64 rows) the same offsets lift the scores further,
    past float32's range relative to the first tile's maximum: the restart
    must also discard the infinite sums."""
    N = 600
    x = I.make_small(1, 2, 1, N, d, dtype, 21)
    x["q"] = x["q"] + 1.0
    x["k"][:, :, 400:411, :] += 8.0
    x["k"][:, :, 350, :] += 4.0
    # LSE reaches about 65 here, where one float32 ulp is 7.6e-6: the absolute
    # 1e-5 bar is below what a float32 result can resolve, so this case allows
    # 4 ulps of the largest LSE on top of it
    q, k = (PT.np64(x[n]) for n in ("q", "k"))
    big = float(np.abs(q @ np.swapaxes(k, -1, -2)).max()) / np.sqrt(d)
    tol = PT.TOL_LSE + 4 * 2.0 ** -23 * big
    PT.run_given(x, dtype, causal, where=f"late dominant scores {dtype} causal={causal}", lse_tol=tol,
                 rows_per_wave=int(rows))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", ["64", "32"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("boost,rate", [(2.0, 0.0), (4.0, 0.0), (4.0, 0.5)])
def test_moderately_late_dominant_scores(dtype, boost, rate, rows, d):
    """One key far into the sequence whose score exceeds the first tile's
    maximum by about 23 (boost 2) or 46 (boost 4) in log2 units: inside the
    fixed-reference range of the 64-row kernel's main loop, so nothing forces
    a restart through the row sums, but relative to that reference its
    probability is above the largest finite float16 (2^16); the 16-bit
    probabilities must not overflow, also once scaled for dropout. (The
    causal 64-row kernel needs at least two full tiles before a workgroup's
    diagonal: N = 600 gives the last workgroups up to 16.) At d = 128 (the
    split-role forward with 64 rows) the same boosts lift the score about 1.4
    times as far, about 33 and 65, where the larger one leaves that range."""
    N = 600
    x = I.make_small(1, 2, 1, N, d, dtype, 23)
    x["q"] = x["q"] + 1.0
    x["k"][:, :, 350, :] += boost
    q, k = (PT.np64(x[n]) for n in ("q", "k"))
    big = float(np.abs(q @ np.swapaxes(k, -1, -2)).max()) / np.sqrt(d)
    tol = PT.TOL_LSE + 4 * 2.0 ** -23 * big
    PT.run_given(x, dtype, True, where=f"moderately late dominant score {dtype} boost={boost} dropout={rate}",
                 lse_tol=tol, dropout_rate=rate, drop_seed=5, rows_per_wave=int(rows))


DROP_SHAPES = [(1, 2, 1, 17, 32), (2, 2, 2, 64, 64), (1, 3, 1, 127, 128), (1, 4, 2, 300, 64),
               (1, 2, 2, 513, 128)]


@pytest.mark.parametrize("rows", ["64", "32"])
@pytest.mark.parametrize("rate", [0.1, 0.5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DROP_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dropout(shape, causal, rate, rows):
    """Dropout fused into every 16-bit kernel: O, LSE and gradients against the
    oracle drawing the same Philox keep decisions (both forward kernels)."""
    B, H, Hkv, N, d = shape
    dtype = "bf16" if N % 2 else "fp16"
    PT.run_small(B, H, Hkv, N, d, dtype, causal, seed=7000 + N + d, dropout_rate=rate,
                 drop_seed=(0x123456789 * (N + 1)) & (2**64 - 1), rows_per_wave=int(rows))


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_block_sparse(causal):
    m = I.random_block_mask(700, 0.5, 3, keep_diagonal=True)
    PT.run_small(1, 4, 2, 700, 64, "bf16", causal, mask=m, seed=31, dropout_rate=0.25, drop_seed=99)


def test_dropout_seed_determinism(gpu_lib):
    """Same seed, same result bit for bit; another seed, other decisions; a rate
    that rounds to no dropout equals the plain kernels."""
    x = I.make_small(1, 2, 2, 300, 64, "bf16", 41)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o1, l1 = gpu_lib.forward(q, k, v, None, True, dropout_rate=0.3, seed=5)
    o2, l2 = gpu_lib.forward(q, k, v, None, True, dropout_rate=0.3, seed=5)
    o3, _ = gpu_lib.forward(q, k, v, None, True, dropout_rate=0.3, seed=6)
    g1 = gpu_lib.backward(q, k, v, o1, l1, do, None, True, dropout_rate=0.3, seed=5)
    g2 = gpu_lib.backward(q, k, v, o2, l2, do, None, True, dropout_rate=0.3, seed=5)
    o0, l0 = gpu_lib.forward(q, k, v, None, True)
    oz, lz = gpu_lib.forward(q, k, v, None, True, dropout_rate=0.001, seed=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    assert not torch.equal(o1, o3)
    assert torch.equal(l1, l0)                      # LSE is that of the undropped scores
    assert torch.equal(oz, o0) and torch.equal(lz, l0)


def test_scale_zero_is_uniform():
    PT.run_small(1, 2, 2, 200, 64, "bf16", True, seed=5, scale=0.0)
    PT.run_small(1, 1, 1, 150, 32, "fp32", False, seed=6, scale=0.0, backward=False)


def test_forward_bitwise_deterministic(gpu_lib):
    x = I.make_small(1, 4, 2, 1000, 128, "bf16", 11, with_grad=False)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = gpu_lib.forward(q, k, v, None, True)
    o2, l2 = gpu_lib.forward(q, k, v, None, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal,N,rate", [(False, 1100, 0.0), (True, 4200, 0.0), (False, 1100, 0.2)])
def test_split_role_kernels_bitwise_repeatable(gpu_lib, causal, N, rate):
    """At head size 128 the long-row forward and the key-block backward hand
    probabilities from producer to consumer waves through LDS: two runs on the
    same inputs agree bit for bit (a missed wait on that hand-over would show
    here as run-to-run differences)."""
    B, H, Hkv, d = 1, 2, 1, 128
    x = I.make_small(B, H, Hkv, N, d, "bf16", 13)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    PT.say(f"split-role repeatability causal={causal} N={N} rate={rate}")
    runs = []
    for _ in range(2):
        o, lse = gpu_lib.forward(q, k, v, None, causal, dropout_rate=rate, seed=3, rows_per_wave=64)
        g = gpu_lib.backward(q, k, v, o, lse, do, None, causal, dropout_rate=rate, seed=3)
        runs.append((o, lse) + tuple(g))
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,H,N,causal", [(1, 2, 1024, False), (64, 16, 512, False), (1, 4, 16384, True)])
def test_default_kernel_is_the_reported_one(gpu_lib, B, H, N, causal):
    """A forward call without a forced kernel runs the one
    fa_forward_kernel_rows names (bench.py credits that kernel): its output is
    bitwise that of the same call forced to it, and differs from the other
    kernel's (the two round differently)."""
    d = 128
    rows = gpu_lib.forward_kernel_rows(B, H, H, N, N, d, causal)
    assert rows in (32, 64)
    g = torch.Generator().manual_seed(B * 1000 + N)
    q, k, v = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    o0, l0 = gpu_lib.forward(q, k, v, None, causal)
    o1, l1 = gpu_lib.forward(q, k, v, None, causal, rows_per_wave=rows)
    o2, _ = gpu_lib.forward(q, k, v, None, causal, rows_per_wave=96 - rows)
    torch.cuda.synchronize()
    PT.say(f"default kernel B={B} H={H} N={N} causal={causal}: {rows} rows")
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert not torch.equal(o0, o2)


def test_forward_allocates_nothing(gpu_lib):
    """With caller-owned outputs the library takes no device memory (O(N) memory:
    only O and LSE are written)."""
    x = I.make_small(1, 2, 2, 2048, 64, "bf16", 12, with_grad=False)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    before = torch.cuda.memory_allocated()
    gpu_lib.forward(q, k, v, None, True, out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == before
    assert free1 == free0


def test_noncontiguous_rejected(gpu_lib):
    x = I.make_small(1, 2, 2, 64, 64, "bf16", 13, with_grad=False)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    with pytest.raises(ValueError):
        gpu_lib.forward(q.transpose(1, 2), k, v)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 2, 777, 64), (1, 3, 1, 300, 32), (3, 2, 2, 1029, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_backward_one_launch_equals_two(gpu_lib, shape, causal):
    """Stage 3 (the dK/dV and dQ kernels in one launch, what fa_backward runs
    for d <= 64 without a block mask) gives the very bits stages 1 and 2 give:
    the same code per workgroup, no atomics."""
    B, H, Hkv, N, d = shape
    x = I.make_small(B, H, Hkv, N, d, "bf16", 51)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.forward(q, k, v, None, causal)
    ws = gpu_lib.workspace(q, k)
    two = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    one = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    for stage in (0, 1, 2):
        gpu_lib.backward_stage(stage, q, k, v, o, lse, do, *two, ws, None, causal)
    for stage in (0, 3):
        gpu_lib.backward_stage(stage, q, k, v, o, lse, do, *one, ws, None, causal)
    full = gpu_lib.backward(q, k, v, o, lse, do, None, causal)
    torch.cuda.synchronize()
    for a, b, c in zip(two, one, full):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b) and torch.equal(b, c)
