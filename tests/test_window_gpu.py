"""GPU parity for sliding-window (band) masks: every output element of the HIP
path against the float64 oracle, for bands narrower than a tile, bands that
end inside a tile, one-sided bands, bands combined with causal masking,
unequal lengths, block masks, packed batches and dropout."""

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


WINDOWS = [(-1, 0), (64, 0), (200, 0), (0, 0), (17, 5), (128, 128), (-1, 64), (300, -1), (33, 700)]
SHAPES = [
    # B, H, Hkv, Nq, Nk, d
    (1, 2, 1, 300, 300, 64),
    (1, 2, 2, 513, 513, 128),
    (2, 2, 1, 100, 400, 64),
    (1, 4, 2, 400, 100, 32),
]


def _seed(*xs):
    return int(sum((i + 3) * 977 * (x + 2) for i, x in enumerate(xs)) % 100003)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", WINDOWS, ids=str)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_window(shape, window, causal):
    B, H, Hkv, Nq, Nk, d = shape
    PT.run_window(B, H, Hkv, Nq, Nk, d, "bf16", causal, window, seed=_seed(*shape, *window, causal))


@pytest.mark.parametrize("rows", ["64", "32"])
@pytest.mark.parametrize("window", WINDOWS, ids=str)
def test_window_forward_kernels(window, rows):
    """Both 16-bit forward kernels, forced through fa_forward_select, over a
    sequence long enough for full tiles inside the band."""
    PT.run_window(1, 2, 1, 1100, 1300, 128, "fp16", False, window, seed=_seed(*window, int(rows)),
                  backward=False, rows_per_wave=int(rows))


@pytest.mark.parametrize("rows", ["64", "32"])
@pytest.mark.parametrize("window", [(600, 0), (500, 100)], ids=str)
def test_window_restart(window, rows):
    """Keys 900..910 whose scores exceed every other by far more than the
    64-row forward's fixed-reference range, under a two-edged band: in the
    256-row workgroups the tiles every row sees in full start well before
    those keys (from key 640 for rows 768..1023 with window (600, 0)), so the
    main loop's row sums overflow and it restarts with lazy rescaling while
    the band's tile order (full tiles, then the partial ones above and below)
    drives its LDS ring (d = 128: the split-role form). The 32-row kernel
    takes the same scores with its lazy reference."""
    Nq, Nk, d = 1100, 1300, 128
    x = I.make_cross(1, 2, 1, Nq, Nk, d, "bf16", _seed(*window, int(rows), 9), with_grad=True)
    x["q"] = x["q"] + 1.0
    x["k"][:, :, 900:911, :] += 8.0
    q, k = (PT.np64(x[n]) for n in ("q", "k"))
    big = float(np.abs(q @ np.swapaxes(k, -1, -2)).max()) / np.sqrt(d)
    PT.run_window(1, 2, 1, Nq, Nk, d, "bf16", False, window, rows_per_wave=int(rows), x=x,
                  lse_tol=PT.TOL_LSE + 4 * 2.0 ** -23 * big)


@pytest.mark.parametrize("window", [(64, 0), (17, 5), (0, 0), (300, -1)], ids=str)
def test_window_fp32(window):
    PT.run_window(1, 2, 1, 200, 260, 32, "fp32", False, window, seed=_seed(*window, 5), backward=False)


@pytest.mark.parametrize("window", [(150, 0), (40, 40)], ids=str)
def test_window_block_sparse(window):
    mask = I.random_block_mask(700, 0.6, _seed(*window), n_keys=700)
    PT.run_window(1, 2, 1, 700, 700, 64, "bf16", True, window, mask=mask, seed=_seed(*window, 1))


@pytest.mark.parametrize("window", [(64, 0), (20, 20)], ids=str)
def test_window_varlen(window):
    PT.run_varlen([5, 300, 1, 257], [40, 300, 9, 129], 2, 1, 64, "bf16", True, seed=_seed(*window, 2),
                  window=window)


@pytest.mark.parametrize("rows", ["0", "64"])
@pytest.mark.parametrize("window,causal", [((100, 0), True), ((150, 60), False)], ids=str)
def test_window_dropout(window, causal, rows):
    """Dropout under a band; rows 64 forces the split-role forward at d = 128,
    whose keep decisions follow the band's tile order."""
    PT.run_window(1, 2, 2, 300, 400, 128, "bf16", causal, window, seed=71, dropout_rate=0.2, drop_seed=72,
                  rows_per_wave=int(rows))


def test_window_large_sampled():
    """Sliding-window causal attention at the throughput workload's size
    (N = 16384, d = 128, 16 heads, band of 4096 keys): one head's sampled rows
    and its full gradients against the oracle."""
    B, H, N, d = 1, 16, 16384, 128
    window = (4095, 0)
    x = I.make_small(B, H, H, N, d, "bf16", 81)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = binding.forward(q, k, v, scale, True, window=window)
    dq, dk, dv = binding.backward(q, k, v, o, lse, do, scale, True, window=window)
    torch.cuda.synchronize()
    h = 9
    rows = np.sort(np.random.default_rng(82).choice(N, size=64, replace=False))
    qd, kd, vd = (PT.np64(x[n][:, h:h + 1]) for n in ("q", "k", "v"))
    oref, lref = oracle.forward(qd, kd, vd, scale, True, rows=rows, window=window)
    PT.check_out(PT.np64(o[:, h:h + 1, rows]), oref, "bf16", "large window forward")
    PT.check_lse(PT.np64(lse[:, h:h + 1, rows]), lref, "large window lse")
    rq, rk, rv = oracle.backward(qd, kd, vd, PT.np64(x["do"][:, h:h + 1]), scale, True, window=window)
    PT.check_grad(PT.np64(dq[:, h:h + 1]), rq, "large window dq")
    PT.check_grad(PT.np64(dk[:, h:h + 1]), rk, "large window dk")
    PT.check_grad(PT.np64(dv[:, h:h + 1]), rv, "large window dv")
