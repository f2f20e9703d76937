"""Seeded synthetic inputs for the attention workloads (no attention arithmetic here).

This module only draws random numbers, rounds them to the storage dtype and
builds block masks. Both the HIP path (tests, bench) and the float64 oracle
consume what it returns; it holds none of the method's arithmetic.

The workloads stand in for the ones the pages measure on (GPT-2 and
long-range-arena training in the nadeemcite summary, "Summary"); those need
models and datasets, so the inputs here are i.i.d. normal draws with the
pages' shapes instead:

* ``single_head_fp32`` is the lesson's worked example ("FlashAttention" lesson,
  Developer tier, flash_numpy.py): one head, N=512, d=32, float32 draws from
  ``numpy.random.default_rng(0)`` in the order Q, K, V.
* the others draw Q, K, V (and the upstream gradient dO when a backward pass
  is timed) in that order, each with C-order shape [B, H or Hkv, N, d], as
  float32 normals from ``default_rng(seed)``, then round to the storage dtype
  with round-to-nearest-even.
"""

from dataclasses import dataclass, field
import math

import numpy as np

MASK_BLOCK = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    dtype: str            # "fp32", "bf16" or "fp16"
    causal: bool
    seed: int
    backward: bool
    sigma: float = 1.0
    sparse: bool = False  # band of 4 diagonal blocks plus 5% random off-band blocks
    check_heads: int = 0  # 0 = every (b, h); k > 0 = k seeded heads of batch 0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def G(self) -> int:
        return self.H // self.Hkv


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_fp32", 1, 1, 1, 512, 32, "fp32", False, 0, False,
                 note="the lesson's worked example, forward only"),
        Workload("gpt2_small_bf16", 8, 12, 12, 1024, 64, "bf16", True, 2, True,
                 note="GPT-2-small attention shape, causal"),
        Workload("long_seq_bf16", 1, 16, 16, 16384, 128, "bf16", True, 3, True, check_heads=2,
                 note="long-sequence causal attention, the throughput workload"),
        Workload("gqa_bf16", 4, 32, 8, 8192, 128, "bf16", True, 4, False,
                 note="grouped-query attention, group of 4, forward only"),
        Workload("block_sparse_fp16", 1, 8, 8, 65536, 64, "fp16", False, 5, True, sigma=0.5,
                 sparse=True, check_heads=1,
                 note="128x128 block mask: band of 4 diagonal blocks + 5% random off-band"),
    ]
}


def _torch_dtype(name):
    import torch
    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[name]


def draw(shape, rng, sigma=1.0):
    """float32 normal draws N(0, sigma) of the given C-order shape."""
    return rng.normal(0.0, sigma, size=shape).astype(np.float32)


def round_to(x, dtype):
    """Round a float32 numpy array to the storage dtype (RNE), as a CPU torch tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(_torch_dtype(dtype))


def band_plus_random_mask(n, seed, band=4, frac=0.05, block=MASK_BLOCK):
    """uint8 [nb, nb] block mask: blocks (I, J) with I-band < J <= I, plus
    round(frac * #off-band) off-band blocks drawn uniformly without replacement
    from ``default_rng(seed)``."""
    nb = -(-n // block)
    m = np.zeros((nb, nb), dtype=np.uint8)
    ii, jj = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    in_band = (jj <= ii) & (jj > ii - band)
    m[in_band] = 1
    off = np.flatnonzero(~in_band.ravel())
    k = int(round(frac * off.size))
    pick = np.random.default_rng(seed).choice(off.size, size=k, replace=False)
    m.ravel()[off[pick]] = 1
    return m


def check_heads(w: Workload):
    """The (b, h) pairs the oracle checks fully for a workload."""
    if w.check_heads == 0:
        return [(b, h) for b in range(w.B) for h in range(w.H)]
    hs = np.random.default_rng(w.seed + 100).choice(w.H, size=w.check_heads, replace=False)
    return [(0, int(h)) for h in sorted(hs)]


def make(w: Workload, with_grad=None):
    """Inputs of a workload as CPU torch tensors in the storage dtype.

    Returns a dict with q, k, v, (do), mask (uint8 numpy array or None).
    """
    rng = np.random.default_rng(w.seed)
    out = {}
    qs = (w.B, w.H, w.N, w.d)
    ks = (w.B, w.Hkv, w.N, w.d)
    out["q"] = round_to(draw(qs, rng, w.sigma), w.dtype)
    out["k"] = round_to(draw(ks, rng, w.sigma), w.dtype)
    out["v"] = round_to(draw(ks, rng, w.sigma), w.dtype)
    if w.backward if with_grad is None else with_grad:
        out["do"] = round_to(draw(qs, rng, w.sigma), w.dtype)
    out["mask"] = band_plus_random_mask(w.N, w.seed + 200) if w.sparse else None
    return out


def make_small(B, H, Hkv, N, d, dtype, seed, sigma=1.0, with_grad=True):
    """Small seeded inputs of any shape (same recipe), as CPU torch tensors."""
    rng = np.random.default_rng(seed)
    out = {
        "q": round_to(draw((B, H, N, d), rng, sigma), dtype),
        "k": round_to(draw((B, Hkv, N, d), rng, sigma), dtype),
        "v": round_to(draw((B, Hkv, N, d), rng, sigma), dtype),
    }
    if with_grad:
        out["do"] = round_to(draw((B, H, N, d), rng, sigma), dtype)
    return out


def make_on_device(B, H, Hkv, N, d, dtype, seed, device, sigma=1.0, with_grad=True):
    """Seeded inputs too large to draw on the host (sequences near the length
    limit): q, k, v (and do) drawn in that order as float32 normals N(0, sigma)
    by torch's generator on ``device`` seeded with ``seed``, then rounded to the
    storage dtype (RNE). Tests hand slices of the same tensors to the oracle."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = _torch_dtype(dtype)

    def one(shape):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma).to(dt)

    out = {"q": one((B, H, N, d)), "k": one((B, Hkv, N, d)), "v": one((B, Hkv, N, d))}
    if with_grad:
        out["do"] = one((B, H, N, d))
    return out


def random_block_mask(n, density, seed, block=MASK_BLOCK, keep_diagonal=False, n_keys=None):
    """uint8 [ceil(n / block), ceil(n_keys / block)] mask with i.i.d.
    Bernoulli(density) blocks (for small tests); n_keys defaults to n."""
    nb = -(-n // block)
    nbk = nb if n_keys is None else -(-n_keys // block)
    m = (np.random.default_rng(seed).random((nb, nbk)) < density).astype(np.uint8)
    if keep_diagonal:
        np.fill_diagonal(m, 1)
    return m


def make_cross(B, H, Hkv, Nq, Nk, d, dtype, seed, sigma=1.0, with_grad=True):
    """Seeded inputs with Nq query rows and Nk keys (same recipe as ``make_small``):
    q, do [B, H, Nq, d]; k, v [B, Hkv, Nk, d]."""
    rng = np.random.default_rng(seed)
    out = {
        "q": round_to(draw((B, H, Nq, d), rng, sigma), dtype),
        "k": round_to(draw((B, Hkv, Nk, d), rng, sigma), dtype),
        "v": round_to(draw((B, Hkv, Nk, d), rng, sigma), dtype),
    }
    if with_grad:
        out["do"] = round_to(draw((B, H, Nq, d), rng, sigma), dtype)
    return out


def offsets(lengths):
    """int32 [len + 1] running offsets 0, l0, l0 + l1, ... of a list of lengths."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def make_packed(lens_q, lens_k, H, Hkv, d, dtype, seed, sigma=1.0, with_grad=True):
    """Seeded packed variable-length inputs: sequence b has lens_q[b] query rows
    and lens_k[b] keys, stored one after another per head (q, do [H, Tq, d];
    k, v [Hkv, Tk, d]); also returns the offsets cu_q, cu_k (int32 numpy)."""
    rng = np.random.default_rng(seed)
    cu_q, cu_k = offsets(lens_q), offsets(lens_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    out = {
        "q": round_to(draw((H, tq, d), rng, sigma), dtype),
        "k": round_to(draw((Hkv, tk, d), rng, sigma), dtype),
        "v": round_to(draw((Hkv, tk, d), rng, sigma), dtype),
        "cu_q": cu_q,
        "cu_k": cu_k,
    }
    if with_grad:
        out["do"] = round_to(draw((H, tq, d), rng, sigma), dtype)
    return out


def geometric_slopes(H):
    """ALiBi's slope set for H heads (Press, Smith and Lewis, 2022): the
    geometric sequence 2^(-8 (h + 1) / H), h = 0 .. H - 1, float32 values."""
    return (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)


def random_slopes(H, seed, hi=1.0):
    """Seeded ALiBi slopes uniform in [0, hi), float32 (steeper and flatter
    than the geometric set, to reach the distance bias's extremes)."""
    return np.random.default_rng(seed).uniform(0.0, hi, size=H).astype(np.float32)


def length_mix(batch, mean, seed, lo=1):
    """A batch of sequence lengths with a document-like spread: lengths drawn
    from an exponential distribution of the given mean, at least lo."""
    x = np.random.default_rng(seed).exponential(mean, size=batch)
    return [max(lo, int(round(v))) for v in x]


def packed_lengths(total, mean, seed):
    """Sequence lengths for a packed batch of ``total`` tokens per head:
    exponential lengths of the given mean (at least 16), drawn until they sum
    to ``total``, the last one trimmed (or merged into its neighbour) so that
    they sum to it exactly."""
    rng = np.random.default_rng(seed)
    out = []
    while sum(out) < total:
        out.append(max(16, int(round(rng.exponential(mean)))))
    out[-1] -= sum(out) - total
    if out[-1] < 1:
        out.pop()
        out[-1] += total - sum(out)
    return out


def quantize_e4m3(x):
    """Per-tensor FP8 (E4M3) quantisation of a float32 numpy array: descale =
    max|x| / 448 (the format's largest finite value), codes = x / descale
    rounded to nearest-even by PyTorch's float8_e4m3fn conversion. Returns
    (uint8 CPU torch tensor of codes, descale)."""
    import torch
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = amax / 448.0 if amax > 0 else 1.0
    codes = torch.from_numpy(np.ascontiguousarray(x / np.float32(descale), dtype=np.float32))
    return codes.to(torch.float8_e4m3fn).view(torch.uint8), descale


def make_fp8(B, H, Hkv, N, d, seed, sigma=1.0):
    """Seeded FP8 inputs: the same normal draws as ``make_small`` (Q, K, V in
    that order), each quantised per tensor with ``quantize_e4m3``. Returns a
    dict with q, k, v (uint8 codes) and q_descale, k_descale, v_descale."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("q", (B, H, N, d)), ("k", (B, Hkv, N, d)), ("v", (B, Hkv, N, d))):
        out[name], out[name + "_descale"] = quantize_e4m3(draw(shape, rng, sigma))
    return out
