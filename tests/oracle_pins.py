"""Checks that pin the float64 oracle to facts that do not come from the oracle.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix. ``test_oracle.py`` runs them on the
oracle as written; ``test_oracle_mutants.py`` plants plausible mistakes in the
oracle (on the CPU) and checks that at least one pin fails for each.

Sources, by page and section:
* worked example: "FlashAttention" lesson (learn.pranaymahendrakar.com),
  Developer tier, flash_numpy.py and its printed Output;
* the online-softmax recurrence: same lesson, Researcher tier, "Online softmax"
  (the equations for m, l and O and the final O / l);
* O = softmax(Q K^T / sqrt(d)) V: same lesson, Researcher tier, "The problem
  being solved";
* causal = earlier words only: same lesson, Beginner tier, "What was broken
  before"; block-sparse: nadeemcite summary, Key Method Details;
* grouped-query attention: the lesson's related-term card "Grouped-query
  attention".
"""

import json
import math
import os

import numpy as np

import oracle.attention as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


# ----------------------------------------------------------------------------------------------
# P-1: the lesson's worked example (this is the single-head fp32 workload)
# ----------------------------------------------------------------------------------------------
def page_inputs():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    rng = np.random.default_rng(g["inputs"]["seed"])
    n, d = g["N"], g["d"]
    q = rng.normal(size=(n, d)).astype(np.float32)
    k = rng.normal(size=(n, d)).astype(np.float32)
    v = rng.normal(size=(n, d)).astype(np.float32)
    return g, q, k, v


def fp32_tiled_recurrence(q, k, v, scale, tile):
    """The lesson's streaming update evaluated in float32, one key tile at a time.

    Running max m, running sum of exponentials l and running unnormalised
    output O; each tile rescales l and O by exp(m_old - m_new) before adding
    its own terms; the result is O / l.
    """
    n = q.shape[0]
    o = np.zeros_like(q)
    m = np.full(n, -np.inf, dtype=np.float32)
    l = np.zeros(n, dtype=np.float32)
    for j in range(0, k.shape[0], tile):
        s = (q @ k[j:j + tile].T) * scale
        m_new = np.maximum(m, s.max(axis=1))
        c = np.exp(m - m_new)
        p = np.exp(s - m_new[:, None])
        l = c * l + p.sum(axis=1)
        o = c[:, None] * o + p @ v[j:j + tile]
        m = m_new
    return o / l[:, None]


def pin_worked_example():
    g, q, k, v = page_inputs()
    pr = g["printed"]
    n, d, tile = g["N"], g["d"], g["key_tile"]
    # the shapes the page printed its buffer sizes for
    assert n * n * 4 == pr["naive_score_bytes"]
    assert n * tile * 4 == pr["tile_score_bytes"]
    assert pr["naive_score_bytes"] // pr["tile_score_bytes"] == pr["ratio"]
    for s, gb in pr["bf16_full_score_GB"].items():
        assert round(int(s) ** 2 * 2 / 1e9, 2) == gb
    scale = np.float32(1.0 / np.sqrt(d))      # float32 scale, as under NumPy 1.x
    o64, lse = A.forward(q[None, None].astype(np.float64), k[None, None].astype(np.float64),
                         v[None, None].astype(np.float64), float(scale))
    o32 = fp32_tiled_recurrence(q, k, v, scale, tile)
    diff = float(np.abs(o32 - o64[0, 0]).max())
    # the page: allclose at 1e-5, largest difference of order 2.4e-7 (float32 rounding)
    assert diff <= pr["outputs_match_allclose_atol"], diff
    assert diff <= 10 * pr["largest_absolute_difference"], diff
    assert np.all(np.isfinite(lse))


# ----------------------------------------------------------------------------------------------
# P-2: the streaming recurrence in float64 equals the definition for every key-tile width
# ----------------------------------------------------------------------------------------------
def recurrence64(q, k, v, scale, tile, causal=False, block_mask=None, block=128):
    """The lesson's online-softmax equations in float64, with -inf for invisible keys.

    A tile that leaves a row's running max at -inf contributes nothing; the
    guard keeps exp(-inf - (-inf)) out of the arithmetic. Returns O / l and
    the log-sum-exp m + ln l.
    """
    n = q.shape[0]
    ii = np.arange(n)[:, None]
    o = np.zeros_like(q)
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    for j in range(0, k.shape[0], tile):
        jj = np.arange(j, min(j + tile, k.shape[0]))[None, :]
        s = (q @ k[j:j + tile].T) * scale
        ok = np.ones(s.shape, dtype=bool)
        if causal:
            ok &= jj <= ii
        if block_mask is not None:
            ok &= np.asarray(block_mask)[ii // block, jj // block] != 0
        s = np.where(ok, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        live = np.isfinite(m_new)
        ref = np.where(live, m_new, 0.0)
        c = np.where(live, np.exp(m - ref), 1.0)
        p = np.exp(s - ref[:, None])
        l = c * l + p.sum(axis=1)
        o = c[:, None] * o + p @ v[j:j + tile]
        m = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(l[:, None] > 0, o / np.where(l > 0, l, 1)[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1)), -np.inf)
    return out, lse


def pin_recurrence():
    n, d = 300, 8
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    for causal, bm in [(False, None), (True, None), (False, mask), (True, mask)]:
        o_ref, l_ref = A.forward(q[None, None], k[None, None], v[None, None], 0.3, causal, bm)
        for tile in (1, 16, 128, 512):
            o, l_ = recurrence64(q, k, v, 0.3, tile, causal, bm)
            assert np.abs(o - o_ref[0, 0]).max() <= 1e-12, (causal, tile)
            assert np.abs(l_ - l_ref[0, 0]).max() <= 1e-12, (causal, tile)


# ----------------------------------------------------------------------------------------------
# P-3: brute force with scalar loops on tiny inputs, and the two-key closed form
# ----------------------------------------------------------------------------------------------
def brute_force(q, k, v, scale, causal):
    """Scalar loops. With fewer queries than keys the queries are the last
    positions of the sequence: query i stands at position i + len(k) - len(q)
    and, under causal masking, sees the keys at or before that position."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    outs, lses = [], []
    for i in range(n):
        pos = i + len(k) - n
        keys = [j for j in range(len(k)) if (not causal or j <= pos)]
        if not keys:
            outs.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        sc = [scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        mx = max(sc)
        w = [math.exp(s - mx) for s in sc]
        z = sum(w)
        outs.append([sum(w[a] * v[j][t] for a, j in enumerate(keys)) / z for t in range(dv)])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


def pin_brute_force():
    seed = 10
    for n in (1, 2, 3, 4):
        for d in (1, 2, 3):
            for causal in (False, True):
                seed += 1
                q, k, v = _rand((n, d), seed), _rand((n, d), seed + 100), _rand((n, d), seed + 200)
                o, l_ = A.forward(q[None, None], k[None, None], v[None, None], 0.7, causal)
                ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
                assert np.abs(o[0, 0] - ob).max() <= 1e-12, (n, d, causal)
                assert np.abs(l_[0, 0] - lb).max() <= 1e-12, (n, d, causal)
    # two keys: o_0 = sigma(s00 - s01) v_0 + (1 - sigma) v_1, L = log(e^s00 + e^s01)
    q, k, v = _rand((2, 3), 77), _rand((2, 3), 78), _rand((2, 3), 79)
    o, l_ = A.forward(q[None, None], k[None, None], v[None, None], 0.5)
    s00, s01 = 0.5 * q[0] @ k[0], 0.5 * q[0] @ k[1]
    sig = 1.0 / (1.0 + math.exp(-(s00 - s01)))
    assert np.abs(o[0, 0, 0] - (sig * v[0] + (1 - sig) * v[1])).max() <= 1e-14
    assert abs(l_[0, 0, 0] - math.log(math.exp(s00) + math.exp(s01))) <= 1e-14


# ----------------------------------------------------------------------------------------------
# P-4: probability rows sum to one; invisible keys carry exactly zero
# ----------------------------------------------------------------------------------------------
def pin_rows_sum_to_one():
    n, d = 260, 8
    q, k = _rand((n, d), 5), _rand((n, d), 6)
    mask = np.array([[1, 0, 0], [1, 1, 0], [1, 0, 1]], dtype=np.uint8)
    for causal, bm in [(False, None), (True, None), (False, mask), (True, mask)]:
        p, _ = A.head_probabilities(q, k, 0.4, causal, bm)
        assert np.abs(p.sum(axis=1) - 1).max() <= 1e-14
        vis = A.visible(np.arange(n), np.arange(n), causal, bm)
        assert np.all(p[~vis] == 0)
        assert np.all(p[vis] > 0)


# ----------------------------------------------------------------------------------------------
# P-5: Q = 0 gives the mean of the visible values and L = ln(#visible)
# ----------------------------------------------------------------------------------------------
def pin_zero_query():
    n, d = 300, 4
    q = np.zeros((n, d))
    k, v = _rand((n, d), 8), _rand((n, d), 9)
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], dtype=np.uint8)
    for causal, bm in [(False, None), (True, None), (False, mask), (True, mask)]:
        o, l_ = A.forward(q[None, None], k[None, None], v[None, None], 0.5, causal, bm)
        for i in range(n):
            keys = [j for j in range(n) if (not causal or j <= i)
                    and (bm is None or bm[i // 128][j // 128])]
            assert np.abs(o[0, 0, i] - v[keys].mean(axis=0)).max() <= 1e-13
            assert abs(l_[0, 0, i] - math.log(len(keys))) <= 1e-13
    # causal, dense: row i is the prefix mean
    o, _ = A.forward(q[None, None], k[None, None], v[None, None], 0.5, True)
    pref = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.abs(o[0, 0] - pref).max() <= 1e-13


# ----------------------------------------------------------------------------------------------
# P-6: one dominant score drags the output row onto that key's value row
# ----------------------------------------------------------------------------------------------
def pin_dominant_score():
    n, d = 64, 16
    q, k, v = _rand((n, d), 11), _rand((n, d), 12), _rand((n, d), 13)
    scale = 0.25
    for i, jstar, c in [(5, 40, 3.0), (20, 3, 6.0), (63, 0, 10.0)]:
        kk = k.copy()
        kk[jstar] = c * q[i]
        s = scale * (q[i] @ kk.T)
        gap = s[jstar] - np.max(np.delete(s, jstar))
        assert gap > 2
        o, _ = A.forward(q[None, None], kk[None, None], v[None, None], scale)
        bound = 2 * (n - 1) * math.exp(-gap) * np.abs(v).max()
        assert np.abs(o[0, 0, i] - v[jstar]).max() <= bound


# ----------------------------------------------------------------------------------------------
# P-7: permutation equivariance (non-causal, dense)
# ----------------------------------------------------------------------------------------------
def pin_permutation():
    n, d = 200, 8
    q, k, v, g = (_rand((1, 1, n, d), s) for s in (21, 22, 23, 24))
    perm = np.random.default_rng(25).permutation(n)
    o, l_ = A.forward(q, k, v, 0.3)
    dq, dk, dv = A.backward(q, k, v, g, 0.3)
    o2, l2 = A.forward(q, k[:, :, perm], v[:, :, perm], 0.3)
    assert np.abs(o2 - o).max() <= 1e-13 and np.abs(l2 - l_).max() <= 1e-13
    dq2, dk2, dv2 = A.backward(q, k[:, :, perm], v[:, :, perm], g, 0.3)
    assert np.abs(dq2 - dq).max() <= 1e-13
    assert np.abs(dk2 - dk[:, :, perm]).max() <= 1e-13
    assert np.abs(dv2 - dv[:, :, perm]).max() <= 1e-13
    o3, l3 = A.forward(q[:, :, perm], k, v, 0.3)
    assert np.abs(o3 - o[:, :, perm]).max() <= 1e-13 and np.abs(l3 - l_[:, :, perm]).max() <= 1e-13
    dq3, dk3, dv3 = A.backward(q[:, :, perm], k, v, g[:, :, perm], 0.3)
    assert np.abs(dq3 - dq[:, :, perm]).max() <= 1e-13
    assert np.abs(dk3 - dk).max() <= 1e-13 and np.abs(dv3 - dv).max() <= 1e-13


# ----------------------------------------------------------------------------------------------
# P-8: causal rows depend only on earlier keys; row 0 sees only key 0
# ----------------------------------------------------------------------------------------------
def pin_causal_locality():
    n, d = 300, 8
    q, k, v = (_rand((1, 1, n, d), s) for s in (31, 32, 33))
    o, l_ = A.forward(q, k, v, 0.5, True)
    for i0 in (0, 17, 127, 128, 250):
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, i0 + 1:] += _rand((n - i0 - 1, d), i0)
        v2[0, 0, i0 + 1:] -= 3.0
        o2, l2 = A.forward(q, k2, v2, 0.5, True)
        assert np.array_equal(o2[0, 0, :i0 + 1], o[0, 0, :i0 + 1])
        assert np.array_equal(l2[0, 0, :i0 + 1], l_[0, 0, :i0 + 1])
    assert np.abs(o[0, 0, 0] - v[0, 0, 0]).max() <= 1e-15
    assert abs(l_[0, 0, 0] - 0.5 * q[0, 0, 0] @ k[0, 0, 0]) <= 1e-14


# ----------------------------------------------------------------------------------------------
# P-9: analytic gradients against central finite differences of f = sum(O * dO)
# ----------------------------------------------------------------------------------------------
def _fd_case(B, H, Hkv, n, d, causal, bm, seed, ncoord=24, h=1e-6, rate=0.0, nk=None):
    nk = n if nk is None else nk
    q = _rand((B, H, n, d), seed)
    k = _rand((B, Hkv, nk, d), seed + 1)
    v = _rand((B, Hkv, nk, d), seed + 2)
    g = _rand((B, H, n, d), seed + 3)
    scale = 0.6
    drop_seed = 1234567 + seed  # a fixed keep mask: the output is then differentiable

    def f(q_, k_, v_):
        o, _ = A.forward(q_, k_, v_, scale, causal, bm, dropout_rate=rate, seed=drop_seed)
        return float((o * g).sum())

    grads = A.backward(q, k, v, g, scale, causal, bm, dropout_rate=rate, seed=drop_seed)
    rng = np.random.default_rng(seed + 4)
    for which, x in enumerate((q, k, v)):
        num, ana = [], []
        for flat in rng.choice(x.size, size=min(ncoord, x.size), replace=False):
            idx = np.unravel_index(flat, x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num.append((f(*args_p) - f(*args_m)) / (2 * h))
            ana.append(grads[which][idx])
        num, ana = np.array(num), np.array(ana)
        err = np.abs(num - ana).max() / max(np.abs(ana).max(), 1e-3)
        assert err <= 1e-6, ("qkv"[which], err)


def pin_finite_differences():
    _fd_case(1, 1, 1, 12, 4, False, None, 40)
    _fd_case(1, 2, 2, 12, 4, True, None, 50)
    _fd_case(2, 4, 2, 10, 3, True, None, 60)                       # grouped-query
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    _fd_case(1, 2, 1, 140, 2, False, mask, 70, ncoord=16)          # block mask, 2 blocks


# ----------------------------------------------------------------------------------------------
# P-10: grouped-query attention equals attention with K, V repeated per query head
# ----------------------------------------------------------------------------------------------
def pin_gqa_repeat():
    B, H, Hkv, n, d = 2, 6, 2, 50, 4
    q = _rand((B, H, n, d), 91)
    k, v = _rand((B, Hkv, n, d), 92), _rand((B, Hkv, n, d), 93)
    g = _rand((B, H, n, d), 94)
    G = H // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        o, l_ = A.forward(q, k, v, 0.5, causal)
        o2, l2 = A.forward(q, kr, vr, 0.5, causal)
        assert np.abs(o - o2).max() <= 1e-14 and np.abs(l_ - l2).max() <= 1e-14
        dq, dk, dv = A.backward(q, k, v, g, 0.5, causal)
        dq2, dk2, dv2 = A.backward(q, kr, vr, g, 0.5, causal)
        assert np.abs(dq - dq2).max() <= 1e-13
        assert np.abs(dk - dk2.reshape(B, Hkv, G, n, d).sum(2)).max() <= 1e-13
        assert np.abs(dv - dv2.reshape(B, Hkv, G, n, d).sum(2)).max() <= 1e-13
    # subset API: per-head contributions add up to the full kv-head gradient
    heads = [(b, h) for b in range(B) for h in range(H)]
    dqs, dks, dvs = A.backward(q, k, v, g, 0.5, True, None, heads)
    dq, dk, dv = A.backward(q, k, v, g, 0.5, True)
    for t, (b, h) in enumerate(heads):
        assert np.abs(dqs[t] - dq[b, h]).max() <= 1e-13
    assert np.abs(dks.reshape(B, Hkv, G, n, d).sum(2) - dk).max() <= 1e-13
    assert np.abs(dvs.reshape(B, Hkv, G, n, d).sum(2) - dv).max() <= 1e-13


# ----------------------------------------------------------------------------------------------
# P-11: block-mask semantics
# ----------------------------------------------------------------------------------------------
def pin_mask_semantics():
    n, d = 300, 4
    q, k, v = (_rand((1, 1, n, d), s) for s in (101, 102, 103))
    g = _rand((1, 1, n, d), 104)
    nb = 3
    ones = np.ones((nb, nb), dtype=np.uint8)
    o, l_ = A.forward(q, k, v, 0.5, False)
    o1, l1 = A.forward(q, k, v, 0.5, False, ones)
    assert np.array_equal(o, o1) and np.array_equal(l_, l1)
    tril = np.tril(ones)
    oc, lc = A.forward(q, k, v, 0.5, True)
    oc2, lc2 = A.forward(q, k, v, 0.5, True, tril)
    assert np.array_equal(oc, oc2) and np.array_equal(lc, lc2)
    # against an explicit N x N additive mask built element by element
    from scipy.special import logsumexp, softmax
    bm = np.array([[1, 0, 1], [0, 0, 1], [1, 1, 0]], dtype=np.uint8)
    full = np.zeros((n, n))
    for i in range(n):
        for j in range(n):
            if not bm[i // 128][j // 128]:
                full[i, j] = -np.inf
    s = 0.5 * q[0, 0] @ k[0, 0].T + full
    om, lm = A.forward(q, k, v, 0.5, False, bm)
    assert np.abs(om[0, 0] - softmax(s, axis=1) @ v[0, 0]).max() <= 1e-13
    assert np.abs(lm[0, 0] - logsumexp(s, axis=1)).max() <= 1e-13
    # gradients against the same explicit mask through torch autograd
    import torch
    tq, tk, tv = (torch.tensor(x[0, 0], requires_grad=True) for x in (q, k, v))
    ts = 0.5 * tq @ tk.T + torch.tensor(full)
    to = torch.softmax(ts, dim=1) @ tv
    to.backward(torch.tensor(g[0, 0]))
    dq, dk, dv = A.backward(q, k, v, g, 0.5, False, bm)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a[0, 0] - b.grad.numpy()).max() <= 1e-12


def pin_empty_rows():
    """A row that sees no key: O = 0, L = -inf, zero gradients, no contribution."""
    n, d = 300, 4
    q, k, v, g = (_rand((1, 1, n, d), s) for s in (111, 112, 113, 114))
    bm = np.array([[1, 0, 0], [0, 0, 0], [1, 1, 1]], dtype=np.uint8)   # block row 1 empty
    o, l_ = A.forward(q, k, v, 0.5, False, bm)
    assert np.all(o[0, 0, 128:256] == 0) and np.all(np.isneginf(l_[0, 0, 128:256]))
    assert np.all(np.isfinite(l_[0, 0, :128])) and np.all(np.isfinite(l_[0, 0, 256:]))
    dq, dk, dv = A.backward(q, k, v, g, 0.5, False, bm)
    assert np.all(dq[0, 0, 128:256] == 0)
    g2 = g.copy()
    g2[0, 0, 128:256] = 1e3             # upstream gradient on empty rows must not leak
    dq2, dk2, dv2 = A.backward(q, k, v, g2, 0.5, False, bm)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


# ----------------------------------------------------------------------------------------------
# P-12: scale 0 gives uniform weights
# ----------------------------------------------------------------------------------------------
def pin_scale_zero():
    n, d = 100, 5
    q, k, v = (_rand((1, 1, n, d), s) for s in (121, 122, 123))
    for causal in (False, True):
        o, l_ = A.forward(q, k, v, 0.0, causal)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        ref = np.cumsum(v[0, 0], axis=0) / cnt[:, None] if causal else np.tile(v[0, 0].mean(0), (n, 1))
        assert np.abs(o[0, 0] - ref).max() <= 1e-13
        assert np.abs(l_[0, 0] - np.log(cnt)).max() <= 1e-13


# ----------------------------------------------------------------------------------------------
# Library cross-check: PyTorch's float64 CPU attention (math path) and autograd
# ----------------------------------------------------------------------------------------------
def pin_torch_sdpa():
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, n, d, causal, seed) in [(2, 4, 4, 130, 16, False, 131), (2, 4, 4, 130, 16, True, 132),
                                            (1, 8, 2, 70, 8, True, 133), (1, 3, 1, 33, 32, False, 134)]:
        q, k, v = _rand((B, H, n, d), seed), _rand((B, Hkv, n, d), seed + 1), _rand((B, Hkv, n, d), seed + 2)
        g = _rand((B, H, n, d), seed + 3)
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=Hkv != H)
        to.backward(torch.tensor(g))
        o, l_ = A.forward(q, k, v, scale, causal)
        dq, dk, dv = A.backward(q, k, v, g, scale, causal)
        assert np.abs(o - to.detach().numpy()).max() <= 1e-12
        assert np.abs(dq - tq.grad.numpy()).max() <= 1e-12
        assert np.abs(dk - tk.grad.numpy()).max() <= 1e-12
        assert np.abs(dv - tv.grad.numpy()).max() <= 1e-12
        # log-sum-exp against torch.logsumexp of the masked scaled scores
        G = H // Hkv
        s = torch.tensor(q) @ torch.tensor(np.repeat(k, G, axis=1)).transpose(-1, -2) * scale
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        assert np.abs(l_ - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


# ----------------------------------------------------------------------------------------------
# Dropout (fused into the kernel per the chipfoundryservices.com glossary "flash attention
# algorithm", "Kernel Fusion"; reading and generator in oracle/dropout.py)
# ----------------------------------------------------------------------------------------------
def pin_philox_known_answers():
    """The generator reproduces Philox4x32-10's published known-answer vectors."""
    from oracle import dropout as Dr
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in kat["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["counter"]], dtype=np.uint64)
        key = [int(x, 16) for x in vec["key"]]
        out = Dr.philox4x32(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in vec["output"]], vec


def pin_dropout_statistics():
    """Keep decisions: the rate they realise, uniform bytes, no correlation between
    neighbouring elements, and every (seed, head, row, key) addressed on its own."""
    from oracle import dropout as Dr
    rows, keys = np.arange(256), np.arange(512)
    b0 = Dr.random_bytes(7, 0, rows, keys).astype(np.int64)
    b1 = Dr.random_bytes(7, 1, rows, keys).astype(np.int64)
    allb = np.concatenate([b0.ravel(), b1.ravel()])
    n = allb.size
    hist = np.bincount(allb, minlength=256)
    chi2 = float(((hist - n / 256) ** 2 / (n / 256)).sum())
    assert chi2 < 255 + 6 * math.sqrt(2 * 255), chi2          # 255 degrees of freedom
    for rate in (0.1, 0.3, 0.5, 0.9):
        t = Dr.threshold(rate)
        kept = float((allb >= t).mean())
        p = (256 - t) / 256
        assert abs(kept - p) < 6 * math.sqrt(p * (1 - p) / n), (rate, kept, p)
    z = (b0 >= 128).astype(np.float64) - 0.5
    for a, bb in ((z[:, :-1], z[:, 1:]), (z[:-1], z[1:]), (z[:, :-4], z[:, 4:]), (z[:-4], z[4:])):
        assert abs(float((a * bb).mean())) < 6 * 0.25 / math.sqrt(a.size)
    assert float((b0 == b1).mean()) < 0.01                     # heads draw different streams
    assert float((b0 == Dr.random_bytes(8, 0, rows, keys)).mean()) < 0.01
    # counter addressing: any subset of rows and keys gives the same bytes
    sub = Dr.random_bytes(7, 0, rows[37:101:3], keys[5:300:7])
    assert np.array_equal(sub, b0[37:101:3][:, 5:300:7])
    # quantised rate: t = round(256 rate), keep scale 256 / (256 - t)
    assert Dr.threshold(0.0) == 0 and Dr.threshold(0.5) == 128 and Dr.threshold(0.999) == 255
    assert Dr.keep_scale(0.25) == 256.0 / 192.0


def pin_dropout_expectation():
    """Averaged over seeds, the dropped output equals the output without dropout
    (kept probabilities are rescaled by the inverse keep probability), and the
    saved log-sum-exp is that of the scores before dropout."""
    q, k, v = _rand((1, 1, 6, 3), 501), _rand((1, 1, 6, 3), 502), _rand((1, 1, 6, 3), 503)
    o_ref, l_ref = A.forward(q, k, v, 0.8, True)
    acc = np.zeros_like(o_ref)
    nseed = 3000
    for sd in range(nseed):
        o, l_ = A.forward(q, k, v, 0.8, True, dropout_rate=0.5, seed=sd)
        assert np.array_equal(l_, l_ref)
        acc += o
    # per element the dropped output has variance below max|v|^2 / keep = 2 max|v|^2
    bound = 6 * math.sqrt(2.0) * np.abs(v).max() / math.sqrt(nseed)
    assert np.abs(acc / nseed - o_ref).max() < bound
    # a rate that rounds to t = 0 keeps everything, unscaled
    o0, l0 = A.forward(q, k, v, 0.8, True, dropout_rate=0.001, seed=3)
    assert np.array_equal(o0, o_ref) and np.array_equal(l0, l_ref)


def pin_dropout_finite_differences():
    """With a fixed keep mask the dropped output is a smooth function of q, k, v;
    its analytic gradients match central differences."""
    _fd_case(1, 1, 1, 12, 4, False, None, 140, rate=0.3)
    _fd_case(1, 2, 2, 12, 4, True, None, 150, rate=0.5)
    _fd_case(2, 4, 2, 10, 3, True, None, 160, rate=0.2)


# ----------------------------------------------------------------------------------------------
# P-15: unequal query and key lengths (queries at the end of the sequence, as beside a KV cache)
# ----------------------------------------------------------------------------------------------
def pin_cross_lengths_brute_force():
    seed = 600
    for nq in (1, 2, 3, 5):
        for nk in (1, 2, 4, 6):
            for causal in (False, True):
                seed += 1
                q, k, v = _rand((nq, 3), seed), _rand((nk, 3), seed + 100), _rand((nk, 2), seed + 200)
                o, l_ = A.forward(q[None, None], k[None, None], v[None, None], 0.9, causal)
                ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.9, causal)
                assert np.abs(o[0, 0] - ob).max() <= 1e-12, (nq, nk, causal)
                assert np.array_equal(np.isinf(l_[0, 0]), np.isinf(lb)), (nq, nk, causal)
                fin = np.isfinite(lb)
                assert np.abs(l_[0, 0][fin] - lb[fin]).max(initial=0.0) <= 1e-12, (nq, nk, causal)


def pin_cross_lengths_suffix():
    """Nq < Nk: the result is the last Nq rows of square causal attention whose
    earlier query rows are anything; with dO zero on those rows the key and
    value gradients agree too. Nq > Nk: the first Nq - Nk rows see nothing and
    the rest is square causal attention over all Nk keys."""
    nk, d = 300, 6
    k, v = _rand((1, 1, nk, d), 71), _rand((1, 1, nk, d), 72)
    for nq in (1, 37, 129, 299):
        qf = _rand((1, 1, nk, d), 73 + nq)
        gf = _rand((1, 1, nk, d), 74 + nq)
        gf[:, :, :nk - nq] = 0.0
        q, g = qf[:, :, nk - nq:], gf[:, :, nk - nq:]
        o, l_ = A.forward(q, k, v, 0.4, True)
        of, lf = A.forward(qf, k, v, 0.4, True)
        assert np.abs(o - of[:, :, nk - nq:]).max() <= 1e-13
        assert np.abs(l_ - lf[:, :, nk - nq:]).max() <= 1e-13
        dq, dk, dv = A.backward(q, k, v, g, 0.4, True)
        dqf, dkf, dvf = A.backward(qf, k, v, gf, 0.4, True)
        assert np.abs(dq - dqf[:, :, nk - nq:]).max() <= 1e-12
        assert np.abs(dk - dkf).max() <= 1e-12 and np.abs(dv - dvf).max() <= 1e-12
    # more queries than keys
    nq = 200
    nk2 = 70
    q = _rand((1, 1, nq, d), 81)
    g = _rand((1, 1, nq, d), 82)
    o, l_ = A.forward(q, k[:, :, :nk2], v[:, :, :nk2], 0.4, True)
    assert np.all(o[0, 0, :nq - nk2] == 0) and np.all(l_[0, 0, :nq - nk2] == -np.inf)
    o2, l2 = A.forward(q[:, :, nq - nk2:], k[:, :, :nk2], v[:, :, :nk2], 0.4, True)
    assert np.abs(o[:, :, nq - nk2:] - o2).max() <= 1e-13 and np.abs(l_[:, :, nq - nk2:] - l2).max() <= 1e-13
    dq, dk, dv = A.backward(q, k[:, :, :nk2], v[:, :, :nk2], g, 0.4, True)
    assert np.all(dq[0, 0, :nq - nk2] == 0)
    dq2, dk2, dv2 = A.backward(q[:, :, nq - nk2:], k[:, :, :nk2], v[:, :, :nk2], g[:, :, nq - nk2:], 0.4, True)
    assert np.abs(dq[:, :, nq - nk2:] - dq2).max() <= 1e-12
    assert np.abs(dk - dk2).max() <= 1e-12 and np.abs(dv - dv2).max() <= 1e-12
    # a single query (decoding) sees every key
    q1 = _rand((1, 1, 1, d), 83)
    o1, l1 = A.forward(q1, k, v, 0.4, True)
    on, ln_ = A.forward(q1, k, v, 0.4, False)
    assert np.array_equal(o1, on) and np.array_equal(l1, ln_)


def pin_cross_lengths_finite_differences():
    _fd_case(1, 2, 1, 5, 3, True, None, 610, nk=9)
    _fd_case(1, 1, 1, 9, 3, True, None, 620, nk=4)
    _fd_case(2, 2, 2, 6, 2, False, None, 630, nk=11)
    mask = np.array([[1, 0, 1]], dtype=np.uint8)
    _fd_case(1, 1, 1, 100, 2, True, mask, 640, ncoord=16, nk=300)   # 1 x 3 block mask


# ----------------------------------------------------------------------------------------------
# P-16: packed variable-length batches equal attention over the concatenation with
# visibility restricted to each sequence (brute force over the whole packed rows)
# ----------------------------------------------------------------------------------------------
def _packed_brute_force(q, k, v, cu_q, cu_k, scale, causal):
    """q: [Tq, d], k, v: [Tk, d] of one head; scalar loops over packed positions."""
    tq, dv = len(q), len(v[0])
    outs, lses = [], []
    for i in range(tq):
        b = max(x for x in range(len(cu_q) - 1) if cu_q[x] <= i)
        while cu_q[b + 1] <= i:
            b += 1
        nq, nk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        pos = (i - cu_q[b]) + nk - nq   # the row's position within its own sequence
        keys = [j for j in range(len(k)) if cu_k[b] <= j < cu_k[b + 1] and (not causal or j - cu_k[b] <= pos)]
        if not keys:
            outs.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        sc = [scale * sum(a * c for a, c in zip(q[i], k[j])) for j in keys]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        z = sum(w)
        outs.append([sum(w[a] * v[j][t] for a, j in enumerate(keys)) / z for t in range(dv)])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


def pin_varlen_brute_force():
    cases = [([0, 3, 3, 8, 9], [0, 5, 7, 9, 9]),      # an empty query run and an empty key run
             ([0, 4, 10], [0, 4, 10]),
             ([0, 1, 2, 3], [0, 6, 7, 12])]
    for n, (cu_q, cu_k) in enumerate(cases):
        H, Hkv, d = 2, 1, 3
        q = _rand((H, cu_q[-1], d), 700 + n)
        k = _rand((Hkv, cu_k[-1], d), 710 + n)
        v = _rand((Hkv, cu_k[-1], d), 720 + n)
        for causal in (False, True):
            o, l_ = A.forward_varlen(q, k, v, cu_q, cu_k, 0.8, causal)
            for h in range(H):
                ob, lb = _packed_brute_force(q[h].tolist(), k[0].tolist(), v[0].tolist(), cu_q, cu_k, 0.8, causal)
                assert np.abs(o[h] - ob).max(initial=0.0) <= 1e-12, (n, causal)
                assert np.array_equal(np.isinf(l_[h]), np.isinf(lb))
                fin = np.isfinite(lb)
                assert np.abs(l_[h][fin] - lb[fin]).max(initial=0.0) <= 1e-12


def pin_varlen_finite_differences():
    cu_q, cu_k = [0, 3, 7, 7, 12], [0, 6, 8, 10, 13]
    H, Hkv, d, scale = 2, 1, 2, 0.7
    q = _rand((H, 12, d), 730)
    k = _rand((Hkv, 13, d), 731)
    v = _rand((Hkv, 13, d), 732)
    g = _rand((H, 12, d), 733)
    for causal, rate in ((True, 0.0), (False, 0.0), (True, 0.4)):
        def f(q_, k_, v_):
            o, _ = A.forward_varlen(q_, k_, v_, cu_q, cu_k, scale, causal, rate, 99)
            return float((o * g).sum())

        grads = A.backward_varlen(q, k, v, g, cu_q, cu_k, scale, causal, rate, 99)
        rng = np.random.default_rng(734)
        for which, x in enumerate((q, k, v)):
            for flat in rng.choice(x.size, size=16, replace=False):
                idx = np.unravel_index(flat, x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += 1e-6
                xm[idx] -= 1e-6
                ap, am = [q, k, v], [q, k, v]
                ap[which], am[which] = xp, xm
                num = (f(*ap) - f(*am)) / 2e-6
                assert abs(num - grads[which][idx]) <= 1e-6 * max(1.0, abs(num)), ("qkv"[which], causal, rate)


def pin_varlen_dropout_streams():
    """Sequence b of a packed batch draws the same keep decisions as batch
    entry b of a fixed-length batch of the same lengths (stream b * H + h,
    positions within the sequence)."""
    B, H, n, d = 3, 2, 20, 4
    q, k, v = (_rand((B, H, n, d), s) for s in (741, 742, 743))
    o, l_ = A.forward(q, k, v, 0.5, True, dropout_rate=0.3, seed=5)
    cu = [0, n, 2 * n, 3 * n]
    pack = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(H, B * n, d))
    ov, lv = A.forward_varlen(pack(q), pack(k), pack(v), cu, cu, 0.5, True, 0.3, 5)
    assert np.abs(ov - pack(o)).max() <= 1e-15
    assert np.abs(lv - l_.transpose(1, 0, 2).reshape(H, B * n)).max() <= 1e-15


# ----------------------------------------------------------------------------------------------
# P-17: sliding-window (band) masks: p - left <= j <= p + right around the query's position p
# ----------------------------------------------------------------------------------------------
def _window_brute_force(q, k, v, scale, causal, left, right):
    nq, nk, dv = len(q), len(k), len(v[0])
    outs, lses = [], []
    for i in range(nq):
        pos = i + nk - nq
        keys = []
        for j in range(nk):
            if causal and j > pos:
                continue
            if left >= 0 and j < pos - left:
                continue
            if right >= 0 and j > pos + right:
                continue
            keys.append(j)
        if not keys:
            outs.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        sc = [scale * sum(a * b for a, b in zip(q[i], k[j])) for j in keys]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        z = sum(w)
        outs.append([sum(w[a] * v[j][t] for a, j in enumerate(keys)) / z for t in range(dv)])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


def pin_window_brute_force():
    seed = 800
    for nq, nk in ((1, 1), (3, 3), (5, 5), (2, 6), (6, 3)):
        for left, right in ((-1, -1), (0, 0), (1, 0), (2, 1), (-1, 2), (3, -1), (0, -1)):
            for causal in (False, True):
                seed += 1
                q, k, v = _rand((nq, 3), seed), _rand((nk, 3), seed + 50), _rand((nk, 2), seed + 90)
                o, l_ = A.forward(q[None, None], k[None, None], v[None, None], 0.8, causal, window=(left, right))
                ob, lb = _window_brute_force(q.tolist(), k.tolist(), v.tolist(), 0.8, causal, left, right)
                assert np.abs(o[0, 0] - ob).max() <= 1e-12, (nq, nk, left, right, causal)
                assert np.array_equal(np.isinf(l_[0, 0]), np.isinf(lb))
                fin = np.isfinite(lb)
                assert np.abs(l_[0, 0][fin] - lb[fin]).max(initial=0.0) <= 1e-12


def pin_window_torch_sdpa():
    """Against PyTorch's float64 CPU attention with an explicit boolean mask
    written out element by element, gradients through autograd."""
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, nq, nk, d, causal, left, right, seed) in [
            (1, 2, 2, 150, 150, 8, True, 40, 0, 811), (2, 4, 2, 90, 200, 8, False, 17, 5, 812),
            (1, 2, 1, 200, 70, 4, True, 0, -1, 813), (1, 1, 1, 257, 257, 16, False, 128, 128, 814)]:
        q, k, v = _rand((B, H, nq, d), seed), _rand((B, Hkv, nk, d), seed + 1), _rand((B, Hkv, nk, d), seed + 2)
        g = _rand((B, H, nq, d), seed + 3)
        allow = np.zeros((nq, nk), dtype=bool)
        for i in range(nq):
            pos = i + nk - nq
            for j in range(nk):
                ok = (not causal or j <= pos) and (left < 0 or j >= pos - left) and (right < 0 or j <= pos + right)
                allow[i, j] = ok
        rows_any = allow.any(axis=1)
        G = H // Hkv
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        kk, vv = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
        # torch returns NaN for rows with no visible key; those rows are checked separately
        to = F.scaled_dot_product_attention(tq, kk, vv, attn_mask=torch.tensor(allow), scale=0.3)
        to = torch.where(torch.tensor(rows_any)[:, None], to, torch.zeros_like(to))
        to.backward(torch.tensor(g))
        o, l_ = A.forward(q, k, v, 0.3, causal, window=(left, right))
        dq, dk, dv = A.backward(q, k, v, g, 0.3, causal, window=(left, right))
        assert np.abs(o - to.detach().numpy()).max() <= 1e-12
        assert np.all(o[:, :, ~rows_any] == 0) and np.all(np.isneginf(l_[:, :, ~rows_any]))
        for a, b in ((dq, tq), (dk, tk), (dv, tv)):
            gr = np.nan_to_num(b.grad.numpy())
            assert np.abs(a - gr).max() <= 1e-12
        s = (torch.tensor(q) @ torch.tensor(np.repeat(k, G, axis=1)).transpose(-1, -2) * 0.3)
        s = s.masked_fill(~torch.tensor(allow), float("-inf"))
        ref = torch.logsumexp(s, dim=-1).numpy()
        assert np.abs(l_[:, :, rows_any] - ref[:, :, rows_any]).max() <= 1e-12


def pin_window_limits():
    n, d = 300, 5
    q, k, v, g = (_rand((1, 2, n, d), s) for s in (821, 822, 823, 824))
    # a band wider than the sequence changes nothing; (-1, 0) is causal masking
    for causal in (False, True):
        o, l_ = A.forward(q, k, v, 0.5, causal)
        o2, l2 = A.forward(q, k, v, 0.5, causal, window=(n, n))
        assert np.array_equal(o, o2) and np.array_equal(l_, l2)
    o, l_ = A.forward(q, k, v, 0.5, True)
    o2, l2 = A.forward(q, k, v, 0.5, False, window=(-1, 0))
    assert np.array_equal(o, o2) and np.array_equal(l_, l2)
    # (0, 0): each query sees exactly its own key
    o, l_ = A.forward(q, k, v, 0.5, False, window=(0, 0))
    assert np.abs(o - v).max() <= 1e-15
    assert np.abs(l_ - 0.5 * (q * k).sum(-1)).max() <= 1e-13
    dq, dk, dv = A.backward(q, k, v, g, 0.5, False, window=(0, 0))
    assert np.abs(dv - g).max() <= 1e-15 and np.abs(dq).max() <= 1e-15 and np.abs(dk).max() <= 1e-15
    # (1, 0) with causal: two keys per row but row 0, the sigmoid closed form
    o, _ = A.forward(q, k, v, 0.5, True, window=(1, 0))
    i = 7
    s0, s1 = 0.5 * q[0, 0, i] @ k[0, 0, i - 1], 0.5 * q[0, 0, i] @ k[0, 0, i]
    sig = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.abs(o[0, 0, i] - (sig * v[0, 0, i - 1] + (1 - sig) * v[0, 0, i])).max() <= 1e-14


def pin_window_finite_differences():
    def case(nq, nk, causal, window, seed, bm=None):
        q = _rand((1, 2, nq, 3), seed)
        k = _rand((1, 1, nk, 3), seed + 1)
        v = _rand((1, 1, nk, 3), seed + 2)
        g = _rand((1, 2, nq, 3), seed + 3)

        def f(q_, k_, v_):
            o, _ = A.forward(q_, k_, v_, 0.6, causal, bm, window=window)
            return float((o * g).sum())

        grads = A.backward(q, k, v, g, 0.6, causal, bm, window=window)
        rng = np.random.default_rng(seed + 4)
        for which, x in enumerate((q, k, v)):
            for flat in rng.choice(x.size, size=16, replace=False):
                idx = np.unravel_index(flat, x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += 1e-6
                xm[idx] -= 1e-6
                ap, am = [q, k, v], [q, k, v]
                ap[which], am[which] = xp, xm
                num = (f(*ap) - f(*am)) / 2e-6
                assert abs(num - grads[which][idx]) <= 1e-6 * max(1.0, abs(num)), ("qkv"[which], window)
    case(12, 12, True, (3, -1), 830)
    case(9, 14, False, (2, 3), 840)
    case(14, 9, True, (4, 0), 850)
    case(140, 140, False, (60, 10), 860, np.array([[1, 1], [0, 1]], dtype=np.uint8))


# ----------------------------------------------------------------------------------------------
# P-18: FP8 (E4M3) inputs: the decoder against PyTorch's float8_e4m3fn and the format's closed
# forms; the per-tensor descales enter as the definition says
# ----------------------------------------------------------------------------------------------
def pin_e4m3_decode():
    import torch
    import oracle.fp8 as F8
    codes = np.arange(256, dtype=np.uint8)
    ours = F8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))      # -0 for 0x80
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and ours[0xC0] == -2.0
    # codes round-trip through PyTorch's encoder
    vals = ours[fin & (codes != 0x80)]
    back = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F8.e4m3_decode(back), vals)


def pin_fp8_descales():
    import torch
    import oracle.fp8 as F8
    rng = np.random.default_rng(901)
    B, H, n, d = 1, 2, 150, 16
    q8, k8, v8 = (torch.from_numpy(rng.normal(0, 2, size=(B, H, n, d))).to(torch.float8_e4m3fn)
                  .view(torch.uint8).numpy() for _ in range(3))
    o1, l1 = F8.forward_fp8(q8, k8, v8, 0.3, 1.0, 1.0, 1.0, True)
    # the same as attention of the decoded values, which are those PyTorch decodes
    dec = [torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.float64).numpy() for x in (q8, k8, v8)]
    o0, l0 = A.forward(dec[0], dec[1], dec[2], 0.3, True)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    # q and k descales enter the scores only through their product with the scale
    o2, l2 = F8.forward_fp8(q8, k8, v8, 0.3, 4.0, 0.25, 1.0, True)
    o3, l3 = F8.forward_fp8(q8, k8, v8, 0.6, 1.0, 0.5, 1.0, True)
    assert np.abs(o2 - o1).max() <= 1e-13 and np.abs(l2 - l1).max() <= 1e-13
    assert np.abs(o3 - o1).max() <= 1e-13 and np.abs(l3 - l1).max() <= 1e-13
    # the value descale scales the output only
    o4, l4 = F8.forward_fp8(q8, k8, v8, 0.3, 1.0, 1.0, 3.0, True)
    assert np.abs(o4 - 3.0 * o1).max() <= 1e-13 and np.array_equal(l4, l1)


# ----------------------------------------------------------------------------------------------
# P-19: score modification, the ALiBi distance bias: s_ij += -slope_h |i + (Nk - Nq) - j|
# ----------------------------------------------------------------------------------------------
def _alibi_brute_force(q, k, v, scale, causal, slope, window=(-1, -1)):
    nq, nk, dv = len(q), len(k), len(v[0])
    outs, lses = [], []
    for i in range(nq):
        pos = i + nk - nq
        keys = [j for j in range(nk) if (not causal or j <= pos) and (window[0] < 0 or j >= pos - window[0])
                and (window[1] < 0 or j <= pos + window[1])]
        if not keys:
            outs.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        sc = [scale * sum(a * b for a, b in zip(q[i], k[j])) - slope * abs(pos - j) for j in keys]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        z = sum(w)
        outs.append([sum(w[a] * v[j][t] for a, j in enumerate(keys)) / z for t in range(dv)])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


def pin_alibi_brute_force():
    seed = 950
    for nq, nk in ((1, 1), (4, 4), (3, 7), (6, 2)):
        for causal in (False, True):
            for slope, window in ((0.5, (-1, -1)), (0.125, (2, -1)), (2.0, (-1, 1))):
                seed += 1
                q, k, v = _rand((nq, 3), seed), _rand((nk, 3), seed + 40), _rand((nk, 2), seed + 80)
                o, l_ = A.forward(q[None, None], k[None, None], v[None, None], 0.7, causal, window=window,
                                  alibi_slopes=[slope])
                ob, lb = _alibi_brute_force(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, slope, window)
                assert np.abs(o[0, 0] - ob).max() <= 1e-12, (nq, nk, causal, slope, window)
                fin = np.isfinite(lb)
                assert np.array_equal(np.isinf(l_[0, 0]), ~fin)
                assert np.abs(l_[0, 0][fin] - lb[fin]).max(initial=0.0) <= 1e-12


def pin_alibi_torch_sdpa():
    """PyTorch's float64 attention with the bias as an additive mask written out
    element by element (-inf where causal masking hides a key); gradients
    through autograd."""
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, nq, nk, d, causal, seed) in [(1, 4, 2, 70, 70, 8, True, 961), (2, 2, 1, 40, 90, 4, False, 962),
                                                 (1, 2, 2, 90, 40, 8, True, 963)]:
        slopes = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]
        q, k, v = _rand((B, H, nq, d), seed), _rand((B, Hkv, nk, d), seed + 1), _rand((B, Hkv, nk, d), seed + 2)
        g = _rand((B, H, nq, d), seed + 3)
        bias = np.zeros((H, nq, nk))
        for h in range(H):
            for i in range(nq):
                pos = i + nk - nq
                for j in range(nk):
                    bias[h, i, j] = -math.inf if (causal and j > pos) else -slopes[h] * abs(pos - j)
        rows_any = np.isfinite(bias).any(axis=2)
        G = H // Hkv
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        kk, vv = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
        to = F.scaled_dot_product_attention(tq, kk, vv, attn_mask=torch.tensor(bias)[None], scale=0.4)
        to = torch.where(torch.tensor(rows_any)[None, :, :, None], to, torch.zeros_like(to))
        to.backward(torch.tensor(g))
        o, l_ = A.forward(q, k, v, 0.4, causal, alibi_slopes=slopes)
        dq, dk, dv = A.backward(q, k, v, g, 0.4, causal, alibi_slopes=slopes)
        assert np.abs(o - to.detach().numpy()).max() <= 1e-12
        for a, b in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.abs(a - np.nan_to_num(b.grad.numpy())).max() <= 1e-12
        sc = torch.tensor(q) @ torch.tensor(np.repeat(k, G, axis=1)).transpose(-1, -2) * 0.4 + torch.tensor(bias)[None]
        ref = torch.logsumexp(sc, dim=-1).numpy()
        fin = np.broadcast_to(rows_any[None], ref.shape)
        assert np.abs(l_[fin] - ref[fin]).max() <= 1e-12


def pin_alibi_limits():
    n, d = 200, 6
    q, k, v = (_rand((1, 2, n, d), s) for s in (971, 972, 973))
    for causal in (False, True):
        o0, l0 = A.forward(q, k, v, 0.5, causal)
        o1, l1 = A.forward(q, k, v, 0.5, causal, alibi_slopes=[0.0, 0.0])
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
        # a steep slope leaves (almost) only the key at distance 0: O -> v_i within 2 sum_j exp(-gap_j)
        slope = 60.0
        o2, _ = A.forward(q, k, v, 0.5, causal, alibi_slopes=[slope, slope])
        s_ = 0.5 * np.einsum("bhid,bhjd->bhij", q, k)
        gap = s_.diagonal(axis1=2, axis2=3)[..., None] - s_ + slope * np.abs(np.arange(n)[:, None] - np.arange(n)[None])
        np.einsum("bhii->bhi", gap)[...] = np.inf
        bound = 2 * np.exp(-gap).sum(axis=-1)[..., None] * np.abs(v).max()
        assert np.all(np.abs(o2 - v) <= bound)


def pin_alibi_finite_differences():
    for causal, nq, nk, seed in ((True, 8, 8, 980), (False, 6, 11, 981)):
        q = _rand((1, 2, nq, 3), seed)
        k = _rand((1, 1, nk, 3), seed + 1)
        v = _rand((1, 1, nk, 3), seed + 2)
        g = _rand((1, 2, nq, 3), seed + 3)
        sl = [0.7, 0.2]

        def f(q_, k_, v_):
            o, _ = A.forward(q_, k_, v_, 0.6, causal, alibi_slopes=sl)
            return float((o * g).sum())

        grads = A.backward(q, k, v, g, 0.6, causal, alibi_slopes=sl)
        rng = np.random.default_rng(seed + 4)
        for which, x in enumerate((q, k, v)):
            for flat in rng.choice(x.size, size=12, replace=False):
                idx = np.unravel_index(flat, x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += 1e-6
                xm[idx] -= 1e-6
                ap, am = [q, k, v], [q, k, v]
                ap[which], am[which] = xp, xm
                num = (f(*ap) - f(*am)) / 2e-6
                assert abs(num - grads[which][idx]) <= 1e-6 * max(1.0, abs(num)), ("qkv"[which], causal)



# ----------------------------------------------------------------------------------------------
# P-17: element masks (an arbitrary boolean predicate per (query, key) pair, shared by every
# batch and head; the "FlashAttention" lesson, Researcher tier, "Beyond hand-written kernels")
# ----------------------------------------------------------------------------------------------
def _masked_brute_force(q, k, v, scale, causal, allow):
    """Scalar loops over an explicit visibility matrix allow[i][j] (and causal
    j <= i + len(k) - len(q))."""
    n, d, dv = len(q), len(q[0]), len(v[0])
    outs, lses = [], []
    for i in range(n):
        pos = i + len(k) - n
        keys = [j for j in range(len(k)) if allow[i][j] and (not causal or j <= pos)]
        if not keys:
            outs.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        sc = [scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        z = sum(w)
        outs.append([sum(w[a] * v[j][t] for a, j in enumerate(keys)) / z for t in range(dv)])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


def pin_elem_mask_brute_force():
    rng = np.random.default_rng(1701)
    seed = 1700
    for nq, nk in ((1, 1), (3, 3), (4, 6), (6, 4), (5, 5)):
        for causal in (False, True):
            for density in (0.3, 0.7):
                seed += 1
                allow = rng.random((nq, nk)) < density
                allow[0] = False                      # a row that sees nothing
                q, k, v = _rand((nq, 3), seed), _rand((nk, 3), seed + 50), _rand((nk, 2), seed + 90)
                o, l_ = A.forward(q[None, None], k[None, None], v[None, None], 0.8, causal, elem_mask=allow)
                ob, lb = _masked_brute_force(q.tolist(), k.tolist(), v.tolist(), 0.8, causal, allow.tolist())
                where = (nq, nk, causal, density)
                assert np.abs(o[0, 0] - ob).max() <= 1e-12, where
                fin = np.isfinite(lb)
                assert np.array_equal(np.isfinite(l_[0, 0]), fin), where
                assert np.abs(l_[0, 0][fin] - lb[fin]).max(initial=0.0) <= 1e-12, where


def pin_elem_mask_torch_sdpa():
    """Against PyTorch's float64 CPU attention with the boolean mask as its
    attn_mask, gradients through autograd (grouped-query and causal cases)."""
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, nq, nk, d, causal, seed) in [(1, 2, 2, 150, 150, 8, False, 1711),
                                                 (2, 4, 2, 90, 200, 8, True, 1712),
                                                 (1, 3, 1, 260, 260, 4, True, 1713)]:
        rng = np.random.default_rng(seed)
        allow = rng.random((nq, nk)) < 0.4
        allow[:, 0] = True                             # every row sees a key (torch gives NaN otherwise)
        q, k, v = _rand((B, H, nq, d), seed), _rand((B, Hkv, nk, d), seed + 1), _rand((B, Hkv, nk, d), seed + 2)
        g = _rand((B, H, nq, d), seed + 3)
        full = allow.copy()
        if causal:
            full &= np.arange(nk)[None, :] <= np.arange(nq)[:, None] + (nk - nq)
        G = H // Hkv
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        to = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1),
                                            attn_mask=torch.tensor(full), scale=0.3)
        to.backward(torch.tensor(g))
        o, l_ = A.forward(q, k, v, 0.3, causal, elem_mask=allow)
        dq, dk, dv = A.backward(q, k, v, g, 0.3, causal, elem_mask=allow)
        assert np.abs(o - to.detach().numpy()).max() <= 1e-12
        s = torch.tensor(q) @ torch.tensor(np.repeat(k, G, axis=1)).transpose(-1, -2) * 0.3
        s = s.masked_fill(~torch.tensor(full), float("-inf"))
        assert np.abs(l_ - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12
        for a, b in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.abs(a - b.grad.numpy()).max() <= 1e-12


def pin_elem_mask_equivalences():
    """Masks that other arguments already express give identical results: all
    true = no mask; lower triangle = causal; constant on 128 x 128 blocks = the
    block mask; a band = the window; a document mask (same document) = the
    packed batch of those documents."""
    n, d = 300, 4
    q, k, v, g = (_rand((1, 2, n, d), s) for s in (1721, 1722, 1723, 1724))
    ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")

    def same(kw_a, kw_b):
        o1, l1 = A.forward(q, k, v, 0.5, **kw_a)
        o2, l2 = A.forward(q, k, v, 0.5, **kw_b)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), (kw_a.keys(), kw_b.keys())
        g1 = A.backward(q, k, v, g, 0.5, **kw_a)
        g2 = A.backward(q, k, v, g, 0.5, **kw_b)
        for a, b in zip(g1, g2):
            assert np.array_equal(a, b)

    same(dict(causal=False), dict(causal=False, elem_mask=np.ones((n, n), dtype=bool)))
    same(dict(causal=True), dict(causal=False, elem_mask=jj <= ii))
    bm = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    same(dict(causal=False, block_mask=bm), dict(causal=False, elem_mask=bm[ii // 128, jj // 128] != 0))
    same(dict(causal=True, window=(37, 0)), dict(causal=False, elem_mask=(jj <= ii) & (jj >= ii - 37)))
    # a document mask equals the packed batch of the documents (forward and backward)
    lens = [70, 1, 129, 100]
    cu = np.concatenate([[0], np.cumsum(lens)])
    doc = np.repeat(np.arange(len(lens)), lens)
    allow = doc[:, None] == doc[None, :]
    for causal in (False, True):
        o1, l1 = A.forward(q, k, v, 0.5, causal, elem_mask=allow)
        o2, l2 = A.forward_varlen(q[0], k[0], v[0], cu, cu, 0.5, causal)
        assert np.abs(o1[0] - o2).max() <= 1e-14 and np.abs(l1[0] - l2).max() <= 1e-13
        d1 = A.backward(q, k, v, g, 0.5, causal, elem_mask=allow)
        d2 = A.backward_varlen(q[0], k[0], v[0], g[0], cu, cu, 0.5, causal)
        for a, b in zip(d1, d2):
            assert np.abs(a[0] - b).max() <= 1e-13


def pin_elem_mask_empty_rows():
    """Rows that see no key under the element mask: O = 0, L = -inf, zero dQ,
    and their upstream gradient reaches no dK or dV."""
    n, d = 200, 4
    q, k, v, g = (_rand((1, 1, n, d), s) for s in (1731, 1732, 1733, 1734))
    allow = np.random.default_rng(1735).random((n, n)) < 0.5
    empty = np.array([0, 5, 130, 199])
    allow[empty] = False
    o, l_ = A.forward(q, k, v, 0.5, False, elem_mask=allow)
    assert np.all(o[0, 0, empty] == 0) and np.all(np.isneginf(l_[0, 0, empty]))
    dq, dk, dv = A.backward(q, k, v, g, 0.5, False, elem_mask=allow)
    assert np.all(dq[0, 0, empty] == 0)
    g2 = g.copy()
    g2[0, 0, empty] = 1e3
    _, dk2, dv2 = A.backward(q, k, v, g2, 0.5, False, elem_mask=allow)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def pin_elem_mask_finite_differences():
    n, d, scale = 14, 3, 0.6
    rng = np.random.default_rng(1741)
    allow = rng.random((n, n)) < 0.5
    allow[:, 3] = True
    q, k, v, g = (_rand((1, 2, n, d), s) for s in (1742, 1743, 1744, 1745))
    k, v = k[:, :1], v[:, :1]                        # grouped-query: two query heads, one kv head
    grads = A.backward(q, k, v, g, scale, True, elem_mask=allow)

    def f(q_, k_, v_):
        o, _ = A.forward(q_, k_, v_, scale, True, elem_mask=allow)
        return float((o * g).sum())

    h = 1e-6
    for which, x in enumerate((q, k, v)):
        num, ana = [], []
        for flat in rng.choice(x.size, size=min(20, x.size), replace=False):
            idx = np.unravel_index(flat, x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p, a_m = [q, k, v], [q, k, v]
            a_p[which], a_m[which] = xp, xm
            num.append((f(*a_p) - f(*a_m)) / (2 * h))
            ana.append(grads[which][idx])
        num, ana = np.array(num), np.array(ana)
        assert np.abs(num - ana).max() / max(np.abs(ana).max(), 1e-3) <= 1e-6, "qkv"[which]

ALL_PINS = [pin_worked_example, pin_recurrence, pin_brute_force, pin_rows_sum_to_one, pin_zero_query,
            pin_dominant_score, pin_permutation, pin_causal_locality, pin_finite_differences,
            pin_gqa_repeat, pin_mask_semantics, pin_empty_rows, pin_scale_zero, pin_torch_sdpa,
            pin_philox_known_answers, pin_dropout_statistics, pin_dropout_expectation,
            pin_dropout_finite_differences, pin_cross_lengths_brute_force, pin_cross_lengths_suffix,
            pin_cross_lengths_finite_differences, pin_varlen_brute_force, pin_varlen_finite_differences,
            pin_varlen_dropout_streams, pin_window_brute_force, pin_window_torch_sdpa, pin_window_limits,
            pin_window_finite_differences, pin_e4m3_decode, pin_fp8_descales, pin_alibi_brute_force,
            pin_alibi_torch_sdpa, pin_alibi_limits, pin_alibi_finite_differences, pin_elem_mask_brute_force,
            pin_elem_mask_torch_sdpa, pin_elem_mask_equivalences, pin_elem_mask_empty_rows,
            pin_elem_mask_finite_differences]
