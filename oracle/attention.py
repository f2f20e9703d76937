"""Float64 reference for exact attention: forward and analytic backward.

Test infrastructure only (see the package docstring). Nothing here is tiled,
fused or reordered beyond what the definition states: each query row's full
score vector over its visible keys is materialised, normalised and applied.
Rows are processed a chunk at a time only so that numpy can vectorise; the
chunking does not change the arithmetic of any row.

Sources (cited by page title and section):
* "FlashAttention" lesson (learn.pranaymahendrakar.com), Researcher tier,
  "The problem being solved": O = softmax(Q K^T / sqrt(d)) V, with S and P
  the N x N score and probability matrices.
* Same lesson, Developer tier, flash_numpy.py ``naive_attention``: the scale
  multiplies Q K^T before the row maximum is subtracted and exp is taken.
* Same lesson, Researcher tier, "IO complexity", and the nadeemcite.github.io
  summary "FlashAttention: Fast and Memory-Efficient Exact Attention with
  IO-Awareness", Core Idea item 3: the backward pass rebuilds P from saved
  softmax statistics. The statistic kept here is L = m + ln(l), the natural-log
  log-sum-exp of a row's scaled scores, so that P = exp(S - L).
* Causal masking: the lesson's Beginner tier ("What was broken before") says a
  word attends to earlier words; read here as key j visible to query i iff
  j <= i (self included). With Nq queries over Nk keys the queries are read
  as the last Nq positions of the sequence (the chipfoundryservices.com
  glossary "flash attention algorithm", "Inference Optimization": attention
  run beside a KV cache), so key j is visible to query i iff
  j <= i + (Nk - Nq); rows with i + (Nk - Nq) < 0 see no key.
* Sliding-window (local) masks: the lesson's Researcher tier, "Beyond
  hand-written kernels" (one tiled kernel serving many masks) and its pointer
  to sparse and block attention patterns. Read here as a band
  window = (left, right) around the query's position p = i + (Nk - Nq): key j
  is visible iff p - left <= j <= p + right, -1 meaning unbounded on that
  side; causal masking is the right bound 0. Band, causal and block masks
  combine by intersection.
* Element masks: the same lesson section describes one tiled kernel serving
  user mask functions (mask_mod) evaluated per (query, key) pair. Read here
  as an arbitrary boolean predicate, given to the oracle written out as a
  dense [Nq, Nk] matrix (True = visible), shared by every batch and head and
  intersected with every other mask (``elem_mask``). Examples: a document
  mask (query and key in the same document), a prefix-LM mask, a random
  mask.
* Score modification: the same lesson section speaks of user functions that
  modify scores (score_mod) inside the one tiled kernel, naming none. Read
  here as the linear distance bias of ALiBi (Press, Smith and Lewis, 2022),
  one slope per query head: s_ij += -slope_h * |i + (Nk - Nq) - j|, added to
  the scaled score before the softmax; it has no gradient of its own.
* Variable-length batches: the same glossary, "Sequence Length Flexibility"
  (arbitrary lengths, no padding). Read here as sequences packed one after
  another per head, each attending only within itself
  (``forward_varlen``, ``backward_varlen``).
* Block-sparse masking: the nadeemcite summary, Key Method Details,
  "Block-sparse extension": a mask over blocks. Read here as a uint8 matrix of
  128 x 128 blocks, nonzero = keep, shared by every batch and head, combined
  with causal masking by intersection.
* Grouped-query attention: the lesson's related-term card "Grouped-query
  attention": a group of query heads shares one key/value head. Read here as
  contiguous groups, kv head = h // (H // Hkv).

The gradient formulas are not on the pages; they are the chain rule through
the row softmax (its Jacobian is diag(p) - p p^T), pinned by finite
differences in the tests.
"""

import numpy as np

from . import dropout as _dropout

MASK_BLOCK = 128  # block-mask granularity in rows and columns


def visible(rows, keys, causal, block_mask, block=MASK_BLOCK, offset=0, window=(-1, -1), elem_mask=None):
    """Boolean matrix a[r, c]: is key ``keys[c]`` visible to query ``rows[r]``.

    Causal: j <= i + offset (offset = Nk - Nq, 0 for square attention). Window
    (left, right): i + offset - left <= j <= i + offset + right, a negative
    bound unbounded. Block mask: mask[i // block][j // block] != 0. Element
    mask: elem_mask[i][j] true. All that are given must hold.
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    a = np.ones((rows.size, keys.size), dtype=bool)
    if causal:
        a &= keys[None, :] <= rows[:, None] + offset
    left, right = window
    if left >= 0:
        a &= keys[None, :] >= rows[:, None] + offset - left
    if right >= 0:
        a &= keys[None, :] <= rows[:, None] + offset + right
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        a &= bm[(rows // block)[:, None], (keys // block)[None, :]]
    if elem_mask is not None:
        a &= np.asarray(elem_mask, dtype=bool)[rows[:, None], keys[None, :]]
    return a


def candidate_keys(rows, n_keys, causal, block_mask, block=MASK_BLOCK, offset=0, window=(-1, -1), elem_mask=None):
    """Keys that at least one of ``rows`` may see (a superset used to gather K, V).

    Keys outside this set are invisible to every row of the chunk, so leaving
    them out drops only terms whose probability is exactly zero.
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(n_keys, dtype=np.int64)
    if rows.size == 0:
        return keys[:0]
    if causal:
        keys = keys[keys <= rows.max() + offset]
    if window[0] >= 0:
        keys = keys[keys >= rows.min() + offset - window[0]]
    if window[1] >= 0:
        keys = keys[keys <= rows.max() + offset + window[1]]
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        any_row = bm[np.unique(rows // block)].any(axis=0)
        keys = keys[any_row[keys // block]]
    if elem_mask is not None:
        keys = keys[np.asarray(elem_mask, dtype=bool)[rows].any(axis=0)[keys]]
    return keys


def _chunks(rows, size):
    for i in range(0, rows.size, size):
        yield rows[i:i + size]


def _row_softmax(q_rows, k_keys, scale, vis, bias=None):
    """Scores, probabilities and log-sum-exp of one chunk of rows.

    s = scale * q k^T (+ bias) over the gathered keys, -inf where a key is
    invisible. L = m + ln(sum exp(s - m)) with m the row maximum (the
    safe-softmax shift of ``naive_attention``); p = exp(s - L). A row with no
    visible key has L = -inf and p = 0 (nothing to attend to, so it
    contributes nothing).
    """
    s = scale * (q_rows @ k_keys.T)
    if bias is not None:
        s = s + bias
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    e = np.exp(s - m0[:, None])
    ssum = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m0 + np.log(np.where(has, ssum, 1.0)), -np.inf)
    p = np.where(has[:, None], e / np.where(has, ssum, 1.0)[:, None], 0.0)
    return s, p, lse


def alibi_bias(rows, keys, slope, offset):
    """-slope * |i + offset - j| for query rows i and keys j (None for no slope)."""
    if slope is None:
        return None
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    return -float(slope) * np.abs((rows[:, None] + offset) - keys[None, :]).astype(np.float64)


def head_probabilities(q, k, scale, causal=False, block_mask=None, rows=None, window=(-1, -1), alibi=None,
                       elem_mask=None):
    """Full probability rows P[rows, :] (Nk keys wide) of one query head.

    q: [Nq, d] float64 query rows of the head, k: [Nk, d] keys of its kv head;
    alibi: this head's slope or None.
    """
    n = k.shape[0]
    off = n - q.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    keys = np.arange(n)
    vis = visible(rows, keys, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)
    _, p, lse = _row_softmax(q[rows], k, scale, vis, alibi_bias(rows, keys, alibi, off))
    return p, lse


def _drop(p, rows, keys, dropout):
    """p with dropout applied (kept values scaled), or p unchanged when dropout is None.

    dropout = (rate, seed, bh): see ``oracle.dropout``."""
    if dropout is None:
        return p
    rate, seed, bh = dropout
    z = _dropout.keep_mask(seed, bh, rows, keys, rate)
    return np.where(z, p * _dropout.keep_scale(rate), 0.0)


def head_forward(q, k, v, scale, causal=False, block_mask=None, rows=None, chunk=256, dropout=None,
                 window=(-1, -1), alibi=None, elem_mask=None):
    """O and L for the given query rows of one head (q: [Nq, d], k, v: [Nk, d]).

    With dropout = (rate, seed, bh) the probabilities are dropped and rescaled
    before they weight V; L is still that of the scores before dropout."""
    n = k.shape[0]
    off = n - q.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.full(rows.size, -np.inf)
    pos = 0
    for ch in _chunks(rows, chunk):
        keys = candidate_keys(ch, n, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)
        if keys.size:
            vis = visible(ch, keys, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)
            _, p, l_ = _row_softmax(q[ch], k[keys], scale, vis, alibi_bias(ch, keys, alibi, off))
            o[pos:pos + ch.size] = _drop(p, ch, keys, dropout) @ v[keys]
            lse[pos:pos + ch.size] = l_
        pos += ch.size
    return o, lse


def head_backward(q, k, v, do, scale, causal=False, block_mask=None, chunk=256, dropout=None, window=(-1, -1),
                  alibi=None, elem_mask=None):
    """Gradients of sum(O * dO) for one query head.

    With p the probability rows, g = dO, and (under dropout) r the dropped and
    rescaled probabilities r_ij = p_ij z_ij c (z the keep decision, c the keep
    scale; without dropout r = p and z c = 1):
      dV_j += sum_i r_ij g_i
      dP_ij = z_ij c (g_i . v_j)          (gradient with respect to p_ij)
      D_i   = sum_j p_ij dP_ij            (equals g_i . o_i)
      dS_ij = p_ij (dP_ij - D_i)          (softmax Jacobian)
      dQ_i  = scale * sum_j dS_ij k_j
      dK_j += scale * sum_i dS_ij q_i
    Returns dq [Nq, d] and this head's contributions dk, dv [Nk, d] to its kv
    head (callers sum them over a grouped-query group).
    """
    n = k.shape[0]
    off = n - q.shape[0]
    rows = np.arange(q.shape[0], dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for ch in _chunks(rows, chunk):
        keys = candidate_keys(ch, n, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)
        if keys.size == 0:
            continue
        vis = visible(ch, keys, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)
        _, p, _ = _row_softmax(q[ch], k[keys], scale, vis, alibi_bias(ch, keys, alibi, off))
        g = do[ch]
        dv[keys] += _drop(p, ch, keys, dropout).T @ g
        dp = _drop(g @ v[keys].T, ch, keys, dropout)
        dd = (p * dp).sum(axis=1)
        ds = p * (dp - dd[:, None])
        dq[ch] = scale * (ds @ k[keys])
        dk[keys] += scale * (ds.T @ q[ch])
    return dq, dk, dv


def _heads(B, H, heads):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return [(int(b), int(h)) for b, h in heads]


def forward(q, k, v, scale, causal=False, block_mask=None, heads=None, rows=None, chunk=256,
            dropout_rate=0.0, seed=0, window=(-1, -1), alibi_slopes=None, elem_mask=None):
    """Attention forward over [B, H, Nq, d] queries and [B, Hkv, Nk, d] keys/values.

    Query head h reads kv head h // (H // Hkv). A block mask has
    ceil(Nq / 128) x ceil(Nk / 128) entries. With ``heads=None`` returns full
    o [B, H, R, d] and lse [B, H, R] (R = len(rows) or Nq); otherwise arrays
    stacked in the order of ``heads`` (a list of (b, h)): o [nh, R, d], lse [nh, R].
    A positive ``dropout_rate`` applies dropout with the generator keyed by
    ``seed`` (``oracle.dropout``); query head (b, h) draws stream b * H + h.
    ``elem_mask``: None or a boolean [Nq, Nk] visibility matrix shared by
    every batch and head.
    """
    B, H, _, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    hl = _heads(B, H, heads)
    outs, lses = [], []
    for b, h in hl:
        dr = (dropout_rate, seed, b * H + h) if dropout_rate > 0 else None
        o, l_ = head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, causal, block_mask, rows, chunk, dr,
                             window, None if alibi_slopes is None else alibi_slopes[h], elem_mask)
        outs.append(o)
        lses.append(l_)
    o = np.stack(outs)
    lse = np.stack(lses)
    if heads is None:
        R = o.shape[1]
        return o.reshape(B, H, R, o.shape[-1]), lse.reshape(B, H, R)
    return o, lse


def backward(q, k, v, do, scale, causal=False, block_mask=None, heads=None, chunk=256,
             dropout_rate=0.0, seed=0, window=(-1, -1), alibi_slopes=None, elem_mask=None):
    """Gradients of sum(O * dO) with respect to q, k, v (dropout as in ``forward``).

    With ``heads=None`` returns full dq [B, H, Nq, d], dk, dv [B, Hkv, Nk, d]
    (dk, dv summed over each kv head's group of query heads). With a list of
    (b, h) returns per-head arrays: dq [nh, Nq, d] and that query head's
    contributions to dk and dv [nh, Nk, d].
    """
    B, H, _, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    if heads is None:
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                dr = (dropout_rate, seed, b * H + h) if dropout_rate > 0 else None
                a, bk, bv = head_backward(q[b, h], k[b, h // G], v[b, h // G], do[b, h],
                                          scale, causal, block_mask, chunk, dr, window,
                                          None if alibi_slopes is None else alibi_slopes[h], elem_mask)
                dq[b, h] = a
                dk[b, h // G] += bk
                dv[b, h // G] += bv
        return dq, dk, dv
    res = [head_backward(q[b, h], k[b, h // G], v[b, h // G], do[b, h], scale, causal, block_mask, chunk,
                         (dropout_rate, seed, b * H + h) if dropout_rate > 0 else None, window,
                         None if alibi_slopes is None else alibi_slopes[h], elem_mask)
           for b, h in _heads(B, H, heads)]
    return tuple(np.stack(x) for x in zip(*res))


def _spans(cu, total):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to the packed length")
    return [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:])]


def forward_varlen(q, k, v, cu_q, cu_k, scale, causal=False, dropout_rate=0.0, seed=0, window=(-1, -1),
                   alibi_slopes=None):
    """Attention over packed variable-length sequences.

    q: [H, Tq, d], k, v: [Hkv, Tk, d]: per head, the rows of every sequence one
    after another; sequence b holds query rows cu_q[b]:cu_q[b + 1] and keys
    cu_k[b]:cu_k[b + 1]. Each sequence is an independent attention problem
    (causal alignment as in ``visible``, with that sequence's own lengths);
    with dropout, query head h of sequence b draws stream b * H + h, indexed by
    row and key positions within the sequence. Returns o [H, Tq, d], lse [H, Tq].
    """
    H, Tq, d = q.shape
    Hkv, Tk = k.shape[0], k.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    qs, ks = _spans(cu_q, Tq), _spans(cu_k, Tk)
    if len(qs) != len(ks):
        raise ValueError("cu_seqlens_q and cu_seqlens_k name different batch sizes")
    o = np.zeros((H, Tq, v.shape[2]))
    lse = np.full((H, Tq), -np.inf)
    for b, ((q0, q1), (k0, k1)) in enumerate(zip(qs, ks)):
        if q1 == q0:
            continue
        for h in range(H):
            dr = (dropout_rate, seed, b * H + h) if dropout_rate > 0 else None
            o[h, q0:q1], lse[h, q0:q1] = head_forward(q[h, q0:q1], k[h // G, k0:k1], v[h // G, k0:k1], scale,
                                                      causal, None, None, 256, dr, window,
                                                      None if alibi_slopes is None else alibi_slopes[h])
    return o, lse


def backward_varlen(q, k, v, do, cu_q, cu_k, scale, causal=False, dropout_rate=0.0, seed=0, window=(-1, -1),
                    alibi_slopes=None):
    """Gradients of sum(O * dO) for ``forward_varlen``: dq [H, Tq, d],
    dk, dv [Hkv, Tk, d] (summed over each kv head's group of query heads)."""
    H, Tq, d = q.shape
    Hkv, Tk = k.shape[0], k.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    qs, ks = _spans(cu_q, Tq), _spans(cu_k, Tk)
    if len(qs) != len(ks):
        raise ValueError("cu_seqlens_q and cu_seqlens_k name different batch sizes")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b, ((q0, q1), (k0, k1)) in enumerate(zip(qs, ks)):
        for h in range(H):
            dr = (dropout_rate, seed, b * H + h) if dropout_rate > 0 else None
            a, bk, bv = head_backward(q[h, q0:q1], k[h // G, k0:k1], v[h // G, k0:k1], do[h, q0:q1], scale,
                                      causal, None, 256, dr, window,
                                      None if alibi_slopes is None else alibi_slopes[h])
            dq[h, q0:q1] = a
            dk[h // G, k0:k1] += bk
            dv[h // G, k0:k1] += bv
    return dq, dk, dv
