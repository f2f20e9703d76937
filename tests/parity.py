"""Helpers that run the HIP path and the float64 oracle on the same seeded inputs
and compare them (used by the GPU parity tests and the smoke check).

Bars (the stated tolerances of the attention workloads):
* float32 outputs (O of a float32 run, and LSE always): max abs error <= 1e-5;
* bf16 / fp16 outputs: max abs error <= 2e-2;
* gradients: per-tensor relative Frobenius error <= 5e-2.
A row that sees no key must come back as O = 0 and LSE = -inf exactly.
"""

import math
import sys

import numpy as np
import torch

import oracle
from exact_attention_110_amd import binding
from exact_attention_110_amd import inputs as I

TOL_F32 = 1e-5
TOL_16 = 2e-2
TOL_LSE = 1e-5
TOL_GRAD = 5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def max_abs(a, b):
    return float(np.abs(a - b).max()) if a.size else 0.0


def check_lse(lse, ref, where, tol=TOL_LSE):
    """tol: one bar, or one per row (an array shaped like ref)."""
    assert lse.shape == ref.shape, where
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref)), f"{where}: -inf rows differ"
    assert np.all(np.isfinite(lse[fin])), f"{where}: non-finite LSE"
    err = max_abs(lse[fin], ref[fin])
    if np.ndim(tol) == 0:
        assert err <= tol, f"{where}: LSE max abs err {err:.3g} > {tol:.3g}"
    else:
        e, t = np.abs(lse[fin] - ref[fin]), np.asarray(tol)[fin]
        assert np.all(e <= t), (f"{where}: LSE err {float(e[np.argmax(e - t)]):.3g} over its bar "
                                f"{float(t[np.argmax(e - t)]):.3g}; rows over: {int((e > t).sum())}")
    return err


def alibi_lse_tol(ref):
    """LSE bar under a distance bias: the bias makes LSE large (hundreds, for
    rows far from every key), where one float32 rounding of the stored value is
    already 2^-24 |LSE| or more; the bar is 1e-5 plus two such roundings."""
    return TOL_LSE + 2.0 ** -22 * np.abs(np.where(np.isfinite(ref), ref, 0.0))


def check_out(o, ref, dtype, where):
    assert np.all(np.isfinite(o)), f"{where}: non-finite O"
    tol = TOL_F32 if dtype == "fp32" else TOL_16
    err = max_abs(o, ref)
    assert err <= tol, f"{where}: O max abs err {err:.3g} > {tol}"
    return err


def rel_frob(x, ref):
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    if den == 0.0:
        return num
    return num / den


def check_grad(g, ref, where):
    assert np.all(np.isfinite(g)), f"{where}: non-finite gradient"
    err = rel_frob(g, ref)
    assert err <= TOL_GRAD, f"{where}: relative Frobenius err {err:.3g} > {TOL_GRAD}"
    return err


def run_small(B, H, Hkv, N, d, dtype, causal, mask=None, seed=0, sigma=1.0, backward=True, scale=None,
              dropout_rate=0.0, drop_seed=0, rows_per_wave=0):
    """Full comparison (every output element) for a small seeded case;
    rows_per_wave 32 or 64 forces that 16-bit forward kernel."""
    where = f"B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} mask={mask is not None} seed={seed}"
    if dropout_rate:
        where += f" dropout={dropout_rate} drop_seed={drop_seed}"
    x = I.make_small(B, H, Hkv, N, d, dtype, seed, sigma, with_grad=backward)
    return run_given(x, dtype, causal, mask, backward, scale, where, dropout_rate=dropout_rate,
                     drop_seed=drop_seed, rows_per_wave=rows_per_wave)


def run_given(x, dtype, causal, mask=None, backward=True, scale=None, where="", lse_tol=TOL_LSE,
              dropout_rate=0.0, drop_seed=0, rows_per_wave=0):
    """Full comparison (every output element) on given CPU tensors q, k, v (and do);
    with a positive dropout_rate both sides drop with the generator keyed by drop_seed."""
    if rows_per_wave:
        where += f" rows_per_wave={rows_per_wave}"
    say("case", where)
    d = x["q"].shape[-1]
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    mt = None if mask is None else torch.from_numpy(mask).to(dev)
    o, lse = binding.forward(q, k, v, scale, causal, mt, dropout_rate=dropout_rate, seed=drop_seed,
                             rows_per_wave=rows_per_wave)
    torch.cuda.synchronize()
    qd, kd, vd = (np64(x[n]) for n in ("q", "k", "v"))
    oref, lref = oracle.forward(qd, kd, vd, scale, causal, mask, dropout_rate=dropout_rate, seed=drop_seed)
    res = {"o": check_out(np64(o), oref, dtype, where), "lse": check_lse(np64(lse), lref, where, lse_tol)}
    if backward and dtype != "fp32":
        do = x["do"].to(dev)
        dq, dk, dv = binding.backward(q, k, v, o, lse, do, scale, causal, mt, dropout_rate=dropout_rate,
                                      seed=drop_seed)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.backward(qd, kd, vd, np64(x["do"]), scale, causal, mask, dropout_rate=dropout_rate,
                                     seed=drop_seed)
        res["dq"] = check_grad(np64(dq), rq, where + " dq")
        res["dk"] = check_grad(np64(dk), rk, where + " dk")
        res["dv"] = check_grad(np64(dv), rv, where + " dv")
    return res


def run_cross(B, H, Hkv, Nq, Nk, d, dtype, causal, mask=None, seed=0, backward=True, dropout_rate=0.0,
              drop_seed=0, rows_per_wave=0):
    """Full comparison for Nq query rows over Nk keys (fa_forward_qk / fa_backward_qk)."""
    where = (f"B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal} mask={mask is not None} "
             f"seed={seed}")
    if dropout_rate:
        where += f" dropout={dropout_rate} drop_seed={drop_seed}"
    x = I.make_cross(B, H, Hkv, Nq, Nk, d, dtype, seed, with_grad=backward)
    return run_given(x, dtype, causal, mask, backward, None, where, dropout_rate=dropout_rate,
                     drop_seed=drop_seed, rows_per_wave=rows_per_wave)


def run_varlen(lens_q, lens_k, H, Hkv, d, dtype, causal, seed=0, backward=True, dropout_rate=0.0,
               drop_seed=0, max_q=None, max_k=None, window=(-1, -1), alibi_slopes=None):
    """Full comparison for a packed variable-length batch (fa_forward_varlen /
    fa_backward_varlen) against the oracle's per-sequence attention."""
    where = (f"lens_q={list(lens_q)} lens_k={list(lens_k)} H{H} Hkv{Hkv} d{d} {dtype} causal={causal} "
             f"window={tuple(window)} seed={seed}")
    if alibi_slopes is not None:
        where += f" alibi={np.round(np.asarray(alibi_slopes, dtype=np.float64), 4).tolist()}"
    if dropout_rate:
        where += f" dropout={dropout_rate} drop_seed={drop_seed}"
    say("case", where)
    x = I.make_packed(lens_q, lens_k, H, Hkv, d, dtype, seed, with_grad=backward)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    cq = torch.from_numpy(x["cu_q"]).to(dev)
    ck = torch.from_numpy(x["cu_k"]).to(dev)
    mq = max(1, max(lens_q)) if max_q is None else max_q
    mk = max(1, max(lens_k)) if max_k is None else max_k
    scale = 1.0 / math.sqrt(d)
    o, lse = binding.forward_varlen(q, k, v, cq, ck, mq, mk, scale, causal, dropout_rate=dropout_rate,
                                    seed=drop_seed, window=window, alibi_slopes=alibi_slopes)
    torch.cuda.synchronize()
    qd, kd, vd = (np64(x[n]) for n in ("q", "k", "v"))
    sl = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float64)
    oref, lref = oracle.forward_varlen(qd, kd, vd, x["cu_q"], x["cu_k"], scale, causal, dropout_rate, drop_seed,
                                       tuple(window), alibi_slopes=sl)
    ltol = TOL_LSE if sl is None else alibi_lse_tol(lref)
    res = {"o": check_out(np64(o), oref, dtype, where), "lse": check_lse(np64(lse), lref, where, ltol)}
    if backward and dtype != "fp32":
        do = x["do"].to(dev)
        dq, dk, dv = binding.backward_varlen(q, k, v, o, lse, do, cq, ck, mq, mk, scale, causal,
                                             dropout_rate=dropout_rate, seed=drop_seed, window=window,
                                             alibi_slopes=alibi_slopes)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.backward_varlen(qd, kd, vd, np64(x["do"]), x["cu_q"], x["cu_k"], scale, causal,
                                            dropout_rate, drop_seed, tuple(window), alibi_slopes=sl)
        res["dq"] = check_grad(np64(dq), rq, where + " dq")
        res["dk"] = check_grad(np64(dk), rk, where + " dk")
        res["dv"] = check_grad(np64(dv), rv, where + " dv")
    return res


def run_window(B, H, Hkv, Nq, Nk, d, dtype, causal, window, mask=None, seed=0, backward=True, dropout_rate=0.0,
               drop_seed=0, rows_per_wave=0, x=None, lse_tol=TOL_LSE):
    """Full comparison with a sliding-window band (fa_forward_qk / fa_backward_qk);
    x: given CPU inputs of that shape instead of the seeded ones."""
    where = (f"B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal} window={tuple(window)} "
             f"mask={mask is not None} seed={seed} rows_per_wave={rows_per_wave}")
    if dropout_rate:
        where += f" dropout={dropout_rate} drop_seed={drop_seed}"
    say("case", where)
    if x is None:
        x = I.make_cross(B, H, Hkv, Nq, Nk, d, dtype, seed, with_grad=backward)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    mt = None if mask is None else torch.from_numpy(mask).to(dev)
    o, lse = binding.forward(q, k, v, scale, causal, mt, dropout_rate=dropout_rate, seed=drop_seed, window=window,
                             rows_per_wave=rows_per_wave)
    torch.cuda.synchronize()
    qd, kd, vd = (np64(x[n]) for n in ("q", "k", "v"))
    oref, lref = oracle.forward(qd, kd, vd, scale, causal, mask, dropout_rate=dropout_rate, seed=drop_seed,
                                window=tuple(window))
    res = {"o": check_out(np64(o), oref, dtype, where), "lse": check_lse(np64(lse), lref, where, lse_tol)}
    if backward and dtype != "fp32":
        do = x["do"].to(dev)
        dq, dk, dv = binding.backward(q, k, v, o, lse, do, scale, causal, mt, dropout_rate=dropout_rate,
                                      seed=drop_seed, window=window)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.backward(qd, kd, vd, np64(x["do"]), scale, causal, mask, dropout_rate=dropout_rate,
                                     seed=drop_seed, window=tuple(window))
        res["dq"] = check_grad(np64(dq), rq, where + " dq")
        res["dk"] = check_grad(np64(dk), rk, where + " dk")
        res["dv"] = check_grad(np64(dv), rv, where + " dv")
    return res


def run_alibi(B, H, Hkv, Nq, Nk, d, dtype, causal, slopes, window=(-1, -1), mask=None, seed=0, backward=True,
              dropout_rate=0.0, drop_seed=0):
    """Full comparison with ALiBi slopes (fa_forward_qk / fa_backward_qk): O and
    gradients to the usual bars, LSE to ``alibi_lse_tol``."""
    sl = np.asarray(slopes, dtype=np.float32)
    where = (f"B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal} window={tuple(window)} "
             f"mask={mask is not None} seed={seed} alibi={np.round(sl.astype(np.float64), 4).tolist()}")
    if dropout_rate:
        where += f" dropout={dropout_rate} drop_seed={drop_seed}"
    say("case", where)
    x = I.make_cross(B, H, Hkv, Nq, Nk, d, dtype, seed, with_grad=backward)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    mt = None if mask is None else torch.from_numpy(mask).to(dev)
    st = torch.from_numpy(sl).to(dev)
    o, lse = binding.forward(q, k, v, scale, causal, mt, dropout_rate=dropout_rate, seed=drop_seed, window=window,
                             alibi_slopes=st)
    torch.cuda.synchronize()
    qd, kd, vd = (np64(x[n]) for n in ("q", "k", "v"))
    # the oracle takes the slopes the kernels read: the float32 values, widened
    sd = sl.astype(np.float64)
    oref, lref = oracle.forward(qd, kd, vd, scale, causal, mask, dropout_rate=dropout_rate, seed=drop_seed,
                                window=tuple(window), alibi_slopes=sd)
    res = {"o": check_out(np64(o), oref, dtype, where), "lse": check_lse(np64(lse), lref, where, alibi_lse_tol(lref))}
    if backward and dtype != "fp32":
        do = x["do"].to(dev)
        dq, dk, dv = binding.backward(q, k, v, o, lse, do, scale, causal, mt, dropout_rate=dropout_rate,
                                      seed=drop_seed, window=window, alibi_slopes=st)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.backward(qd, kd, vd, np64(x["do"]), scale, causal, mask, dropout_rate=dropout_rate,
                                     seed=drop_seed, window=tuple(window), alibi_slopes=sd)
        res["dq"] = check_grad(np64(dq), rq, where + " dq")
        res["dk"] = check_grad(np64(dk), rk, where + " dk")
        res["dv"] = check_grad(np64(dv), rv, where + " dv")
    return res


# The FP8 matrix instruction (v_mfma_f32_32x32x64_f8f6f4) sums its 64 exact
# E4M3 products less precisely than float32 does: measured over 65536 random
# dot products, its error reached 2294 * 2^-24 * sum|products| (a sequential
# float32 sum: 2.45 * 2^-24). The bars below take FP8_SUM = 2^-11 relative to
# sum|products|, 3.6 times the largest measured, per score.
FP8_SUM = 2.0 ** -11


def fp8_score_error(qd, kd, scale, rows=None):
    """Per-row bound on the error of any of the row's scores."""
    qs = qd if rows is None else qd[rows]
    return FP8_SUM * scale * (np.abs(qs) @ np.abs(kd).T).max(axis=1)


def fp8_bound(qd, kd, vd, scale, causal, o_ref, rows=None):
    """Per-element bound on |O - O_ref| of the FP8 forward, derived from its
    arithmetic: each probability p (relative to its row maximum) is rounded to
    E4M3 before it weights V: at most 2^-4 p for a normal code, and for
    p < 2^-6, where the code may be subnormal (spacing 2^-9), at most
    max(2^-4 p, min(p, 2^-10)). The row is divided by l = 1 / (normalised
    maximum), so that part is P_max[r] * sum_j e_j |v_jc|. Score errors ds
    (``fp8_score_error``) change every weight by a factor within exp(+-2 ds)
    (the score and the normaliser), adding 2.1 ds sum_j P_j |v_jc|; the 16-bit
    rounding of O adds 2^-8 |O| (half an ulp and the float32 sums), and 2e-5
    covers the float32 exponentials."""
    p, _ = oracle.head_probabilities(qd, kd, scale, causal, rows=rows)
    pmax = p.max(axis=1, keepdims=True)
    rel = np.divide(p, pmax, out=np.zeros_like(p), where=pmax > 0)
    e = np.where(rel >= 2.0 ** -6, 2.0 ** -4 * rel, np.maximum(2.0 ** -4 * rel, np.minimum(rel, 2.0 ** -10)))
    ds = fp8_score_error(qd, kd, scale, rows)[:, None]
    return pmax * (e @ np.abs(vd)) + 2.1 * ds * (p @ np.abs(vd)) + 2.0 ** -8 * np.abs(o_ref) + 2e-5


def fp8_lse_bound(qd, kd, scale, lse_ref, rows=None):
    """Bound on |LSE - LSE_ref| of the FP8 forward: LSE moves no more than its
    largest score error (``fp8_score_error``); the float32 running sum of n
    probabilities adds n 2^-24 relative to l, and the float32 steps of the
    scale product, exp2, log2 and the final multiply a few ulps of |LSE|. The
    float32 bar 1e-5 applies where it is the larger."""
    n = kd.shape[0]
    b = (fp8_score_error(qd, kd, scale, rows) + (n + 8) * 2.0 ** -24
         + 8 * 2.0 ** -24 * np.abs(np.nan_to_num(lse_ref)) + 1e-6)
    return np.maximum(b, TOL_LSE)


def run_fp8(B, H, Hkv, N, d, causal, seed=0, out_dtype="bf16", heads=None, rows=None):
    """FP8 forward against the oracle on the decoded inputs: O within the
    derived per-element bound, LSE within 1e-5."""
    where = f"fp8 B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} out={out_dtype} seed={seed}"
    say("case", where)
    import oracle.fp8 as F8
    x = I.make_fp8(B, H, Hkv, N, d, seed)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[out_dtype]
    o, lse = binding.forward_fp8(q, k, v, x["q_descale"], x["k_descale"], x["v_descale"], scale, causal,
                                 out_dtype=tdt)
    torch.cuda.synchronize()
    o, lse = np64(o), np64(lse)
    G = H // Hkv
    hl = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    worst = 0.0
    for b, h in hl:
        qd = F8.e4m3_decode(x["q"][b, h].numpy()) * x["q_descale"]
        kd = F8.e4m3_decode(x["k"][b, h // G].numpy()) * x["k_descale"]
        vd = F8.e4m3_decode(x["v"][b, h // G].numpy()) * x["v_descale"]
        oref, lref = oracle.head_forward(qd, kd, vd, scale, causal, rows=rows)
        ob = o[b, h] if rows is None else o[b, h][rows]
        lb = lse[b, h] if rows is None else lse[b, h][rows]
        assert np.all(np.isfinite(ob)), f"{where}: non-finite O"
        bound = fp8_bound(qd, kd, vd, scale, causal, oref, rows)
        err = np.abs(ob - oref)
        ratio = float((err / bound).max())
        worst = max(worst, ratio)
        assert ratio <= 1.0, f"{where} head ({b},{h}): O error {float(err.max()):.3g} exceeds its bound (ratio {ratio:.3g})"
        lb_tol = fp8_lse_bound(qd, kd, scale, lref, rows)
        fin = np.isfinite(lref)
        assert np.array_equal(np.isneginf(lb), np.isneginf(lref)), f"{where}: -inf rows differ"
        lerr = np.abs(lb[fin] - lref[fin])
        if not np.all(lerr <= lb_tol[fin]):
            rr = np.flatnonzero(fin)[np.argmax(lerr - lb_tol[fin])]
            raise AssertionError(f"{where} head ({b},{h}): LSE error {float(np.abs(lb[rr] - lref[rr])):.3g} at row "
                                 f"{rr} (LSE {float(lref[rr]):.4f}, kernel {float(lb[rr]):.6f}) exceeds its bound "
                                 f"{float(lb_tol[rr]):.3g}; rows over the bound: {int((lerr > lb_tol[fin]).sum())}")
    say(f"  worst error / bound {worst:.3f}")
    return worst
