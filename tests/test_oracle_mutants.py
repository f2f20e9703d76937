"""Plant plausible mistakes in a copy of the oracle and check that a pin catches each.

Each mutant is the oracle's source with one textual edit, loaded as a separate
module on the CPU; the pins in ``oracle_pins`` are then run against it. A
mutant that every pin accepts would mean the pins leave that part of the
oracle unchecked.
"""

import importlib.util
import os
import types

import pytest

import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "causal_strict": ("a &= keys[None, :] <= rows[:, None]", "a &= keys[None, :] < rows[:, None]"),
    "causal_reversed": ("a &= keys[None, :] <= rows[:, None]", "a &= keys[None, :] >= rows[:, None]"),
    "mask_transposed": ("bm[(rows // block)[:, None], (keys // block)[None, :]]",
                        "bm[(keys // block)[None, :], (rows // block)[:, None]]"),
    "scale_dropped": ("s = scale * (q_rows @ k_keys.T)", "s = q_rows @ k_keys.T"),
    "lse_without_max": ("m0 + np.log(np.where(has, ssum, 1.0))", "np.log(np.where(has, ssum, 1.0))"),
    "output_uses_keys": ("o[pos:pos + ch.size] = _drop(p, ch, keys, dropout) @ v[keys]",
                         "o[pos:pos + ch.size] = _drop(p, ch, keys, dropout) @ k[keys]"),
    "dv_wrong_operand": ("dv[keys] += _drop(p, ch, keys, dropout).T @ g", "dv[keys] += _drop(p, ch, keys, dropout).T @ q[ch]"),
    "ds_sign": ("ds = p * (dp - dd[:, None])", "ds = p * (dp + dd[:, None])"),
    "ds_drops_p": ("ds = p * (dp - dd[:, None])", "ds = (dp - dd[:, None])"),
    "dd_drops_p": ("dd = (p * dp).sum(axis=1)", "dd = dp.sum(axis=1)"),
    "dk_missing_scale": ("dk[keys] += scale * (ds.T @ q[ch])", "dk[keys] += ds.T @ q[ch]"),
    "dq_transposed_keys": ("dq[ch] = scale * (ds @ k[keys])", "dq[ch] = scale * (ds @ v[keys])"),
    "gqa_modulo": ("o, l_ = head_forward(q[b, h], k[b, h // G], v[b, h // G]",
                   "o, l_ = head_forward(q[b, h], k[b, h % Hkv], v[b, h % Hkv]"),
    "gqa_backward_modulo": ("dk[b, h // G] += bk", "dk[b, h % Hkv] += bk"),
    "candidate_keys_short": ("keys = keys[keys <= rows.max() + offset]", "keys = keys[keys < rows.max() + offset]"),
    "candidate_keys_no_offset": ("keys = keys[keys <= rows.max() + offset]", "keys = keys[keys <= rows.max()]"),
    "offset_sign": ("off = n - q.shape[0]", "off = q.shape[0] - n"),
    "offset_top_left_forward": ("        if keys.size:\n            vis = visible(ch, keys, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)",
                                "        if keys.size:\n            vis = visible(ch, keys, causal, block_mask, window=window, elem_mask=elem_mask)"),
    "offset_top_left_backward": ("        vis = visible(ch, keys, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)\n        _, p, _ =",
                                 "        vis = visible(ch, keys, causal, block_mask, window=window, elem_mask=elem_mask)\n        _, p, _ ="),
    "varlen_keys_from_query_spans": ("head_forward(q[h, q0:q1], k[h // G, k0:k1], v[h // G, k0:k1]",
                                     "head_forward(q[h, q0:q1], k[h // G, q0:q1], v[h // G, q0:q1]"),
    "window_left_strict": ("a &= keys[None, :] >= rows[:, None] + offset - left",
                           "a &= keys[None, :] > rows[:, None] + offset - left"),
    "window_left_sign": ("a &= keys[None, :] >= rows[:, None] + offset - left",
                         "a &= keys[None, :] >= rows[:, None] + offset + left"),
    "window_right_ignores_offset": ("a &= keys[None, :] <= rows[:, None] + offset + right",
                                    "a &= keys[None, :] <= rows[:, None] + right"),
    "window_candidates_short": ("keys = keys[keys >= rows.min() + offset - window[0]]",
                                "keys = keys[keys > rows.min() + offset - window[0]]"),
    "window_dropped_in_backward": ("        vis = visible(ch, keys, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)\n        _, p, _ =",
                                   "        vis = visible(ch, keys, causal, block_mask, offset=off, elem_mask=elem_mask)\n        _, p, _ ="),
    "elem_mask_transposed": ("np.asarray(elem_mask, dtype=bool)[rows[:, None], keys[None, :]]",
                             "np.asarray(elem_mask, dtype=bool).T[rows[:, None], keys[None, :]]"),
    "elem_mask_inverted": ("a &= np.asarray(elem_mask, dtype=bool)[rows[:, None], keys[None, :]]",
                           "a &= ~np.asarray(elem_mask, dtype=bool)[rows[:, None], keys[None, :]]"),
    "elem_mask_dropped_in_backward": ("        vis = visible(ch, keys, causal, block_mask, offset=off, window=window, elem_mask=elem_mask)\n        _, p, _ =",
                                      "        vis = visible(ch, keys, causal, block_mask, offset=off, window=window)\n        _, p, _ ="),
    "elem_mask_candidates_first_row": ("keys = keys[np.asarray(elem_mask, dtype=bool)[rows].any(axis=0)[keys]]",
                                       "keys = keys[np.asarray(elem_mask, dtype=bool)[rows[:1]].any(axis=0)[keys]]"),
    "alibi_sign": ("return -float(slope) * np.abs(", "return float(slope) * np.abs("),
    "alibi_no_abs": ("np.abs((rows[:, None] + offset) - keys[None, :]).astype(np.float64)",
                     "((rows[:, None] + offset) - keys[None, :]).astype(np.float64)"),
    "alibi_no_offset": ("np.abs((rows[:, None] + offset) - keys[None, :])", "np.abs((rows[:, None]) - keys[None, :])"),
    "alibi_dropped_in_backward": ("_, p, _ = _row_softmax(q[ch], k[keys], scale, vis, alibi_bias(ch, keys, alibi, off))",
                                  "_, p, _ = _row_softmax(q[ch], k[keys], scale, vis)"),
    "varlen_dk_overwrite": ("dk[h // G, k0:k1] += bk", "dk[h // G, k0:k1] = bk"),
    "varlen_dropout_stream": ("dr = (dropout_rate, seed, b * H + h) if dropout_rate > 0 else None\n            o[h, q0:q1]",
                              "dr = (dropout_rate, seed, h) if dropout_rate > 0 else None\n            o[h, q0:q1]"),
    "dropout_unscaled": ("return np.where(z, p * _dropout.keep_scale(rate), 0.0)", "return np.where(z, p, 0.0)"),
    "dropout_scaled_by_rate": ("return np.where(z, p * _dropout.keep_scale(rate), 0.0)",
                               "return np.where(z, p / rate, 0.0)"),
    "dropout_dp_unmasked": ("dp = _drop(g @ v[keys].T, ch, keys, dropout)", "dp = g @ v[keys].T"),
    "dropout_dv_undropped": ("dv[keys] += _drop(p, ch, keys, dropout).T @ g", "dv[keys] += p.T @ g"),
    "dropout_before_softmax": ("o[pos:pos + ch.size] = _drop(p, ch, keys, dropout) @ v[keys]",
                               "o[pos:pos + ch.size] = (lambda r: r / np.maximum(r.sum(1, keepdims=True), 1e-300))"
                               "(_drop(p, ch, keys, dropout)) @ v[keys]"),
}


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, old
    src = src.replace(old, new)
    mod = types.ModuleType("oracle.attention_mutant")
    mod.__file__ = SRC
    mod.__package__ = "oracle"  # its relative import of oracle.dropout resolves
    exec(compile(src, SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod = _load_mutant(*MUTANTS[name])
    monkeypatch.setattr(P, "A", mod)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception:          # an assertion or a crash both expose the mistake
            caught.append(pin.__name__)
    assert caught, f"no pin detects mutant {name}"


SRC_FP8 = os.path.join(os.path.dirname(SRC), "fp8.py")

MUTANTS_FP8 = {
    "e4m3_bias_8": ("(e - 7)", "(e - 8)"),
    "e4m3_subnormal_exponent": ("np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)"),
    "e4m3_no_nan": ("return np.where((c & 0x7F) == 0x7F, np.nan, v)", "return v"),
    "e4m3_sign_lost": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = 1.0"),
    "fp8_k_descale_dropped": ("k = e4m3_decode(k8) * float(k_descale)", "k = e4m3_decode(k8)"),
    "fp8_v_descale_on_q": ("q = e4m3_decode(q8) * float(q_descale)",
                           "q = e4m3_decode(q8) * float(q_descale) * float(v_descale)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS_FP8))
def test_fp8_mutant_is_caught(name, monkeypatch):
    import sys
    import oracle
    old, new = MUTANTS_FP8[name]
    src = open(SRC_FP8).read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle.fp8")
    mod.__file__ = SRC_FP8
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), SRC_FP8 + " (mutant)", "exec"), mod.__dict__)
    monkeypatch.setitem(sys.modules, "oracle.fp8", mod)
    monkeypatch.setattr(oracle, "fp8", mod)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin detects mutant {name}"
