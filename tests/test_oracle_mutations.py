"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the independent pins catch every one of them.

Each mutation is a textual edit of ``oracle/attention.py``; the edited source
is executed as a throwaway module. The pins used here exclude the
scalar-loop-vs-vectorised comparison, so a mistake must be caught by a closed
form, an invariant, a library reduction or a hand-derived fixture.
"""

import os
import types

import pytest

from oracle_pins import INDEPENDENT_PINS, run_pin

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "attention.py")

# (id, original text, mistaken text); when the same line exists in both the
# vectorised and the scalar forms, both are edited.
MUTATIONS = [
    ("no_position_offset", "p = rows + (L - S)", "p = rows"),
    ("no_position_offset_bf", "p = i + L - S", "p = i"),
    ("gqa_modulo", "g = h // G", "g = h % Hkv"),
    ("gqa_modulo_bf", "g = h // (H // Hkv)", "g = h % Hkv"),
    ("distance_sign", "d = p[:, None] - j[None, :]", "d = j[None, :] - p[:, None]"),
    ("distance_sign_bf", "d = p - j", "d = j - p"),
    ("extent_inclusive", "(d >= 0) & (d < rel_extent)", "(d >= 0) & (d <= rel_extent)"),
    ("extent_no_lower_bound_bf", "bias = rl[t, h, d] if 0 <= d < rel_extent else 0.0",
     "bias = rl[t, h, d] if d < rel_extent else 0.0"),
    ("extent_inclusive_bf", "bias = rl[t, h, d] if 0 <= d < rel_extent else 0.0",
     "bias = rl[t, h, min(d, rel_extent - 1)] if 0 <= d <= rel_extent else 0.0"),
    ("scale_dropped", "s = softmax_scale * (qh @ K.T)", "s = (qh @ K.T)"),
    ("scale_dropped_bf", "scores.append(softmax_scale * dot + bias)", "scores.append(dot + bias)"),
    ("bias_scaled", "s = s + np.where(in_range, bias, 0.0)",
     "s = s + softmax_scale * np.where(in_range, bias, 0.0)"),
    ("bias_scaled_bf", "scores.append(softmax_scale * dot + bias)",
     "scores.append(softmax_scale * (dot + bias))"),
    ("causal_excludes_self", "hi = min(hi, p + 1)", "hi = min(hi, p)"),
    ("causal_excludes_self_bf", "if causal and j > p:", "if causal and j >= p:"),
    ("window_off_by_one", "lo = max(lo, p - wl)", "lo = max(lo, p - wl + 1)"),
    ("window_right_off_by_one", "hi = min(hi, p + wr + 1)", "hi = min(hi, p + wr)"),
    ("local_bias_row", "R = _f64(rel_logits[t0 + rows, h, :]) if E > 0 else None",
     "R = _f64(rel_logits[rows, h, :]) if E > 0 else None"),
    ("pv_uses_keys", "o[has] = (w[has] @ Vb[:, g, :]) / l[has, None]",
     "o[has] = (w[has] @ Kb[:, g, :]) / l[has, None]"),
    ("no_normalisation", "o[has] = (w[has] @ Vb[:, g, :]) / l[has, None]",
     "o[has] = (w[has] @ Vb[:, g, :])"),
    ("page_slot_swap", "return cache[pages].reshape(npages * bs, cache.shape[2], cache.shape[3])[:L]",
     "return cache[pages].transpose(0, 1).reshape(npages * bs, cache.shape[2], cache.shape[3])[:L]"),
    ("combine_unweighted", "out[t0 + r, h, :] = sum(math.exp(lk - LSE) * pk for lk, pk in zip(lses, parts))",
     "out[t0 + r, h, :] = sum(pk for lk, pk in zip(lses, parts)) / len(parts)"),
    ("combine_lse_no_log", "lses.append(m_k + math.log(l_k))", "lses.append(m_k + l_k)"),
    # the row log-sum-exp returned with return_lse=True
    ("lse_max_plus_sum", "m + np.log(np.where(has, l, 1.0))", "m + np.where(has, l, 1.0)"),
    ("lse_log2", "m + np.log(np.where(has, l, 1.0))", "m + np.log2(np.where(has, l, 1.0))"),
    ("lse_max_dropped", "m + np.log(np.where(has, l, 1.0))", "np.log(np.where(has, l, 1.0))"),
    ("lse_empty_zero", "np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)",
     "np.where(has, m + np.log(np.where(has, l, 1.0)), 0.0)"),
    ("lse_sum_without_max", "l = w.sum(axis=1)", "l = w.sum(axis=1) * np.exp(m)"),
    ("window_left_zero_ignored", "    if wl >= 0:\n        lo = max(lo, p - wl)",
     "    if wl > 0:\n        lo = max(lo, p - wl)"),
    ("empty_row_nan", "o = np.zeros((len(rows), D))", "o = np.full((len(rows), D), np.nan)"),
    ("pages_of_first_request", "pages = block_table[b, :npages]", "pages = block_table[0, :npages]"),
    ("query_rows_no_offset", "qh = _f64(q[t0 + rows, h, :])", "qh = _f64(q[rows, h, :])"),
    ("output_rows_no_offset", "out[t0 + rows, h, :] = o", "out[rows, h, :] = o"),
]


def _mutant(orig, new):
    src = open(SRC).read()
    assert orig in src, orig
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src.replace(orig, new), SRC + ":mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mid,orig,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(mid, orig, new):
    mod = _mutant(orig, new)
    caught = []
    for pin in INDEPENDENT_PINS:
        try:
            run_pin(pin, mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"mutation {mid} was not caught by any independent pin"
