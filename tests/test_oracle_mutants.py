"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (on the CPU only: the copy is executed
as a fresh module and never touches the GPU path) and checks that at least one pin of
tests/oracle_pins.py fails on it.  A mutant that slipped past every pin would mean the pins do not
constrain that part of the oracle.
"""

import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "attention.py")

# (name, text in the oracle, planted replacement)
MUTANTS = [
    ("dropped_scale", "s = scale * (q @ k.T)", "s = (q @ k.T)"),
    ("mask_off_by_one", "s = np.where(j > q_offset + i, -np.inf, s)",
     "s = np.where(j >= q_offset + i, -np.inf, s)"),
    ("mask_transposed", "s = np.where(j > q_offset + i, -np.inf, s)",
     "s = np.where(j < q_offset + i, -np.inf, s)"),
    ("decode_offset_ignored", "s = np.where(j > q_offset + i, -np.inf, s)",
     "s = np.where(j > i, -np.inf, s)"),
    ("brute_offset_ignored", "if (not causal) or j <= q_offset + i]", "if (not causal) or j <= i]"),
    ("merge_unweighted", "o = np.sum((w / tot[None, :])[:, :, None] * outs, axis=0)",
     "o = np.mean(outs, axis=0)"),
    ("merge_lse_no_max", "lse = mx + np.log(tot)", "lse = np.log(tot)"),
    ("split_offset_not_shifted", "s = scores_head64(q, k[b0:b1], causal, scale, q_offset - b0)",
     "s = scores_head64(q, k[b0:b1], causal, scale, q_offset)"),
    ("lse_without_max", "lse = m + np.log(l)", "lse = np.log(l)"),
    ("unnormalised_p", "p = e / l[:, None]", "p = e"),
    ("dv_untransposed", "dv = p.T @ do", "dv = p @ do"),
    ("dp_wrong_operand", "dp = do @ v.T", "dp = do @ do.T"),
    ("ds_no_row_term", "ds = p * (dp - row_dot[:, None])", "ds = p * dp"),
    ("ds_sign", "ds = p * (dp - row_dot[:, None])", "ds = p * (row_dot[:, None] - dp)"),
    ("dq_no_scale", "dq = scale * (ds @ k)", "dq = (ds @ k)"),
    ("dk_untransposed", "dk = scale * (ds.T @ q)", "dk = scale * (ds @ q)"),
    ("online_no_acc_rescale", "acc = alpha[:, None] * acc + p @ v[c0:c1]", "acc = acc + p @ v[c0:c1]"),
    ("online_no_l_rescale", "l = alpha * l + np.sum(p, axis=1)", "l = l + np.sum(p, axis=1)"),
    ("online_mask_off_by_one", "s = np.where(j > i, -np.inf, s)\n            m_new",
     "s = np.where(j >= i + 1, -np.inf, s)\n            s = np.where(j == i, -np.inf, s)\n            m_new"),
    ("rows_causal_end", "end = i + 1 if causal else k.shape[0]", "end = i if causal else k.shape[0]"),
    ("rows_no_scale", "s = scale * (k[:end] @ q[i])", "s = (k[:end] @ q[i])"),
    ("rows_dq_no_row_term", "ds = p * (dp - np.sum(p * dp))", "ds = p * dp"),
    ("rows_dq_wrong_operand", "dp = v[:end] @ do[i]", "dp = k[:end] @ do[i]"),
    ("driver_wrong_head", "o[b, h], lse[b, h] = attention_head_fwd64(q[b, h], k[b, h], v[b, h], causal, scale)",
     "o[b, h], lse[b, h] = attention_head_fwd64(q[b, h], k[b, 0], v[b, h], causal, scale)"),
]


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # AssertionError, or a crash caused by the mistake
            failures.append(f"{pin.__name__}: {type(exc).__name__}")
    assert failures, f"mutant {name} passed every pin"
