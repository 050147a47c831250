"""Every deliberately broken copy of the backward oracle must fail at least one pin (CPU only)."""

import functools
import os

import pytest

import oracle
import oracle_bwd_pins

# (name, [(original text, replacement), ...]); each original must occur in fa_oracle_bwd.c
MUTANTS = [
    ("ds_drops_delta", [("dp[j] = p[j] * (acc - Di);", "dp[j] = p[j] * acc;")]),
    ("ds_sign", [("dp[j] = p[j] * (acc - Di);", "dp[j] = p[j] * (Di - acc);")]),
    ("dv_uses_ds", [("dvh[j * d + c] += p[j] * (double)doi[c];", "dvh[j * d + c] += dp[j] * (double)doi[c];")]),
    ("dq_drops_scale", [("dqh[i * d + c] += job->scale * dp[j] * (double)kh[j * d + c];",
                         "dqh[i * d + c] += dp[j] * (double)kh[j * d + c];")]),
    ("dk_uses_dout", [("dkh[j * d + c] += job->scale * dp[j] * (double)qi[c];",
                       "dkh[j * d + c] += job->scale * dp[j] * (double)doi[c];")]),
    ("dq_uses_v", [("dqh[i * d + c] += job->scale * dp[j] * (double)kh[j * d + c];",
                    "dqh[i * d + c] += job->scale * dp[j] * (double)vh[j * d + c];")]),
    ("softmax_not_normalised", [("        p[j] /= l;", "        p[j] /= 1.0;")]),
    ("causal_ignored", [("return causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;", "return Nk;")]),
    ("causal_excludes_diagonal", [("return causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;",
                                   "return causal ? (i > 0 ? (i < Nk ? i : Nk) : 1) : Nk;")]),
    ("delta_from_v", [("Di += (double)doi[c] * o[c];", "Di += (double)doi[c] * (double)vh[c];")]),
    ("keys_strided_by_queries", [("*kh = job->k + bh * Nk * d;", "*kh = job->k + bh * Nq * d;")]),
    ("dp_transposed_dims", [("acc += (double)doi[c] * (double)vh[j * d + c];",
                             "acc += (double)doi[c] * (double)vh[j * d + (d - 1 - c)];")]),
    ("window_left_off_by_one", [("l = i - job->win_left;", "l = i - job->win_left + 1;")]),
    ("window_right_off_by_one", [("h = i + job->win_right + 1;", "h = i + job->win_right;")]),
    ("padding_ignored", [("h = job->key_lens[b];", "h = h;")]),
    ("padding_of_first_batch", [("row_range(job, bh / job->H, i, &lo, &hi);", "row_range(job, 0, i, &lo, &hi);")]),
    ("empty_rows_take_every_key", [("continue; /* no visible key: O_i = 0, no gradient */",
                                    "{ lo = 0; hi = Nk; } /* mutant */")]),
]


def _mutant_source(subs):
    with open(os.path.join(os.path.dirname(oracle.__file__), "fa_oracle_bwd.c")) as f:
        src = f.read()
    for old, new in subs:
        assert old in src, f"mutation target not found: {old!r}"
        src = src.replace(old, new)
    return src


@pytest.mark.parametrize("name,subs", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_pins_catch_mutant(name, subs, tmp_path):
    src = tmp_path / f"{name}.c"
    src.write_text(_mutant_source(subs))
    lib = oracle.load_bwd(oracle.build_bwd(str(src), str(tmp_path / f"lib{name}.so")))
    bwd = functools.partial(oracle.attention_bwd, lib=lib)
    caught = []
    for pin in oracle_bwd_pins.ALL_PINS:
        try:
            pin(bwd)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
