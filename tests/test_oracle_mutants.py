"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that the pins catch every one of them: evidence that the pins constrain the
oracle's arithmetic, not only that the oracle passes them."""

import functools
import os

import pytest

import oracle
import oracle_pins

# (name, [(original text, replacement), ...]); each original must occur in fa_oracle.c
MUTANTS = [
    ("scale_dropped", [("return scale * acc;", "return acc;")]),
    ("score_sign", [("acc += (double)qi[c] * (double)kj[c];", "acc -= (double)qi[c] * (double)kj[c];")]),
    ("feature_index_reversed", [("(double)kj[c]", "(double)kj[d - 1 - c]")]),
    ("accumulate_in_float", [("double acc = 0.0;", "float acc = 0.0f;")]),
    ("causal_excludes_diagonal", [("return causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;",
                                   "return causal ? (i > 0 ? (i < Nk ? i : Nk) : 1) : Nk;")]),
    ("causal_sees_next_key", [("return causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;",
                               "return causal ? (i + 2 < Nk ? i + 2 : Nk) : Nk;")]),
    ("causal_ignored", [("return causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;", "return Nk;")]),
    ("causal_bottom_right", [("int64_t nvis = visible_keys(i, Nk, job->causal);",
                              "int64_t nvis = visible_keys(i + (Nk > Nq ? Nk - Nq : 0), Nk, job->causal);")]),
    ("keys_strided_by_query_length", [("const float *kh = job->k + bh * Nk * d;",
                                       "const float *kh = job->k + bh * Nq * d;")]),
    ("lse_base2", [("*lse_out = m + log(l);", "*lse_out = m + log2(l);")]),
    ("lse_drops_max", [("*lse_out = m + log(l);", "*lse_out = log(l);")]),
    ("no_max_subtraction", [("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
                            ("*lse_out = m + log(l);", "*lse_out = log(l);")]),
    ("no_normalisation", [("        o_row[c] /= l;\n    *lse_out", "        o_row[c] /= 1.0;\n    *lse_out")]),
    ("value_row_reversed", [("const float *vj = vh + j * d;", "const float *vj = vh + (nvis - 1 - j) * d;")]),
    ("online_sum_not_rescaled", [("l *= alpha;", "l *= 1.0;")]),
    ("online_alpha_inverted", [("exp(m - m_new)", "exp(m_new - m)")]),
    ("online_output_not_rescaled", [("o_row[c] *= alpha;", "o_row[c] *= 1.0;")]),
    ("window_left_off_by_one", [("l = i - job->win_left;", "l = i - job->win_left + 1;")]),
    ("window_right_off_by_one", [("h = i + job->win_right + 1;", "h = i + job->win_right;")]),
    ("padding_ignored", [("h = job->key_lens[b];", "h = h;")]),
    ("padding_of_first_batch", [("visible_range(job, bh / job->H, i, &k_lo, &k_hi);",
                                 "visible_range(job, 0, i, &k_lo, &k_hi);")]),
    ("window_keys_not_offset", [("const float *kv0 = kh + k_lo * d, *vv0 = vh + k_lo * d;",
                                 "const float *kv0 = kh, *vv0 = vh;")]),
    ("empty_row_lse_zero", [("*lse_out = -INFINITY;", "*lse_out = 0.0;")]),
]


def _mutant_source(subs):
    with open(os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")) as f:
        src = f.read()
    for old, new in subs:
        assert old in src, f"mutation target not found: {old!r}"
        src = src.replace(old, new, 1) if old.startswith("*lse_out") else src.replace(old, new)
    return src


@pytest.mark.parametrize("name,subs", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, subs, tmp_path):
    src = tmp_path / f"{name}.c"
    src.write_text(_mutant_source(subs))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / f"lib{name}.so")))
    fwd = functools.partial(oracle.attention_fwd, lib=lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(fwd)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
