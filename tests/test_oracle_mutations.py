"""The oracle's pins must be strong enough to catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's C source (on the CPU),
builds it, routes the oracle through that build and runs the pins that should object.
A mutant that passes every listed pin fails this test.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as obuild

from tests import test_oracle_attention as A
from tests import test_oracle_codec as C
from tests import test_oracle_rope as R

MUTANTS = [
    ("rotation sign", "const double complex z = CMPLX(ora_f16_to_f64(x[re_at]), ora_f16_to_f64(x[im_at]));",
     "const double complex z = CMPLX(ora_f16_to_f64(x[re_at]), -ora_f16_to_f64(x[im_at]));",
     [R.test_pair0_turns_by_position_radians_textbook, R.test_plain_matches_complex_multiplication]),
    ("rotation direction", "factor[j] = rp->inverse ? conj(f) : f;", "factor[j] = rp->inverse ? f : conj(f);",
     [R.test_pair0_turns_by_position_radians_textbook, R.test_plain_matches_complex_multiplication]),
    ("frequency exponent", "-2.0 * (double)j / (double)rp->n_rot", "-1.0 * (double)j / (double)rp->n_rot",
     [R.test_frequency_schedule_textbook, R.test_plain_matches_complex_multiplication]),
    ("exponent uses head dim", "-2.0 * (double)j / (double)rp->n_rot", "-2.0 * (double)j / 128.0",
     [R.test_tail_half_width_schedule]),
    ("rotate the head start", "const int o = d - rp->n_rot;", "const int o = 0;",
     [R.test_tail_half_width_schedule, R.test_yarn_position_zero_scales_by_mscale]),
    ("YaRN mix swapped", "w = omega * (rp->freq_scale * (1.0 - gamma) + gamma);",
     "w = omega * (rp->freq_scale * gamma + (1.0 - gamma));",
     [R.test_yarn_limits_equal_plain_rotation]),
    ("mscale dropped", "f = rp->mscale * CMPLX(cos(theta), sin(theta));", "f = CMPLX(cos(theta), sin(theta));",
     [R.test_pair_norm_scaled_by_mscale_only, R.test_yarn_position_zero_scales_by_mscale]),
    ("half-split partner adjacent", "const int64_t im_at = rp->pairing ? re_at + half : re_at + 1;",
     "const int64_t im_at = rp->pairing ? re_at + 1 : re_at + 1;",
     [R.test_half_split_is_adjacent_rotation_of_permuted_dims,
      R.test_half_split_matches_complex_multiplication]),
    ("half-split pairs from the head start", "const int64_t re_at = head + o + (rp->pairing ? j : 2 * j);",
     "const int64_t re_at = head + (rp->pairing ? j : o + 2 * j);",
     [R.test_half_split_tail_keeps_head_dims]),
    ("inverse ignored", "factor[j] = rp->inverse ? conj(f) : f;", "factor[j] = f;",
     [R.test_inverse_at_pos_is_forward_at_minus_pos, R.test_inverse_undoes_forward_in_fp64]),
    ("table column shifted", "(double)rp->cos_table[(int64_t)p * half + j]",
     "(double)rp->cos_table[(int64_t)p * half + (j + 1) % half]",
     [R.test_table_rotation_closed_form]),
    ("table rows not by position", "(double)rp->sin_table[(int64_t)p * half + j]",
     "(double)rp->sin_table[(int64_t)(r % rp->table_rows) * half + j]",
     [R.test_table_gather_follows_positions, R.test_table_rotation_closed_form]),
    ("corr dim without 2", "(2.0 * M_PI * beta)", "(M_PI * beta)",
     [R.test_yarn_correction_dims_turn_beta_circles]),
    ("ramp inverted", "    return 1.0 - along;", "    return along;",
     [R.test_yarn_ramp_endpoints_and_linearity]),
    ("unit parameter set ignored", "return unit_set ? &sets[unit_set[u]] : &sets[0];", "return &sets[0];",
     [A.test_unit_parameter_sets_equal_separate_calls]),
    ("causal mask off by one", "const int nvis = lens[u] + tt + 1;",
     "const int nvis = lens[u] + tt > 0 ? lens[u] + tt : 1;",
     [A.test_zero_query_gives_prefix_mean, A.test_brute_force_torch_float64]),
    ("no causal mask", "const int nvis = lens[u] + tt + 1;", "const int nvis = L;",
     [A.test_zero_query_gives_prefix_mean]),
    ("GQA head mapping", "const int g = h / G;", "const int g = h % hkv;",
     [A.test_brute_force_torch_float64, A.test_single_token_returns_its_value_row]),
    ("scale dropped", "row[j] = (j < nvis) ? scale * row[j] : -INFINITY;",
     "row[j] = (j < nvis) ? row[j] : -INFINITY;",
     [A.test_brute_force_torch_float64]),
    ("softmax not normalised", "row[j] /= sum;", "row[j] /= 1.0;",
     [A.test_probabilities_sum_to_one]),
    ("decode skips the new key", "const int nk = lens[u] + 1;", "const int nk = lens[u] > 0 ? lens[u] : 1;",
     [A.test_prefill_equals_successive_decodes]),
    ("decode scale dropped", "s[j] = scale * s[j];", "s[j] = s[j];",
     [A.test_prefill_equals_successive_decodes]),
    ("append at row 0", "const int64_t dst = (((int64_t)u * hkv + g) * s_cap + lens[u] + tt) * d;",
     "const int64_t dst = (((int64_t)u * hkv + g) * s_cap + tt) * d;",
     [A.test_append_writes_only_its_rows]),
    ("rounding truncates", "nearbyint(a / quantum)", "floor(a / quantum)",
     [C.test_encode_midpoints_ties_to_even]),
    ("f16 decode as bf16-style shift", "v = ldexp((double)(m + 1024), e - 25);",
     "v = ldexp((double)(m + 1024), e - 24);",
     [C.test_decode_every_bit_pattern]),
    ("score dims out of order", "dot[j] += qi * ki[j];", "dot[j] += qi * ki[(j + 1) % nk];",
     [A.test_brute_force_torch_float64]),
]


def _param_args(fn):
    """Default arguments for the parametrised pins (first parameter set)."""
    marks = getattr(fn, "pytestmark", [])
    for m in marks:
        if m.name == "parametrize":
            names = [x.strip() for x in m.args[0].split(",")] if isinstance(m.args[0], str) \
                else list(m.args[0])
            vals = m.args[1][0]
            if len(names) == 1:
                vals = (vals,)
            return dict(zip(names, vals))
    return {}


def _detects(fn) -> bool:
    try:
        fn(oracle, **_param_args(fn))
    except (AssertionError, ValueError, FloatingPointError):
        return True
    return False


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, pins):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as td:
        cpath = os.path.join(td, "m.c")
        lpath = os.path.join(td, "libm.so")
        open(cpath, "w").write(mutated)
        subprocess.run(["gcc", *obuild.CFLAGS, cpath, "-o", lpath, "-lm"], check=True)
        with oracle.use_library(lpath):
            caught = [p.__name__ for p in pins if _detects(p)]
    assert caught, "no pin caught the planted mistake: " + name
