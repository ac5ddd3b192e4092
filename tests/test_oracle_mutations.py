"""Plant plausible mistakes in a copy of the CPU oracle and check that the pins
catch every one of them.  Each mutant is a textual edit of c3d_oracle.c,
compiled into a temporary library that replaces the oracle for the duration
of one test.  CPU only; mutations are chosen to stay in bounds.
"""
import os
import subprocess

import pytest

import oracle as O
from tests import test_oracle_pins as P

SRC = O.SRC

# (name, original text, mutated text, occurrence index or None for all)
MUTATIONS = [
    ("conv_pad_sign", "o0 * P->s[0] - P->p[0] + (int64_t)k0 * P->d[0]",
     "o0 * P->s[0] + P->p[0] + (int64_t)k0 * P->d[0]", 0),
    ("conv_dilation_dropped", "o1 * P->s[1] - P->p[1] + (int64_t)k1 * P->d[1]",
     "o1 * P->s[1] - P->p[1] + (int64_t)k1", 0),
    ("conv_kernel_axes_swapped", "w[idx5(oc, icg, k0, k1, k2, cin_g, P->k[0], P->k[1], P->k[2])]",
     "w[idx5(oc, icg, k2, k1, k0, cin_g, P->k[2], P->k[1], P->k[0])]", 0),
    ("conv_bias_dropped", "double acc = bias ? (double)bias[oc] : 0.0;", "double acc = 0.0;", 0),
    ("conv_group_offset_dropped", "const int64_t ic = g * cin_g + icg;", "const int64_t ic = icg;", 0),
    ("conv_out_len_off_by_one", "return num / s + 1;", "return num / s + (num % s != 0);", 0),
    ("convT_kernel_flipped", "i0 * P->s[0] - P->p[0] + (int64_t)k0 * P->d[0]",
     "i0 * P->s[0] - P->p[0] + (int64_t)(P->k[0] - 1 - k0) * P->d[0]", 0),
    ("convT_group_offset_dropped", "const int64_t ic = g * cin_g + icg;", "const int64_t ic = icg;", 1),
    ("convT_out_len_no_plus_one", "+ (int64_t)d * (k - 1) + op + 1;", "+ (int64_t)d * (k - 1) + op;", 0),
    ("convT_gather_divisibility_dropped", "if (t0 < 0 || t0 % P->s[0] != 0 || t0 / P->s[0] >= xs[2]) continue;",
     "if (t0 < 0 || t0 / P->s[0] >= xs[2]) continue;", 0),
    ("bn_unbiased_variance", "v /= cnt;", "v /= (cnt - 1.0);", 0),
    ("bn_eps_dropped", "1.0 / sqrt(v + eps)", "1.0 / sqrt(v)", 0),
    ("bn_beta_dropped", "*e = ga * (*e - mu) * inv + be;", "*e = ga * (*e - mu) * inv;", 0),
    ("avgpool_wrong_divisor", "1.0 / ((double)w * w * w)", "1.0 / ((double)w * w)", 0),
    ("maxpool_takes_min", "if (v > m) m = v;\n                            }",
     "if (v < m || m == -INFINITY) m = v;\n                            }", 0),
    ("lse_shift_not_added_back", "out[n * plane + t] = m + log(s);", "out[n * plane + t] = log(s);", 0),
    ("lse_no_shift_inside_exp", "s += exp(in[(n * C + c) * plane + t] - m);",
     "s += exp(in[(n * C + c) * plane + t]);", 0),
    ("relu_inverted", "if (!(v[t] > 0.0)) v[t] = 0.0;", "if (v[t] > 0.0) v[t] = 0.0;", 0),
    ("running_var_biased", "batch_var_biased[c] * (double)count / (double)(count - 1);",
     "batch_var_biased[c];", 0),
    ("running_momentum_swapped", "running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * batch_mean[c];",
     "running_mean[c] = momentum * running_mean[c] + (1.0 - momentum) * batch_mean[c];", 0),
    ("eval_running_mean_dropped", "(double)gamma[c] * (y[e] - rm) / rs + (double)beta[c];",
     "(double)gamma[c] * y[e] / rs + (double)beta[c];", 0),
    ("eval_eps_dropped", "const double rm = running_mean[c], rs = sqrt((double)running_var[c] + eps);",
     "const double rm = running_mean[c], rs = sqrt((double)running_var[c]);", 0),
    ("fused_pool_rows_shifted", "oracle_conv3d_rows(x, xs, w, cout, P, bias, j0 * pool, j0 * pool + pool, y);",
     "oracle_conv3d_rows(x, xs, w, cout, P, bias, j0 * pool / 2, j0 * pool / 2 + pool, y);", 0),
]


def _pins():
    """The pins, as zero-argument callables (a few seeds of each parametrised pin)."""
    out = [
        P.test_size_formulas_page_examples, P.test_size_formulas_match_torch_shapes,
        P.test_conv3d_impulse_response, P.test_conv3d_constant_input, P.test_conv3d_kk1_equals_per_slice_conv2d,
        P.test_conv3d_at_matches_full, P.test_convT_taps_page_l2_p72_worked_example,
        P.test_convT_taps_page_l1_p77_worked_example, P.test_convT_valid_pair_counts_by_ones,
        P.test_convT_checkerboard_s2_p1_d2, P.test_convT_sublattice_equals_stride1_conv,
        P.test_convT_stride1_is_flipped_conv, P.test_avgpool_twice_equals_avgpool4,
        P.test_avgpool_matches_torch_and_drops_tail, P.test_maxpool_matches_torch,
        P.test_batchnorm_matches_torch_and_invariants, P.test_batchnorm_commutes_with_avgpool,
        P.test_logsumexp_page_examples, P.test_logsumexp_closed_forms_and_bounds, P.test_relu,
        P.test_convT_bn_avgpool_bias_cancels_and_gamma_zero, P.test_convT_pool_counts_page_l2_p72,
        P.test_conv_maxpool_lse_relu_bounds, P.test_workload_output_shapes,
    ]
    for s in range(4):
        out.append(lambda s=s: P.test_conv3d_matches_torch_float64(s))
        out.append(lambda s=s: P.test_convT_matches_torch_float64(s))
        out.append(lambda s=s: P.test_convT_gather_equals_scatter(s))
        out.append(lambda s=s: P.test_adjoint_identity(s))
    out.append(lambda: P.test_convT_bn_avgpool_matches_torch_module(dict(x_shape=(4, 3, 8, 8, 8), cout=16, pool=4)))
    out.append(lambda: P.test_convT_bn_eval_avgpool_matches_torch_module(P.EVAL_CASES[0]))
    out.append(P.test_convT_bn_eval_with_batch_statistics_equals_training_mode)
    out.append(lambda: P.test_bn_running_update_matches_torch_module(0.1))
    out.append(P.test_bn_running_update_closed_forms)
    out.append(lambda: P.test_conv_maxpool_lse_relu_matches_torch_module(dict(x_shape=(2, 4, 8, 8, 8), cout=8)))
    return out


def _mutate(text, old, new, occ):
    parts = text.split(old)
    assert len(parts) > 1, f"mutation anchor not found: {old!r}"
    if occ is None:
        return new.join(parts)
    assert occ < len(parts) - 1, f"occurrence {occ} of {old!r} not found"
    return old.join(parts[: occ + 1]) + new + old.join(parts[occ + 1:])


def test_unmutated_oracle_passes_all_pins():
    O._LIB = None
    for pin in _pins():
        pin()


@pytest.mark.parametrize("name,old,new,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new, occ):
    text = open(SRC).read()
    mutant = _mutate(text, old, new, occ)
    assert mutant != text
    src = tmp_path / "mutant.c"
    src.write_text(mutant)
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", lib_path, str(src), "-lm"],
                   check=True)
    saved = O._LIB
    O._LIB = O.load(lib_path)
    caught = []
    try:
        for pin in _pins():
            try:
                pin()
            except (AssertionError, ValueError) as e:  # a pin failed: the mistake is caught
                caught.append(getattr(pin, "__name__", "pin") + ": " + str(e)[:80])
                break
    finally:
        O._LIB = saved
    assert caught, f"planted mistake {name} was not caught by any pin"
