"""The pins catch plausible oracle mistakes (CPU only).

Each case plants one mistake in a copy of oracle/oracle.c: a dropped term, a
wrong sign or power, a transposed index, a biased/unbiased swap, a missing
eps.  It then compiles the copy into a temporary library and runs the pin
tests against it.  At least one pin must fail for every mutant, so the pins
constrain every part of the oracle they claim to cover.  The real oracle is
never modified.
"""
import importlib.util
import os
import subprocess

import pytest

import test_oracle_bn as pb
import test_oracle_rows as pr
from bwd_bn_stats_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = [
    ("bn_var_unbiased", "*var = ks_value(&q) / M;", "*var = ks_value(&q) / (M - 1.0);"),
    ("bn_y_drops_beta", "y[i] = gamma[c] * xhat + beta[c];", "y[i] = gamma[c] * xhat;"),
    ("bn_dx_drops_dbeta", "(M * dy[i] - dbeta - xhat * dgamma)", "(M * dy[i] - xhat * dgamma)"),
    ("bn_dx_sign", "(M * dy[i] - dbeta - xhat * dgamma)", "(M * dy[i] - dbeta + xhat * dgamma)"),
    # plane index without the channel stride (stays in bounds: n + c < N*C)
    ("bn_index_drops_C", "return (size_t)((n * C + c) * HW + j);", "return (size_t)((n + c) * HW + j);"),
    ("bn_running_var_biased", "+ momentum * var * (double)M / (double)(M - 1);", "+ momentum * var;"),
    ("bn_k1_power", "grads[2 * C + c] = -scale * inv_std * inv_std * ks_value(&sdyxc) / M;",
     "grads[2 * C + c] = -scale * inv_std * ks_value(&sdyxc) / M;"),
    ("bn_k2_sign", "grads[3 * C + c] = -scale * dbeta / M;", "grads[3 * C + c] = scale * dbeta / M;"),
    ("ln_dvar_power", "double dvar = -0.5 * rs * rs * rs * ks_value(&sgx);",
     "double dvar = -0.5 * rs * rs * ks_value(&sgx);"),
    ("ln_dmean_sign", "double dmean = -ks_value(&sg);", "double dmean = ks_value(&sg);"),
    ("ln_dx_drops_dmean", "+ 2.0 * dvar * (xr[j] - mu) / H + dmean / H;", "+ 2.0 * dvar * (xr[j] - mu) / H;"),
    ("ln_dweight_no_rstd", "ks_add(&sw[j], dy[i] * (x[i] - mean[r]) * rstd[r]);",
     "ks_add(&sw[j], dy[i] * (x[i] - mean[r]));"),
    ("ln_weight_ignored", "double g = dyr[j] * (w ? w[j] : 1.0);", "double g = dyr[j];"),
    ("rms_no_eps", "rms[r] = sqrt(ks_value(&s) / (double)cols + eps);", "rms[r] = sqrt(ks_value(&s) / (double)cols);"),
    ("rms_dx_factor", "dxr[j] = g * rinv + 2.0 * t * xr[j];", "dxr[j] = g * rinv + t * xr[j];"),
    ("rms_dweight_no_rinv", "ks_add(&sw[j], dyr[j] * xr[j] * rinv);", "ks_add(&sw[j], dyr[j] * xr[j]);"),
    ("ln_fwd_drops_bias", "yr[j] = (xr[j] - mu) * rs * (w ? w[j] : 1.0) + (b ? b[j] : 0.0);",
     "yr[j] = (xr[j] - mu) * rs * (w ? w[j] : 1.0);"),
    ("act_leaky_fwd_no_slope", "if (act == 2) return z > 0.0 ? z : slope * z;",
     "if (act == 2) return z > 0.0 ? z : z;"),
    ("act_relu_bwd_passes", "return act == 1 ? 0.0 : slope;", "return act == 1 ? 1.0 : slope;"),
    ("act_leaky_bwd_unit", "return act == 1 ? 0.0 : slope;", "return act == 1 ? 0.0 : 1.0;"),
    ("act_mask_inverted", "if (act == 0 || z > 0.0) return 1.0;", "if (act == 0 || z < 0.0) return 1.0;"),
    ("infer_drops_mean", "y[i] = act_value(act, slope, g * (x[i] - running_mean[c]) / sd + b);",
     "y[i] = act_value(act, slope, g * x[i] / sd + b);"),
    ("infer_no_eps", "const double sd = sqrt(running_var[c] + eps);", "const double sd = sqrt(running_var[c]);"),
    ("bda_drops_dresidual", "const double h = (dresidual ? dresidual[i] : 0.0) + dx[i];",
     "const double h = dx[i];"),
    ("bda_no_scale", "const double a = h * scale * m;", "const double a = h * m;"),
    ("bda_mask_ignored", "const double m = mask ? (mask[i] ? 1.0 : 0.0) : 1.0;", "const double m = 1.0;"),
    ("bda_dbias_sums_dh", "ks_add(&sa[j], a);", "ks_add(&sa[j], h);"),
    ("rms_fwd_inverted", "yr[j] = (w ? w[j] : 1.0) * (xr[j] / rms);", "yr[j] = (w ? w[j] : 1.0) * (xr[j] * rms);"),
]

PINS = [
    ("bn_torch_small", lambda m: pb.test_bn_matches_torch_fp64(m, (2, 3, 2, 3), 11, 0.0, 1.0)),
    ("bn_torch_ragged", lambda m: pb.test_bn_matches_torch_fp64(m, (3, 37, 41, 40), 1001, 5.0, 0.5)),
    ("bn_fd", pb.test_bn_finite_differences),
    ("bn_exact", pb.test_bn_exact_rational),
    ("bn_invariants", pb.test_bn_invariants_and_coefficient_form),
    ("bn_large_offset", pb.test_bn_large_offset_variance),
    ("bn_special", pb.test_bn_special_cases),
    ("ln_torch", lambda m: pr.test_ln_matches_torch_fp64(m, 3, 7, 1)),
    ("ln_fd", pr.test_ln_finite_differences),
    ("ln_invariants", pr.test_ln_invariants),
    ("ln_exact", pr.test_ln_exact_rational_given_stats),
    ("rms_torch", lambda m: pr.test_rms_matches_torch_fp64(m, 3, 7, 1, wl.F32)),
    ("rms_fd", pr.test_rms_finite_differences),
    ("rms_invariants", pr.test_rms_invariant_and_special_cases),
    ("rms_exact", pr.test_rms_exact_rational),
    ("ln_fwd_torch", lambda m: pr.test_ln_forward_matches_torch(m, 3, 7, 1)),
    ("rms_fwd_torch", lambda m: pr.test_rms_forward_matches_torch(m, 3, 7, 1)),
    ("fwd_exact", pr.test_forwards_exact_rational),
    ("bn_act_relu", lambda m: pb.test_bn_act_matches_torch(m, "relu", 0.0)),
    ("bn_act_leaky", lambda m: pb.test_bn_act_matches_torch(m, "leaky_relu", 0.2)),
    ("bn_act_fd", pb.test_bn_act_finite_differences),
    ("bn_infer_torch", lambda m: pb.test_bn_infer_matches_torch(m, "relu", 0.0)),
    ("bn_infer_batch", pb.test_bn_infer_with_batch_statistics_is_training_forward),
    ("bda_torch", lambda m: pr.test_bda_matches_torch(m, 6, 10, 0.3, 71)),
    ("bda_special", pr.test_bda_special_cases),
    ("bda_exact", pr.test_bda_exact_rational),
]


def _load_mutant(tmp_path, text):
    c = tmp_path / "mutant.c"
    c.write_text(text)
    so = tmp_path / "libmutant.so"
    import oracle
    subprocess.run(["gcc", *oracle.GCC_FLAGS, str(c), "-o", str(so), "-lm"], check=True,
                   capture_output=True)
    spec = importlib.util.spec_from_file_location("oracle_mutant",
                                                  os.path.join(ROOT, "oracle", "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = str(so)
    mod._lib = None
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site of {name} not found in oracle.c"
    mod = _load_mutant(tmp_path, src.replace(old, new))
    caught = []
    for pin_name, pin in PINS:
        try:
            pin(mod)
        except BaseException as e:  # assertion, pytest.raises failure, bad-argument error
            if isinstance(e, (KeyboardInterrupt, SystemExit)):
                raise
            caught.append(pin_name)
    print(f"{name}: caught by {caught}")
    assert caught, f"no pin catches the mutant {name}"
