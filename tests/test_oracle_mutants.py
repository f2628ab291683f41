"""The oracle's pins catch plausible slips.

Each case plants one mistake in a copy of oracle/ (a dropped term, a wrong sign
or index, swapped operands or axes, the pages' own garbled readings) and runs
the pin tests of that file against the copy in a child pytest: at least one pin
must fail.  An unmodified copy must pass, so a failure is the planted
mistake's doing.  CPU only; the mistakes live in temporary copies and never
touch oracle/ itself.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C, OPT, MLP = "hashgrid_oracle.c", "optim_oracle.py", "mlp_oracle.py"
PINS = {C: "tests/test_oracle_pins.py", OPT: "tests/test_oracle_optim.py", MLP: "tests/test_oracle_mlp.py"}

# name -> (file, text in the oracle, planted replacement)
MUTANTS = {
    # hash
    "hash_add_not_xor": (C, "h ^= c[d] * kPrimes[d];", "h += c[d] * kPrimes[d];"),
    "hash_y_z_primes_swapped": (C, "1LL, 2654435761LL, 805459861LL,", "1LL, 805459861LL, 2654435761LL,"),
    "hash_negative_remainder_mirrored": (C, "return r < 0 ? r + T : r;", "return r < 0 ? -r : r;"),
    # resolutions
    "resolution_divides_by_L": (C, "/ (double)(n_levels - 1));", "/ (double)(n_levels));"),
    "resolution_rounds_not_floors": (C, "res[l] = (int32_t)floor((double)n_min * pow(b, (double)l));",
                                     "res[l] = (int32_t)lround((double)n_min * pow(b, (double)l));"),
    # voxel location and weights
    "scale_by_N_minus_1": (C, "float scaled = xp[d] * (float)N;", "float scaled = xp[d] * (float)(N - 1);"),
    "fraction_of_unrounded_product": (C, "frac[d] = (double)scaled - (double)fl;",
                                      "frac[d] = (double)xp[d] * (double)N - (double)fl;"),
    "weights_x_z_swapped": (C, "        w *= up ? frac[d] : 1.0 - frac[d];",
                            "        w *= up ? frac[dims - 1 - d] : 1.0 - frac[dims - 1 - d];"),
    "weights_flipped": (C, "        w *= up ? frac[d] : 1.0 - frac[d];", "        w *= up ? 1.0 - frac[d] : frac[d];"),
    "corner_offset_from_wrong_bit": (C, "int up = (k >> (dims - 1 - d)) & 1;\n        c[d]",
                                     "int up = (k >> d) & 1;\n        c[d]"),
    "resolution_in_fp32": (C, "double b = exp((log((double)n_max) - log((double)n_min)) / (double)(n_levels - 1));\n"
                                 "    for (int l = 0; l < n_levels; ++l) res[l] = (int32_t)floor((double)n_min * pow(b, (double)l));",
                           "float b = expf((logf((float)n_max) - logf((float)n_min)) / (float)(n_levels - 1));\n"
                           "    for (int l = 0; l < n_levels; ++l) res[l] = (int32_t)floorf((float)n_min * powf(b, (float)l));"),
    "negative_voxels_clamped": (C, "v[d] = (int64_t)fl;", "v[d] = fl < 0 ? 0 : (int64_t)fl;"),
    "weights_y_flipped": (C, "        w *= up ? frac[d] : 1.0 - frac[d];",
                          "        w *= (up ^ (d == 1)) ? frac[d] : 1.0 - frac[d];"),
    # forward
    "forward_drops_last_corner": (C, "for (int k = 0; k < K; ++k) {\n                double wk = corner(v, frac, D, k, c);\n"
                                     "                int64_t e = spatial_hash(c, D, T);\n                for (int j = 0; j < F; ++j) acc[j]",
                                  "for (int k = 0; k < K - 1; ++k) {\n                double wk = corner(v, frac, D, k, c);\n"
                                  "                int64_t e = spatial_hash(c, D, T);\n                for (int j = 0; j < F; ++j) acc[j]"),
    "forward_feature_index_fixed": (C, "acc[j] += wk * table_value(g, table, l, e, j);",
                                    "acc[j] += wk * table_value(g, table, l, e, 0);"),
    "half_subnormals_flushed": (C, "if (e == 0) v = ldexp((double)m, -24);", "if (e == 0) v = 0.0;"),
    "half_exponent_bias_16": (C, "else v = ldexp(1.0 + (double)m / 1024.0, e - 15);",
                              "else v = ldexp(1.0 + (double)m / 1024.0, e - 16);"),
    # backward
    "backward_overwrites": (C, "grad[((int64_t)l * T + e) * F + j] +=", "grad[((int64_t)l * T + e) * F + j] ="),
    "backward_reads_feature_0": (C, "wk * (double)dout[p * dout_stride + (int64_t)l * F + j];",
                                 "wk * (double)dout[p * dout_stride + (int64_t)l * F];"),
    "backward_ignores_row_stride": (C, "wk * (double)dout[p * dout_stride + (int64_t)l * F + j];",
                                    "wk * (double)dout[p * (int64_t)L * F + (int64_t)l * F + j];"),
    "backward_drops_last_corner": (C, "for (int k = 0; k < K; ++k) {\n                double wk = corner(v, frac, D, k, c);\n"
                                      "                int64_t e = spatial_hash(c, D, T);\n                for (int j = 0; j < F; ++j)\n"
                                      "                    grad",
                                   "for (int k = 0; k < K - 1; ++k) {\n                double wk = corner(v, frac, D, k, c);\n"
                                   "                int64_t e = spatial_hash(c, D, T);\n                for (int j = 0; j < F; ++j)\n"
                                   "                    grad"),
    # dL/dx
    "input_grad_weight_of_wrong_axis": (C, "else dw *= up ? frac[q] : 1.0 - frac[q];",
                                        "else dw *= up ? frac[d] : 1.0 - frac[d];"),
    "input_grad_sign": (C, "if (q == d) dw *= up ? 1.0 : -1.0;", "if (q == d) dw *= up ? -1.0 : 1.0;"),
    "input_grad_missing_chain_factor": (C, "acc[d] += (double)res[l] * dw * s;", "acc[d] += dw * s;"),
    "input_grad_other_weights_flipped": (C, "else dw *= up ? frac[q] : 1.0 - frac[q];",
                                         "else dw *= up ? 1.0 - frac[q] : frac[q];"),
    # Adam
    "adam_bias_correction_power": (OPT, "m_hat = m1 / (1.0 - beta1 ** t)", "m_hat = m1 / (1.0 - beta1 ** (t + 1))"),
    "adam_second_moment_not_squared": (OPT, "(1.0 - beta2) * (g * g)", "(1.0 - beta2) * g"),
    "adam_eps_inside_root": (OPT, "np.sqrt(v_hat) + eps", "np.sqrt(v_hat + eps)"),
    "adam_first_moment_uses_beta2": (OPT, "m_hat = m1 / (1.0 - beta1 ** t)", "m_hat = m1 / (1.0 - beta2 ** t)"),
    # MLP head
    "mlp_second_relu_dropped": (MLP, "h2 = _r(np.maximum(z2, 0.0), round_fp16)", "h2 = _r(z2, round_fp16)"),
    "mlp_output_bias_dropped": (MLP, "y = h2 @ W3.T + b3", "y = h2 @ W3.T"),
    "mlp_dW2_wrong_activation": (MLP, "dW2=(dz2.T @ cache[\"h1\"])", "dW2=(dz2.T @ cache[\"h2\"])"),
    "mlp_db1_from_layer_2": (MLP, "db1=dz1.sum(0)", "db1=dz2.sum(0)"),
    "mlp_relu_mask_dropped": (MLP, "dz2 = _r(_sum(g3, W3, None, acc32) * (cache[\"z2\"] > 0), on)",
                              "dz2 = _r(_sum(g3, W3, None, acc32), on)"),
    # the backward's binary16 rounding points and its power-of-two scale
    "mlp_dz1_not_rounded": (MLP, "dz1 = _r(_sum(dz2, W2, None, acc32) * (cache[\"z1\"] > 0), on)",
                            "dz1 = _sum(dz2, W2, None, acc32) * (cache[\"z1\"] > 0)"),
    "mlp_first_layer_sum_in_float64": (MLP, "z1 = _sum(e16, W1.T, b1, acc32)", "z1 = _sum(e16, W1.T, b1, False)"),
    "mlp_dy_rounded_before_scaling": (MLP, "g3 = _r(np.asarray(dy, dtype=np.float64) * s, on)",
                                      "g3 = _r(np.asarray(dy, dtype=np.float64), on) * s"),
    "mlp_de_rounded_to_half": (MLP, "de = (dz1 @ W1) / s", "de = _r(dz1 @ W1, on) / s"),
    "mlp_dW1_not_unscaled": (MLP, "dW1=(dz1.T @ cache[\"e\"]) / s", "dW1=dz1.T @ cache[\"e\"]"),
}


def _planted_copy(base, name):
    """tmp/<name>/oracle: a copy of oracle/ with MUTANTS[name] planted (name None: unmodified)."""
    top = os.path.join(base, name or "unmodified")
    dst = os.path.join(top, "oracle")
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__"))
    if name:
        f, old, new = MUTANTS[name]
        path = os.path.join(dst, f)
        with open(path) as fh:
            text = fh.read()
        assert text.count(old) == 1, f"{name}: the text to replace is not unique in {f}"
        with open(path, "w") as fh:
            fh.write(text.replace(old, new))
    return top


def _run_pins(top, pin_file):
    env = dict(os.environ, HG_ORACLE_DIR=top, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", pin_file, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_copy_passes_every_pin(tmp_path):
    top = _planted_copy(str(tmp_path), None)
    for pin_file in sorted(set(PINS.values())):
        rc, out = _run_pins(top, pin_file)
        assert rc == 0, f"{pin_file} fails on an unmodified copy of the oracle:\n{out}"


def test_every_planted_mistake_fails_a_pin(tmp_path):
    def one(name):
        top = _planted_copy(str(tmp_path), name)
        rc, out = _run_pins(top, PINS[MUTANTS[name][0]])
        return name, rc, out
    workers = max(1, min(8, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(one, sorted(MUTANTS)))
    # rc 1: tests ran and at least one failed; anything else (0 passed, 2+ errors) is not a catch
    missed = [(name, rc, out) for name, rc, out in results if rc != 1]
    assert not missed, "planted mistakes that no pin caught:\n" + "\n".join(
        f"--- {name} (pytest exit {rc})\n{out}" for name, rc, out in missed)
