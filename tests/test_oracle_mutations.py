"""The oracle's pins must catch plausible mistakes in the oracle (not GPU).

Each mutant below plants one mistake -- a dropped term, a wrong sign, bias or
index, a swapped operand, a missing reset -- in a private copy of oracle/
(oracle.c or oracle/__init__.py), rebuilds that copy and runs the pin tests
(tests/test_oracle_*.py) against it in a subprocess.  A mutant passes this
test only if at least one pin fails on it.  The unmutated copy must pass every
pin, so a broken copy cannot make the mutants look caught.

Nothing here touches the HIP library: the copies hold oracle/, synth/ (the
seeded input generators the pins use) and the pin tests only.
"""
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_convert.py", "tests/test_oracle_layout_memory.py",
        "tests/test_oracle_reduce_check.py", "tests/test_oracle_adamw.py"]
C, PY = "oracle/oracle.c", "oracle/__init__.py"

# name -> (file, text in the oracle, replacement)
MUTANTS = {
    # 16-bit formats
    "decode_bias_off_by_one": (C, "int bias = (1 << (f.exp_bits - 1)) - 1;\n    int emax = (1 << f.exp_bits) - 1;\n    int sign",
                               "int bias = (1 << (f.exp_bits - 1));\n    int emax = (1 << f.exp_bits) - 1;\n    int sign"),
    "decode_subnormal_exponent": (C, "ldexp((double)frac, 1 - bias - f.frac_bits)", "ldexp((double)frac, -bias - f.frac_bits)"),
    "decode_nan_as_inf": (C, "v = frac ? NAN : INFINITY;", "v = INFINITY;"),
    "encode_ties_away_from_zero": (C, "(rem == 0.5 && fmod(r, 2.0) == 1.0)", "(rem == 0.5)"),
    "encode_truncates": (C, "r += 1.0;", "r += 0.0;"),
    "encode_no_binade_carry": (C, "if (r >= ldexp(1.0, fb + 1)) {", "if (r > ldexp(1.0, fb + 1)) {"),
    "encode_overflow_threshold": (C, "if (field >= emax) return", "if (field > emax) return"),
    "encode_subnormal_quantum": (C, "if (E < emin) E = emin;", ""),
    # layout and buckets
    "layout_pads_to_world_only": (C, "int64_t unit = (int64_t)world * (int64_t)align;", "int64_t unit = (int64_t)world;"),
    "layout_always_pads": (C, "int64_t groups = total / unit + (total % unit != 0);", "int64_t groups = total / unit + 1;"),
    "layout_offsets_at_ends": (C, "tensor_offset[k] = total;\n", "tensor_offset[k] = total + numel[k];\n"),
    "buckets_close_at_cap": (C, "fill + numel[k] > cap", "fill + numel[k] >= cap"),
    "buckets_fill_not_reset": (C, "            fill = 0;\n        }\n        fill += numel[k];", "        }\n        fill += numel[k];"),
    # copy-in / write-back
    "gather_no_zero_fill": (C, "for (int64_t i = 0; i < flat_count; ++i) flat[i] = 0;", ""),
    "scatter_off_by_one": (C, "tensors[k][j] = flat[offset[k] + j];", "tensors[k][j] = flat[offset[k] + j + (j + 1 < numel[k])];"),
    # reduce and check
    "reduce_drops_rank0": (C, "for (int32_t r = 0; r < n_ranks; ++r) acc = acc + (float)val",
                           "for (int32_t r = 1; r < n_ranks; ++r) acc = acc + (float)val"),
    "reduce_drops_last_rank": (C, "r < n_ranks; ++r) acc = acc + (float)val", "r < n_ranks - 1; ++r) acc = acc + (float)val"),
    "reduce_accumulates_in_fp64": (C, "float acc = 0.0f;\n        for (int32_t r = 0; r < n_ranks; ++r) acc = acc + (float)val[src[r][i]];",
                                   "double acc = 0.0;\n        for (int32_t r = 0; r < n_ranks; ++r) acc = acc + val[src[r][i]];"),
    "reduce_starts_from_rank0": (C, "float acc = 0.0f;\n        for (int32_t r = 0; r < n_ranks;",
                                 "float acc = (float)val[src[0][i]];\n        for (int32_t r = 1; r < n_ranks;"),
    "check_misses_nan": (C, "if (!isfinite(x)) flag = 1;", "if (isinf(x)) flag = 1;"),
    "check_norm_not_unscaled": (C, "double g = (double)((float)x * inv_scale);", "double g = x;"),
    "check_unscale_in_fp64": (C, "double g = (double)((float)x * inv_scale);", "double g = x * (double)inv_scale;"),
    "check_l1_not_l2": (C, "s = s + g * g;", "s = s + fabs(g);"),
    "check_not_accumulated": (C, "uint32_t flag = *overflow;\n    double s = *sumsq;", "uint32_t flag = 0;\n    double s = 0.0;"),
    "clip_without_eps": (C, "(sqrt(sumsq) + 1e-6)", "(sqrt(sumsq))"),
    "clip_scales_up": (C, "return c < 1.0 ? (float)c : 1.0f;", "return (float)c;"),
    "clip_uses_sumsq": (C, "(double)max_norm / (sqrt(sumsq) + 1e-6)", "(double)max_norm / (sumsq + 1e-6)"),
    # AdamW
    "adam_bc2_uses_beta1": (C, "c->bc2 = (float)(1.0 - pow((double)hp->beta2, t));", "c->bc2 = (float)(1.0 - pow((double)hp->beta1, t));"),
    "adam_bias_correction_t_minus_1": (C, "c->bc1 = (float)(1.0 - pow((double)hp->beta1, t));", "c->bc1 = (float)(1.0 - pow((double)hp->beta1, t + 1.0));"),
    "adam_no_weight_decay": (C, "float p = master[i] * c.decay;", "float p = master[i];"),
    "adam_l2_decay_in_gradient": (C, "g = g * coef;                               /* clip                 */",
                                  "g = g * coef + hp->weight_decay * master[i];"),
    "adam_eps_inside_sqrt": (C, "(mh / (sqrtf(vh) + c.eps))", "(mh / sqrtf(vh + c.eps))"),
    "adam_m_coefficients_swapped": (C, "c.b1 * exp_avg[i] + c.omb1 * g", "c.omb1 * exp_avg[i] + c.b1 * g"),
    "adam_v_not_squared": (C, "c.omb2 * (g * g)", "c.omb2 * g"),
    "adam_no_bias_correction": (C, "float mh = m / c.bc1;", "float mh = m;"),
    "adam_no_clip": (C, "g = g * coef;                               /* clip                 */", ""),
    "adam_no_unscale": (C, "float g = (float)val[red[i]] * inv_scale;", "float g = (float)val[red[i]];"),
    "adam_ignores_overflow": (C, "    if (overflow) return;\n    const double* val", "    const double* val"),
    "adam_sign_flipped": (C, "p = p - c.lr * (mh / (sqrtf(vh) + c.eps));", "p = p + c.lr * (mh / (sqrtf(vh) + c.eps));"),
    "adam_param16_wrong_format": (C, "param16[i] = encode16((double)p, f);", "param16[i] = encode16((double)p, fmt_of(dtype == O_BF16 ? O_FP16 : O_BF16));"),
    "init_master_drops_sign": (C, "master[i] = (float)val[param16[i]];", "master[i] = (float)val[param16[i] & 0x7FFF];"),
    # loss scaler
    "scaler_no_floor": (C, "s->scale = fmax(s->scale / 2.0, s->min_scale);", "s->scale = s->scale / 2.0;"),
    "scaler_clean_not_reset": (C, "s->clean = 0;\n        s->skipped += 1;", "s->skipped += 1;"),
    "scaler_window_off_by_one": (C, "if (s->clean == s->window) {", "if (s->clean == s->window - 1) {"),
    # Python side: memory closed forms and the step driver
    "memory_stage2_grads_unsharded": (PY, "grads = 2 * (part if stage >= 2 else phi)", "grads = 2 * (part if stage >= 3 else phi)"),
    "memory_optimizer_8_bytes": (PY, "optim = 12 * (part if stage >= 1 else phi)", "optim = 8 * (part if stage >= 1 else phi)"),
    "step_counts_skipped_steps": (PY, "    applied = not overflow\n    if applied:\n        t = t + 1\n",
                                  "    applied = not overflow\n    t = t + 1\n    if applied:\n"),
    "step_norm_per_owner": (PY, "overflow, sumsq = check(red, dtype, inv, overflow, sumsq)", "overflow, sumsq = check(red, dtype, inv)"),
    "step_divisor_ignored": (PY, "inv = float(np.float32(1.0 / (scaler.scale * divisor)))",
                             "inv = float(np.float32(1.0 / scaler.scale))"),
    "step_scaler_not_updated": (PY, "    scaler.update(overflow)\n    return res, t", "    return res, t"),
}


def _copy_tree(dst):
    ign = shutil.ignore_patterns("__pycache__", "*.pyc", ".pytest_cache")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"), ignore=ign)
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(dst, "synth"), ignore=ign)
    os.makedirs(os.path.join(dst, "tests"))
    for f in PINS + ["tests/conftest.py", "tests/_common.py"]:
        shutil.copy(os.path.join(ROOT, f), os.path.join(dst, f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))


def _run_pins(dst, mutation):
    """-> (returncode, first failed pin or '', log tail)."""
    _copy_tree(dst)
    if mutation is not None:
        rel, old, new = mutation
        path = os.path.join(dst, rel)
        text = open(path).read()
        assert text.count(old) == 1, f"mutation target not unique in {rel}: {old!r}"
        open(path, "w").write(text.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    b = subprocess.run([sys.executable, "-c", "import oracle; oracle.build()"], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=120)
    if b.returncode != 0:
        return b.returncode, "build", b.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-rf", "-p", "no:cacheprovider",
                        *PINS], cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    m = re.search(r"^FAILED (\S+)", r.stdout, re.M)
    return r.returncode, m.group(1) if m else "", r.stdout[-3000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    base = tmp_path_factory.mktemp("oracle_mutants")
    jobs = {"unmutated": None, **MUTANTS}
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        futs = {k: ex.submit(_run_pins, str(base / k), v) for k, v in jobs.items()}
        return {k: f.result() for k, f in futs.items()}


def test_unmutated_copy_passes_every_pin(outcomes):
    rc, failed, log = outcomes["unmutated"]
    assert rc == 0, log


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(outcomes, name):
    rc, failed, log = outcomes[name]
    assert failed != "build", log
    assert rc == 1 and failed, f"mutant {name} passed every pin:\n{log}"
