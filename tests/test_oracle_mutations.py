"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped term, a
swapped coefficient, a wrong sign or comparison, a missing rounding rule), builds
the copy on the CPU and runs the oracle's pin tests against it in a fresh process
(the build is selected with BITOPT_ORACLE_LIB).  Every mutant must fail at least
one pin; the unmutated source must pass them all.  Nothing here touches a GPU.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle.build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_optim.py", "tests/test_oracle_codec.py",
             "tests/test_oracle_codebook.py"]

# (name, text in the oracle source, replacement).  The text must occur exactly once.
MUTANTS = [
    # codebook construction (dynamic data type)
    ("codebook_no_half_bin", "((double)frac + 0.5) / bins", "(double)frac / bins"),
    ("codebook_decade_off_by_one", "pow(10.0, -(double)zeros)", "pow(10.0, -(double)zeros - 1.0)"),
    # codec
    ("nearest_tie_larger_index", "if (d < bd) { bd = d; best = j; }",
     "if (d <= bd) { bd = d; best = j; }"),
    ("absmax_signed_max", "float a = fabsf(s[i]);", "float a = s[i];"),
    ("no_subnormal_prescale", "(A < 0x1p-126f) ? 0x1p24f : 1.0f", "1.0f"),
    ("half_ties_away", "(rem == halfway && (q & 1))", "(rem == halfway)"),
    ("bf16_truncate", "u += 0x7fffu + lsb;", "u += 0u * lsb;"),
    # step scalars
    ("no_bias_correction_m", "s->ic1 = (float)(1.0 / (1.0 - pow(b1, (double)t)));", "s->ic1 = 1.0f;"),
    ("bias_correction_v_no_sqrt", "(1.0 / sqrt(1.0 - pow(b2, (double)t)))",
     "(1.0 / (1.0 - pow(b2, (double)t)))"),
    ("decay_without_lr", "(1.0 - (double)h->lr * (double)h->weight_decay)",
     "(1.0 - (double)h->weight_decay)"),
    ("beta3_schedule_swapped", "exp(lb1 * lb3 / ((1.0 - f) * lb3 + f * lb1))",
     "exp(lb1 * lb3 / ((1.0 - f) * lb1 + f * lb3))"),
    ("alpha_schedule_ignored", "return alpha * (f < 1.0 ? f : 1.0);", "return alpha;"),
    # skip_zeros
    ("skip_zeros_ignored", "skip[i] = h->skip_zeros && (gv[i] == 0.0f);", "skip[i] = 0;"),
    # Adam
    ("adam_m_uses_omb2", "t2 = sc->omb1 * gi; m = t1 + t2;\n            float gg",
     "t2 = sc->omb2 * gi; m = t1 + t2;\n            float gg"),
    ("adam_v_not_squared", "float gg = gi * gi;\n            t1 = sc->b2 * v;",
     "float gg = gi;\n            t1 = sc->b2 * v;"),
    ("adam_eps_inside_sqrt", "float d = sqrtf(v) * sc->rs2;\n            d = d + sc->eps;\n",
     "float d = sqrtf(v + sc->eps) * sc->rs2;\n"),
    # AdEMAMix
    ("ademamix_slow_ema_dropped", "t2 = sc->alpha_t * m2;", "t2 = 0.0f * m2;"),
    ("ademamix_slow_ema_uses_beta1", "t1 = sc->b3t * m2; t2 = sc->omb3 * gi;",
     "t1 = sc->b1 * m2; t2 = sc->omb1 * gi;"),
    # Momentum
    ("momentum_decay_sign", "float g2 = gi + t1;          /* decay",
     "float g2 = gi - t1;          /* decay"),
    ("momentum_dampened", "buf = t1 + g2;", "buf = t1 + sc->omb1 * g2;"),
    # RMSprop / Adagrad
    ("rmsprop_square_without_decay", "float gg = g2 * g2;\n            t1 = sc->b1 * v;",
     "float gg = gi * gi;\n            t1 = sc->b1 * v;"),
    ("adagrad_sum_not_squared", "v = v + gg;", "v = v + g2;"),
    # Lion
    ("lion_sign_of_old_state", "dv[i] = sc->lr * sign_of(c);", "dv[i] = sc->lr * sign_of(m);"),
    ("lion_state_uses_beta1", "t1 = sc->b2 * m; t2 = sc->omb2 * gi; m = t1 + t2;",
     "t1 = sc->b1 * m; t2 = sc->omb1 * gi; m = t1 + t2;"),
    # max_unorm and write-back
    ("max_unorm_comparison_flipped", "if (U > lim)", "if (U < lim)"),
    ("max_unorm_not_relative", "double lim = (double)h->max_unorm * P;",
     "double lim = (double)h->max_unorm;"),
    ("adamw_decay_dropped", "float pd = pv[i] * sc->decay;", "float pd = pv[i];"),
    ("coupled_update_sign", "pn = pv[i] - d;   /* coupled decay */", "pn = pv[i] + d;"),
]


def _source():
    with open(obuild.SRC) as f:
        return f.read()


def _run_pins(lib_path):
    env = dict(os.environ, BITOPT_ORACLE_LIB=lib_path, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", *PIN_FILES, "-x", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _build_and_run(name, text, tmpdir):
    src = os.path.join(tmpdir, f"{name}.c")
    with open(src, "w") as f:
        f.write(text)
    lib = obuild.build(force=True, extra_flags=["-w"], out=os.path.join(tmpdir, f"{name}.so"),
                       src=src)
    return _run_pins(lib)


def test_mutations_are_unique_text():
    src = _source()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"{name}: mutation site found {src.count(old)} times"
        assert old != new


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = _source()
    jobs = [("unmutated", src)] + [(name, src.replace(old, new, 1)) for name, old, new in MUTANTS]
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_build_and_run, name, text, str(tmp_path)) for name, text in jobs}
        results = {name: f.result() for name, f in futs.items()}
    rc, out = results.pop("unmutated")
    assert rc == 0, f"the unmutated oracle fails its pins:\n{out}"
    survivors = [name for name, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"mutants that pass every pin: {survivors}"
