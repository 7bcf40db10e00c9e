"""Each plausible mistake planted in a copy of the oracle is caught by the pins.

The mutants are built from the oracle's C source by a one-line text change, in
a temporary directory, on the CPU; the pin suites then run against each mutant
in a subprocess and must fail: test_oracle_pins.py and
test_chunk_rederivation.py for the forward recurrence, test_oracle_backward.py
for the backward pass. A mutant that crashes also counts as caught.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

MUTANTS = {
    "decay_dropped": [("s[j] = s[j] * at[j];", "s[j] = s[j];")],
    "delta_sign_flipped": [("const double u = beta * (vi - p);", "const double u = beta * (vi + p);")],
    "beta_ignored": [("const double u = beta * (vi - p);", "const double u = (vi - p);")],
    "readout_uses_key": [("r += s[j] * qt[j];", "r += s[j] * kt[j];")],
    "readout_before_update": [
        ("      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] + u * kt[j];\n", ""),
        ("        J->o[(tok * H + h) * (int64_t)dv + i0 + i] = r;\n      }\n",
         "        J->o[(tok * H + h) * (int64_t)dv + i0 + i] = r;\n      }\n"
         "      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] + u * kt[j];\n")],
    "decay_after_correction": [
        ("      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] * at[j];\n", ""),
        ("      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] + u * kt[j];\n",
         "      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] + u * kt[j];\n"
         "      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] * at[j];\n")],
    "initial_state_ignored": [("J->init ? (double)", "0 ? (double)")],
    "sequence_offset_ignored": [("const int64_t t_begin = J->cu[n],", "const int64_t t_begin = 0 * J->cu[n],")],
    # the comparison's normaliser taken across slices instead of per slice
    "checker_o_running_max": [("""    if (o_cand) {
      for (int32_t n = 0; n < num_seqs; ++n)
        for (int32_t h = 0; h < H; ++h) {
          double num = 0.0, den = 0.0;""", """    if (o_cand) {
      double den = 0.0;
      for (int32_t n = 0; n < num_seqs; ++n)
        for (int32_t h = 0; h < H; ++h) {
          double num = 0.0;""")],
    "checker_state_global_max": [
        ("""        double rel = slice_rel(final_cand + s * state_elems, f_buf + s * state_elems, state_elems, &nonfinite);""",
         """        double rel = s ? 0.0 : slice_rel(final_cand, f_buf, (int64_t)num_seqs * H * state_elems, &nonfinite);"""),
        ("""        double rel = slice_rel(snap_cand + s * state_elems, s_buf + s * state_elems, state_elems, &nonfinite);""",
         """        double rel = s ? 0.0 : slice_rel(snap_cand, s_buf, n_snap * H * state_elems, &nonfinite);""")],
    "snapshot_one_token_late": [("if (J->interval > 0 && J->snap && (t + 1) % J->interval == 0) {",
                                 "if (J->interval > 0 && J->snap && t % J->interval == 0 && t > 0) {"),
                                ("const int64_t slot = J->snap_base[n] + (t + 1) / J->interval - 1;",
                                 "const int64_t slot = J->snap_base[n] + t / J->interval - 1;")],
}


BACKWARD_MUTANTS = {
    "bwd_readout_term_dropped": [("dS[(int64_t)i * dk + j] += dot[i] * qt[j];",
                                  "dS[(int64_t)i * dk + j] += 0.0 * dot[i] * qt[j];")],
    "bwd_dq_from_previous_state": [("r += St[(int64_t)i * dk + j] * dot[i];", "r += Sp[(int64_t)i * dk + j] * dot[i];")],
    "bwd_dk_read_term_sign": [("dkt[j] -= r;", "dkt[j] += r;")],
    "bwd_dalpha_from_new_state": [("dat[j] += g * Sp[(int64_t)i * dk + j];", "dat[j] += g * St[(int64_t)i * dk + j];")],
    "bwd_decay_not_propagated": [("dS[(int64_t)i * dk + j] = g * at[j];", "dS[(int64_t)i * dk + j] = g;")],
    "bwd_dbeta_scaled_by_beta": [("db += u[i] * r;", "db += beta * u[i] * r;")],
    "bwd_dv_unscaled": [("J->dv_out[v_off + i] = beta * w[i];", "J->dv_out[v_off + i] = w[i];")],
    "bwd_correction_not_removed": [("const double g = dS[(int64_t)i * dk + j] - beta * w[i] * kt[j];",
                                    "const double g = dS[(int64_t)i * dk + j];")],
    "bwd_wrong_checkpoint": [("memcpy(buf, ckpt + m * se,", "memcpy(buf, ckpt + (m > 0 ? m - 1 : 0) * se,")],
    "bwd_final_gradient_ignored": [("dS[e] = J->d_final ? ", "dS[e] = 0 ? ")],
}

FORWARD_SUITES = ("test_oracle_pins.py", "test_chunk_rederivation.py")
BACKWARD_SUITES = ("test_oracle_backward.py",)


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(BACKWARD_MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = open(SRC).read()
    edits, suites = (MUTANTS[name], FORWARD_SUITES) if name in MUTANTS else (BACKWARD_MUTANTS[name], BACKWARD_SUITES)
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new, 1)
    inc = os.path.join(ROOT, "include")
    csrc = tmp_path / "kda_oracle_mutant.c"
    csrc.write_text(src.replace('#include "../include/kda_oracle.h"', '#include "kda_oracle.h"'))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-I", inc, "-o", str(lib),
                    str(csrc), "-lpthread", "-lm"], check=True)
    env = dict(os.environ, KDA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in suites]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
