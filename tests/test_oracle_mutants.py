"""Each plausible mistake planted in a copy of the oracle is caught by the pins.

The mutants are built from the oracle's C source by a one-line text change, in
a temporary directory, on the CPU; the pin suites (test_oracle_pins.py and
test_chunk_rederivation.py) then run against each mutant in a subprocess and
must fail. A mutant that crashes also counts as caught.
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
    "snapshot_one_token_late": [("if (J->interval > 0 && J->snap && (t + 1) % J->interval == 0) {",
                                 "if (J->interval > 0 && J->snap && t % J->interval == 0 && t > 0) {"),
                                ("const int64_t slot = J->snap_base[n] + (t + 1) / J->interval - 1;",
                                 "const int64_t slot = J->snap_base[n] + t / J->interval - 1;")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
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
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_chunk_rederivation.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
