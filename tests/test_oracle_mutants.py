"""Plant mistakes in a copy of the oracle and check that the pins catch each.

Every mutant is one plausible error in the token-by-token recurrence (a
dropped term, a wrong sign, a wrong side or index, a transposed operand).  A
mutant that passes every pin would mean the pins cannot tell that mistake from
the method, so the test fails.  Everything here runs on the CPU.
"""
import os
import re
import shutil
import tempfile

import pytest

import oracle
import oracle_pins
from oracle import build as obuild

# (name, original text in recurrent_chain, replacement)
MUTANTS = [
    ("drop_decay", "S[c * dv + j] *= at[c];", "S[c * dv + j] *= 1.0;"),
    ("decay_on_value_side", "S[c * dv + j] *= at[c];", "S[c * dv + j] *= at[j % dk];"),
    ("read_before_decay", "acc += S[c * dv + j] * e[c];", "acc += S[c * dv + j] * e[c] / at[c];"),
    ("read_with_key_not_erase", "acc += S[c * dv + j] * e[c];", "acc += S[c * dv + j] * kt[c];"),
    ("output_from_old_state", "acc += S[c * dv + j] * qt[c];",
     "acc += (S[c * dv + j] - kt[c] * (z[j] - r[j])) * qt[c];"),
    ("output_transposed", "acc += S[c * dv + j] * qt[c];",
     "acc += S[(j % dk) * dv + (c % dv)] * qt[c];"),
    ("drop_erase_gate", "e[c] = bt[c] * kt[c];", "e[c] = kt[c];"),
    ("drop_write_gate", "z[j] = wt[j] * vt[j];", "z[j] = vt[j];"),
    ("erase_gate_on_query", "e[c] = bt[c] * kt[c];", "e[c] = bt[c] * qt[c];"),
    ("write_gate_on_key_side", "z[j] = wt[j] * vt[j];", "z[j] = bt[j % dk] * vt[j];"),
    ("delta_sign", "S[c * dv + j] += kt[c] * (z[j] - r[j]);", "S[c * dv + j] += kt[c] * (z[j] + r[j]);"),
    ("write_address_is_erase", "S[c * dv + j] += kt[c] * (z[j] - r[j]);",
     "S[c * dv + j] += e[c] * (z[j] - r[j]);"),
    ("ignore_initial_state", "if (S0) memcpy(S, S0 + soff, sizeof(double) * dk * dv);", ""),
]


# (name, original text in backward_chain, replacement): plausible mistakes in
# the adjoint of one token
BWD_MUTANTS = [
    ("dq_from_old_state", "acc += S[c * dv + j] * gt[j];", "acc += Sprev[c * dv + j] * gt[j];"),
    ("no_output_seed_into_state", "dS[c * dv + j] += qt[c] * gt[j];", "(void)0;"),
    ("du_with_erase_not_key", "acc += dS[c * dv + j] * kt[c];", "acc += dS[c * dv + j] * e[c];"),
    ("dk_from_z_not_u", "acc += dS[c * dv + j] * u[j];", "acc += dS[c * dv + j] * z[j];"),
    ("de_sign", "de[c] = -acc;", "de[c] = acc;"),
    ("de_through_old_state", "acc += Sbar[c * dv + j] * du[j];", "acc += Sprev[c * dv + j] * du[j];"),
    ("no_erase_term_in_state_grad", "dS[c * dv + j] -= e[c] * du[j];", "(void)0;"),
    ("dalpha_with_new_state", "acc += dS[c * dv + j] * Sprev[c * dv + j];",
     "acc += dS[c * dv + j] * S[c * dv + j];"),
    ("no_decay_on_state_grad", "dS[c * dv + j] *= at[c];", "(void)0;"),
    ("db_with_query", "dbt[c] = de[c] * kt[c];", "dbt[c] = de[c] * qt[c];"),
    ("no_erase_path_into_dk", "dkt[c] += de[c] * bt[c];", "(void)0;"),
    ("dw_dv_swapped", "dwt[j] = du[j] * vt[j];", "dwt[j] = du[j] * wt[j];"),
    ("no_final_state_seed", "if (dSf) memcpy(dS, dSf + soff, sz * sizeof(double));", ""),
]


def _mutate(src: str, old: str, new: str, fn: str = "recurrent_chain") -> str:
    start = src.index(f"static void {fn}(")
    ends = [i for i in (src.find("\nstatic ", start + 1), src.find("#define CHAIN_LOOP", start)) if i > 0]
    end = min(ends)  # the next function, or the exported wrappers
    body = src[start:end]
    assert body.count(old) == 1, f"mutation anchor not unique in {fn}: {old!r}"
    return src[:start] + body.replace(old, new) + src[end:]


def _pins_failing(lib_path, pins=None):
    orc = oracle.Oracle(oracle.load(lib_path))
    failing = []
    for pin in (oracle_pins.PINS if pins is None else pins):
        try:
            pin(orc)
        except AssertionError:
            failing.append(pin.__name__)
    return failing


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="gdn2_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_copy_passes(tmpdir_mod):
    src = open(obuild.SRC).read()
    path = os.path.join(tmpdir_mod, "clean.c")
    open(path, "w").write(src)
    lib = obuild.compile_oracle(path, os.path.join(tmpdir_mod, "libclean.so"))
    assert _pins_failing(lib) == []
    assert _pins_failing(lib, oracle_pins.BACKWARD_PINS) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmpdir_mod, name, old, new):
    src = _mutate(open(obuild.SRC).read(), old, new)
    path = os.path.join(tmpdir_mod, f"{name}.c")
    open(path, "w").write(src)
    lib = obuild.compile_oracle(path, os.path.join(tmpdir_mod, f"lib{name}.so"))
    failing = _pins_failing(lib)
    assert failing, f"mutant {name} passes every pin"


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_backward_mutant_is_caught(tmpdir_mod, name, old, new):
    src = _mutate(open(obuild.SRC).read(), old, new, fn="backward_chain")
    path = os.path.join(tmpdir_mod, f"bwd_{name}.c")
    open(path, "w").write(src)
    lib = obuild.compile_oracle(path, os.path.join(tmpdir_mod, f"libbwd_{name}.so"))
    failing = _pins_failing(lib, oracle_pins.BACKWARD_PINS)
    assert failing, f"backward mutant {name} passes every backward pin"
