"""Every planted mistake in the oracle fails at least one pin.

Each mutant is a copy of ``oracle/kda_oracle.c`` with one line of the
recurrence replaced by a plausible mistake, compiled to its own library on the
CPU.  The replaced text must occur exactly once in the source, so that a change
to the oracle that moves it makes this test fail instead of silently testing
nothing."""
import os

import pytest

import oracle
from pins import CONV_PINS, RECURRENCE_PINS

# Lines of the recurrence as they stand in the oracle (each ends with the
# macro's line continuation).
DECAY = "for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];    \\"
WRITE_BLOCK = ("/* S_t = S' + k_t u_t^T */                                             \\\n"
               "                    for (int i = 0; i < dk; ++i)                                           \\\n"
               "                        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * u[j];\\\n")
READ_BLOCK = ("                    /* o_t = S_t^T q_t */                                                  \\\n"
              "                    for (int j = 0; j < dv; ++j) ot[j] = 0;                                \\\n"
              "                    for (int i = 0; i < dk; ++i)                                           \\\n"
              "                        for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];\\\n")
WRITE = "for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * u[j];\\"
U = "for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - y[j]);               \\"

# (name, [(text of the real oracle, the planted mistake), ...])
MUTANTS = [
    ("decay_after_write",
     [(DECAY, "for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= 1;           \\"),
      (WRITE, "for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = (S[(size_t)i * dv + j] "
              "+ kt[i] * u[j]) * alpha[i];\\")]),
    ("read_before_write", [(WRITE_BLOCK + READ_BLOCK,
                            READ_BLOCK.lstrip() + "                    " + WRITE_BLOCK)]),
    ("decay_along_value_columns",
     [(DECAY, "for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[j%dk];\\")]),
    ("erase_sign_flipped",
     [(U, "for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] + y[j]);               \\")]),
    ("beta_on_v_only",
     [(U, "for (int j = 0; j < dv; ++j) u[j] = bt * vt[j] - y[j];                 \\")]),
    ("alpha_exp_minus_g",
     [("for (int i = 0; i < dk; ++i) alpha[i] = (REAL)EXPF(gt[i]);             \\",
       "for (int i = 0; i < dk; ++i) alpha[i] = (REAL)EXPF(-gt[i]);            \\")]),
    ("key_dropped_from_write",
     [(WRITE, "for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += u[j];        \\")]),
    ("read_with_k",
     [("for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];\\",
       "for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * kt[i];\\")]),
    ("conv_tap_order_reversed",
     [("for (int j = 0; j < 4; ++j) acc += w[(size_t)c * 4 + j] * hist[t + j];",
       "for (int j = 0; j < 4; ++j) acc += w[(size_t)c * 4 + 3 - j] * hist[t + j];")]),
    ("l2_eps_outside_sqrt",
     [("const double inv = 1.0 / sqrt(ss + eps);",
       "const double inv = 1.0 / (sqrt(ss) + eps);")]),
]


@pytest.mark.parametrize("name,patches", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, patches):
    src = open(oracle.SRC).read()
    for real, planted in patches:
        assert src.count(real) == 1, f"{name}: the patched text is not found exactly once"
        src = src.replace(real, planted)
    mpath = os.path.join(tmp_path, f"kda_oracle_{name}.c")
    with open(mpath, "w") as f:
        f.write(src)
    lib = os.path.join(tmp_path, f"libkda_oracle_{name}.so")
    oracle.build(lib, src=mpath)
    orc = oracle.Oracle(lib)
    failed = []
    for pin in RECURRENCE_PINS + CONV_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
