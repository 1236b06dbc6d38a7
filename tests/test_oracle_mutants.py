"""Every planted mistake in the oracle fails at least one pin.

Each mutant is a build of ``oracle/kda_oracle.c`` with ``-DKDA_ORACLE_MUTANT=n``:
1 decay after the write, 2 read before the write, 3 decay along value columns,
4 erase sign flipped, 5 beta applied to v only, 6 alpha = exp(-g),
7 key dropped from the rank-1 write, 8 read with k instead of q."""
import os

import pytest

import oracle
from pins import RECURRENCE_PINS

MUTANTS = list(range(1, 9))


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(tmp_path, mutant):
    path = os.path.join(tmp_path, f"libkda_oracle_m{mutant}.so")
    oracle.build(path, mutant=mutant)
    orc = oracle.Oracle(path)
    assert orc.mutant == mutant
    failed = []
    for pin in RECURRENCE_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant} passed every pin"
