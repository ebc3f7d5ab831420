"""Planted mistakes: each deliberately broken oracle build must fail at least one pin."""
import os
import tempfile

import pytest

import oracle
import oracle_pins as P
from oracle import build as ob

MUTANTS = {
    1: "tie-break by id descending",
    2: "mask test passes when any required bit is set",
    3: "one probe too few",
    4: "coarse ranks clusters by ascending score",
    5: "dot product drops the last dimension",
    6: "Bloom bit index taken from the wrong bits",
    7: "dequantisation ignores the query scale",
    8: "a request of several masks tests only its first one",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_rejected(mutant):
    with tempfile.TemporaryDirectory() as td:
        path = ob.build(out=os.path.join(td, f"liboracle_m{mutant}.so"), mutant=mutant)
        orc = oracle.Oracle(path)
        failed = []
        for pin in P.ALL_PINS:
            kwargs = {"trials": 100_000} if pin is P.pin_bloom else {}
            try:
                pin(orc, **kwargs)
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"
