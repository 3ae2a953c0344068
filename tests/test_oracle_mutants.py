"""Each planted mistake in the oracle (a dropped term, an off-by-one bound, a
wrong head or batch index, a transposed operand) must fail at least one pin.

The mutants are compiled from mfa_oracle.c with -DORACLE_MUTANT=n on the CPU.
"""
import os

import pytest

from oracle import Oracle, build_oracle
from tests.oracle_pins import ALL_PINS

MUTANTS = {
    1: "scale dropped",
    2: "causal bound excludes the diagonal",
    3: "causal window one key too wide",
    4: "kv head chosen by modulo instead of grouping",
    5: "K used in place of V",
    6: "LSE without the max shift",
    7: "soft-cap without the division by the cap",
    8: "key mask ignored",
    9: "bidirectional window twice as wide",
    10: "q_offset ignored",
    11: "softmax normalisation dropped",
    12: "Q indexed as [B, H, L, D]",
    13: "batch 0's key mask used for every batch",
    14: "soft-cap applied before the scale",
    15: "additive mask indexed with query and key swapped",
    16: "dropout pattern drawn with query and key swapped",
    17: "backward without the derivative of the scale and soft-cap",
    18: "dropout reading word 0 of the block for every key",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_pins_catch_mutant(mutant, tmp_path):
    path = os.path.join(str(tmp_path), f"libmfa_oracle_m{mutant}.so")
    build_oracle(path, mutant=mutant)
    orc = Oracle(path)
    assert orc.mutant == mutant
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mutant} ({MUTANTS[mutant]})"
