"""Planted mistakes in the oracle (built on the CPU only) must each fail a pin.

Every variant is the oracle source compiled with -DORC_MUTANT=k; the list
below names the mistake each one plants.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    1: "merge advances the wrong pointer on a smaller query index",
    2: "norm sums |v| instead of v^2",
    3: "no zero-norm guard (0/0)",
    4: "divides the dot by the query norm only",
    5: "transpose scatters items in reverse order",
    6: "transpose stores global instead of chunk-local item ids",
    7: "row checksum uses raw instead of normalised query values",
    8: "merge multiplies the query value by itself (wrong operand)",
    9: "absolute-value closed form keeps the sign",
}


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_mutant_is_caught(k, tmp_path):
    path = oracle.build(path=os.path.join(str(tmp_path), "mut%d.so" % k), mutant=k)
    o = oracle.Oracle(path)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %d (%s) passed every pin" % (k, MUTANTS[k])
