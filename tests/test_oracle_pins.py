"""The float64 oracle against facts that do not come from the oracle itself."""
import pins


def test_worked_examples(orc):
    pins.pin_worked_examples(orc)


def test_bruteforce_dense(orc):
    pins.pin_bruteforce(orc)


def test_scipy_normalized_product(orc):
    pins.pin_scipy(orc)


def test_cosine_invariants(orc):
    pins.pin_invariants(orc)


def test_chunk_transpose_vs_scipy(orc):
    pins.pin_csc(orc)


def test_closed_form_checksums(orc):
    pins.pin_checksums(orc)


def test_validator(orc):
    import numpy as np
    from synth import HostCSR
    ok = pins.csr_from_rows([[(1, 1.0), (5, 2.0)], [], [(0, 3.0)]], 8)
    assert orc.validate(ok) == (0, -1)
    bad_order = HostCSR(ok.indptr, np.array([5, 1, 0], np.int32), ok.values, 3, 8)
    assert orc.validate(bad_order) == (2, 0)
    dup = HostCSR(ok.indptr, np.array([1, 1, 0], np.int32), ok.values, 3, 8)
    assert orc.validate(dup) == (2, 0)
    oob = HostCSR(ok.indptr, np.array([1, 5, 8], np.int32), ok.values, 3, 8)
    assert orc.validate(oob) == (3, 2)
    nan = HostCSR(ok.indptr, ok.indices, np.array([1, np.nan, 2], np.float32), 3, 8)
    assert orc.validate(nan) == (4, 0)
    ptr = HostCSR(np.array([0, 2, 1, 3], np.int32), ok.indices, ok.values, 3, 8)
    assert orc.validate(ptr)[0] == 1
