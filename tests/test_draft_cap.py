"""Draft-cap cost model ("Draft caps and calibration", sections "Play with it"
and "How mlx-dspark picks it"): the oracle pinned to closed forms, a worked
example and an exact rational re-evaluation; the C ABI's mla_draft_cap against
the oracle (host-only entry point, no GPU needed)."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import draft_cap as dc


def test_accepted_geometric_closed_form():
    # 1 + p + ... + p^C = (1 - p^(C+1)) / (1 - p) for p != 1, C + 1 for p = 1
    for p in (Fraction(0), Fraction(1, 2), Fraction(3, 4), Fraction(9, 10), Fraction(1)):
        for C in range(0, 25):
            exact = Fraction(C + 1) if p == 1 else (1 - p ** (C + 1)) / (1 - p)
            assert dc.accepted(float(p), C) == pytest.approx(float(exact), rel=1e-14, abs=0)


def test_worked_example():
    # p = 0.8, drafter 0.1, verify curve 1.0, 1.1, 1.3, 1.6, 2.0 (widths 1..5):
    #   C = 1: 1.8   / (0.1 + 1.1) = 1.5
    #   C = 2: 2.44  / (0.1 + 1.3) = 1.742857...
    #   C = 3: 2.952 / (0.1 + 1.6) = 1.736470...
    #   C = 4: 3.3616 / (0.1 + 2.0) = 1.600761...
    verify = [1.0, 1.1, 1.3, 1.6, 2.0]
    want = [1.5, 2.44 / 1.4, 2.952 / 1.7, 3.3616 / 2.1]
    for C, w in zip(range(1, 5), want):
        assert dc.speedup(0.8, C, 0.1, verify) == pytest.approx(w, rel=1e-13)
    assert dc.best_cap(0.8, 0.1, verify) == (2, pytest.approx(2.44 / 1.4, rel=1e-13))


def test_flat_curve_drafts_to_the_limit():
    # verifying w rows costs the same as one (the page's datacenter case): with a
    # free drafter every extra draft adds expected tokens, so the largest cap wins
    verify = [1.0] * 9
    cap, s = dc.best_cap(0.7, 0.0, verify)
    assert cap == 8 and s == pytest.approx(dc.accepted(0.7, 8))


def test_no_survivors_means_no_speculation():
    cap, s = dc.best_cap(0.0, 0.05, [1.0, 1.01, 1.02])
    assert (cap, s) == (0, 1.0)


def test_unit_of_the_curve_does_not_matter():
    verify = [3.7, 4.1, 4.9, 6.0, 7.7]
    scaled = [x * 1e-6 for x in verify]
    assert dc.best_cap(0.85, 0.2, verify)[0] == dc.best_cap(0.85, 0.2, scaled)[0]


def _exact_best(p, drafter, verify):
    p, drafter = Fraction(p), Fraction(drafter)
    verify = [Fraction(v) for v in verify]
    best, cap = Fraction(1), 0
    for C in range(1, len(verify)):
        acc = sum(p ** k for k in range(C + 1))
        s = acc / (drafter + verify[C] / verify[0])
        if s > best:
            best, cap = s, C
    return cap, best


def _curves(seed, count=300):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        W = int(rng.integers(1, 17))
        steps = rng.uniform(0.0, 0.4, size=W)
        steps[0] = 0.0
        verify = list(np.cumsum(steps) + rng.uniform(0.5, 2.0))   # increasing curve, arbitrary unit
        yield float(rng.uniform(0.0, 1.0)), float(rng.uniform(0.0, 0.5)), verify


def test_oracle_matches_exact_rational_evaluation():
    for p, drafter, verify in _curves(1):
        cap, best = dc.best_cap(p, drafter, verify)
        ecap, ebest = _exact_best(p, drafter, verify)
        assert cap == ecap
        assert best == pytest.approx(float(ebest), rel=1e-12)


def test_c_abi_matches_oracle():
    import mla_speculative_decode_amd as mla
    for p, drafter, verify in list(_curves(2)) + [(0.8, 0.1, [1.0, 1.1, 1.3, 1.6, 2.0]), (1.0, 0.0, [2.0] * 5),
                                                  (0.0, 0.0, [1.0])]:
        cap, best, by_cap = mla.draft_cap(verify, p, drafter)
        ocap, obest = dc.best_cap(p, drafter, verify)
        assert cap == ocap
        assert best == pytest.approx(obest, rel=1e-12)
        assert by_cap[0] == 1.0
        for C in range(1, len(verify)):
            assert by_cap[C] == pytest.approx(dc.speedup(p, C, drafter, verify), rel=1e-12)


def test_c_abi_rejects_bad_arguments():
    import mla_speculative_decode_amd as mla
    from mla_speculative_decode_amd._lib import MlaError
    for args in (([], 0.5, 0.1), ([1.0, 2.0], 1.5, 0.1), ([1.0, 2.0], -0.1, 0.1), ([1.0, 2.0], 0.5, -1.0),
                 ([1.0, 0.0], 0.5, 0.1), ([1.0, float("nan")], 0.5, 0.1), ([1.0, 2.0], 0.5, float("inf"))):
        with pytest.raises(MlaError):
            mla.draft_cap(*args)
