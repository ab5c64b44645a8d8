"""Pins of the oracle's query-count threshold (CPU only).

The closed form and the cost-model search are two independent routes; they
are checked against each other over a grid, and both against the values the
pages print (tests/golden/thresholds.txt, each line citing its page).
"""

import math
from fractions import Fraction

import pytest

from oracle import threshold as th
from tests.conftest import golden_path


def _golden():
    rows = []
    with open(golden_path("thresholds.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            form, r, n, v, T, exp, *cite = line.split()
            rows.append((form, int(r), int(n), int(v), int(T), int(exp), " ".join(cite)))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]}-{r[1]}/{r[2]}/{r[3]}-T{r[4]}")
def test_printed_thresholds(row):
    form, r, n, v, T, exp, cite = row
    if form == "unfloored":
        ratio = Fraction(r * (n + v), 2 * r - n - v)
        assert round(ratio) == exp, cite
        assert math.floor(ratio) == th.max_absorbed_closed(r, n, v), cite
        return
    TT = 0 if form == "limit" else T
    assert th.max_absorbed_closed(r, n, v, TT) == exp, cite
    assert th.max_absorbed_search(r, n, v, TT) == exp, cite


def test_nonpositive_denominator_gives_one():
    # "The change": a non-positive 2r - n - v returns 1.
    for (r, n, v) in [(128, 128, 128), (64, 128, 0), (100, 150, 60), (1, 1, 1)]:
        assert 2 * r - n - v <= 0
        for T in (0, 1, 7, 8192):
            assert th.max_absorbed_closed(r, n, v, T) == 1
            assert th.max_absorbed_search(r, n, v, T) == 1


def test_tie_goes_to_absorbed():
    # 512/256/256: r(n+v)/(2r-n-v) = 512 exactly; the guard is L <= max_absorbed.
    assert th.select_path(512, 256, 256, 512) == (th.ABSORBED, 512)
    assert th.select_path(512, 256, 256, 513) == (th.MATERIALIZED, 512)
    # at the tie the two cost-model sides are equal
    assert th.absorbed_cost(512, 256, 256, 512, 0) == th.materialized_cost(512, 256, 256, 512, 0)


def test_cold_cache_materialised_wins():
    # PR #1817 opening: on a cold cache (T == L) the order reverses and materialising wins.
    for (r, n, v) in [(512, 128, 128), (512, 192, 256), (512, 256, 256), (256, 64, 64), (1024, 128, 512)]:
        for L in (2, 3, 8, 64, 379, 2048):
            path, m = th.select_path(r, n, v, L, T=L)
            assert path == th.MATERIALIZED and m < L
        # L == 1 is clamped to the absorbed path ("L=1 takes the same branch either way")
        assert th.select_path(r, n, v, 1, T=1)[0] == th.ABSORBED


def test_finite_form_tends_to_limit():
    for (r, n, v) in [(512, 128, 128), (512, 192, 256), (512, 256, 256)]:
        lim = th.max_absorbed_closed(r, n, v, 0)
        prev = 0
        for T in (1, 16, 512, 2048, 8192, 32768, 1 << 20, 1 << 30, 1 << 40):
            m = th.max_absorbed_closed(r, n, v, T)
            assert m >= prev and m <= lim
            prev = m
        # the finite bound approaches the limit from below: it reaches the limit's
        # floor unless the limit ratio is itself an integer (512/256/256), where it
        # stops one short
        exact = (r * (n + v)) % (2 * r - n - v) == 0
        assert th.max_absorbed_closed(r, n, v, 1 << 40) == (lim - 1 if exact else lim)


def test_known_finite_values():
    # values the closed form gives and the search confirms (not printed on the pages)
    expect = {(512, 128, 128): {512: 128, 2048: 157, 8192: 167, 32768: 169},
              (512, 256, 256): {512: 256, 2048: 409, 8192: 481, 32768: 504}}
    for geo, tab in expect.items():
        for T, m in tab.items():
            assert th.max_absorbed_closed(*geo, T) == m
            assert th.max_absorbed_search(*geo, T) == m


def test_closed_form_equals_search_grid():
    checked = 0
    for r in range(64, 1025, 64):
        for n in range(0, 513, 64):
            for v in range(0, 513, 64):
                d = n + v
                if 2 * r - d > 0 and r * d // (2 * r - d) > 5000:
                    continue  # keep the linear search short; large ratios are covered below
                for T in (0, 1, 2, 63, 512, 8192, 65536):
                    assert th.max_absorbed_closed(r, n, v, T) == th.max_absorbed_search(r, n, v, T), (r, n, v, T)
                    checked += 1
    assert checked > 5000


def test_closed_form_equals_search_large_ratio():
    # denominators of 1..4 give very large thresholds
    for (r, n, v) in [(512, 511, 512), (512, 512, 510), (256, 255, 255), (100, 99, 100)]:
        for T in (0, 4096, 65536):
            assert th.max_absorbed_closed(r, n, v, T) == th.max_absorbed_search(r, n, v, T)


def test_float_helper_agrees_with_integers():
    # The page's helper computes int(r(n+v)/denom) in floating point; on these
    # geometries the integer form returns the same value.
    for r in range(64, 1025, 32):
        for n in range(0, 513, 32):
            for v in range(0, 513, 32):
                denom = 2 * r - n - v
                ref = 1 if denom <= 0 else max(1, int(r * (n + v) / denom))
                assert th.max_absorbed_closed(r, n, v) == ref


def test_m3max_measured_ordering_consistent_with_limit():
    # The M3 Max sweep (PR #1817, "Where the paths cross") found absorbed faster at
    # L = 1 and 398 and materialised faster at 512 and 2048; the limit threshold 398
    # sends each of those L to the faster side.
    rows = []
    with open(golden_path("crossover_m3max.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                L, a, m = line.split()
                rows.append((int(L), float(a), float(m)))
    for L, a, m in rows:
        faster = th.ABSORBED if a < m else th.MATERIALIZED
        assert th.select_path(512, 192, 256, L, T=0)[0] == faster
