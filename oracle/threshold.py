"""Query-count threshold between the absorbed and materialised MLA paths.

TEST INFRASTRUCTURE ONLY (the oracle): imported by the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the product path.

Two independent routes to the same integer, so that each checks the other:

* closed form -- the helper of "One guard, 110x off the verify step", section
  "The change" (denominator 2r - n - v; a non-positive denominator gives 1;
  otherwise the floor of r(n+v)/denominator, clamped below at 1), and the
  finite-cache form of mlx-lm PR #1817 ("fix: Speed up multi-token decode by
  computing the absorbed MLA threshold", opening paragraphs): with d = n + v
  and T the cache length, absorbed wins while L < r d / (r d / T + 2r - d).
  Both are evaluated in exact integer arithmetic (the PR's review thread
  suggests integers to avoid float-boundary rounding).

* cost-model search -- the per-head cost model of "One guard...", section
  "The threshold is not a constant": absorbed ~ 2 L Kv r (attention) +
  L r (n+v) (fold); materialised ~ Kv r (n+v) (expand) + L Kv (n+v) (attend).
  The limit form drops the fold term and divides by Kv.  The search walks L
  upward and returns the last L at which absorbed costs no more than
  materialised.

Readings (where the pages leave a point open):
* ties go to the absorbed path: the guard is ``L <= max_absorbed`` ("The
  change"), so max_absorbed is the largest L with absorbed <= materialised;
* T is the latent length the block attends over, including its own L rows;
  T == 0 selects the limit form;
* the clamp to at least 1, and the return of 1 for a non-positive
  denominator 2r - n - v, apply to the finite form as well, so a single
  query always takes the absorbed path.
"""

from __future__ import annotations

ABSORBED = 0
MATERIALIZED = 1


def max_absorbed_closed(r: int, n: int, v: int, T: int = 0) -> int:
    """Closed form, exact integers.  T == 0 is the long-cache limit."""
    r, n, v, T = int(r), int(n), int(v), int(T)
    d = n + v
    denom = 2 * r - d
    if denom <= 0:
        return 1
    if T == 0:
        q = (r * d) // denom
    else:
        # L < r d / (r d / T + 2r - d)  <=>  L <= floor(T r d / (r d + T (2r - d)))  (ties absorbed)
        q = (T * r * d) // (r * d + T * denom)
    return max(1, q)


def absorbed_cost(r: int, n: int, v: int, L: int, T: int) -> int:
    """Per-head multiply-adds of the absorbed path; T == 0: per unit Kv, fold dropped."""
    d = n + v
    if T == 0:
        return 2 * L * r
    return 2 * L * T * r + L * r * d


def materialized_cost(r: int, n: int, v: int, L: int, T: int) -> int:
    """Per-head multiply-adds of the materialised path; T == 0: per unit Kv."""
    d = n + v
    if T == 0:
        return r * d + L * d
    return T * r * d + L * T * d


def max_absorbed_search(r: int, n: int, v: int, T: int = 0, cap: int = 1 << 22) -> int:
    """Largest L >= 1 with absorbed_cost <= materialised_cost, by walking L upward."""
    r, n, v, T = int(r), int(n), int(v), int(T)
    if 2 * r - (n + v) <= 0:
        return 1
    best = 0
    L = 1
    while L <= cap and absorbed_cost(r, n, v, L, T) <= materialized_cost(r, n, v, L, T):
        best = L
        L += 1
    return max(1, best)


def select_path(r: int, n: int, v: int, L: int, T: int = 0) -> tuple[int, int]:
    """(path, max_absorbed): absorbed iff L <= max_absorbed."""
    m = max_absorbed_closed(r, n, v, T)
    return (ABSORBED if L <= m else MATERIALIZED), m
