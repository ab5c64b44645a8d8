"""Draft-cap cost model of speculative decoding.

TEST INFRASTRUCTURE ONLY (the oracle): imported by the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the product path.

"Draft caps and calibration" (mlx-dspark docs), section "Play with it": for a
cap C (drafted tokens verified per round), with p the probability that each
drafted token survives,

    speedup(C) ~ accepted(C) / (drafter + verify(C + 1))
    accepted(C) = 1 + p + p^2 + ... + p^C      tokens committed per round
    verify(w)   = cost of one pass over w rows, in single-token steps

and the section "How mlx-dspark picks it": the engine measures the verify
curve and the drafter's cost and derives the best fixed cap from them.

Readings (where the pages leave a point open):
* the measured verify costs may be in any unit; they are expressed in
  single-token steps by dividing by the cost of the one-row pass;
* caps run from 1 to W - 1 for a curve measured at widths 1..W (cap C
  verifies C + 1 rows);
* when no cap beats plain decoding (speedup <= 1) speculation is off: cap 0,
  speedup 1 (the same page parks speculation when it would lose);
* ties go to the smaller cap.
"""

from __future__ import annotations


def accepted(p: float, C: int) -> float:
    """Expected tokens committed per round: the sum of p^k for k = 0..C."""
    total = 0.0
    for k in range(C + 1):
        total += p ** k
    return total


def speedup(p: float, C: int, drafter: float, verify: list[float]) -> float:
    """speedup(C) with verify[w - 1] the measured cost of a w-row pass."""
    one_step = verify[0]
    return accepted(p, C) / (drafter + verify[C] / one_step)


def best_cap(p: float, drafter: float, verify: list[float]) -> tuple[int, float]:
    """(cap, speedup) maximising speedup over caps 1..len(verify) - 1; (0, 1.0)
    when none beats plain decoding."""
    cap, best = 0, 1.0
    for C in range(1, len(verify)):
        s = speedup(p, C, drafter, verify)
        if s > best:
            cap, best = C, s
    return cap, best
