"""Pooled top-k indexer: window-of-four pooling with an incremental tail, scores, selection.

TEST INFRASTRUCTURE ONLY (the oracle): imported by the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the product path.

"One guard, 110x off the verify step", sections "The sparse model is
different" and "The same bug, one layer over":

* the indexer pools the cached keys into windows of four, windows starting at
  positions that are multiples of four, before scoring them, and picks the top
  `budget` cached positions (2048 on the pages);
* pooling the whole cache every step costs O(T), so completed windows are
  cached and only the tail is recomputed; a window completed before the tail
  cannot change, since tokens only append;
* the incremental path may be taken for any number S of new tokens, under four
  guards: the cache has a pool, there is no padding, the batch shape matches,
  and the cache is exactly as long as the pool remembers (a cache trimmed after
  a speculative rejection fails the last one, so a stale pool never carries
  rejected tokens forward);
* a wide step pools exactly as the same tokens fed one at a time.

Readings where the pages are silent: a window's pooled key is the mean of the
key rows it holds (the tail window, with fewer than four rows, the mean of
those); the score of a window is the dot product of a query vector (one per
sequence) with its pooled key; every position carries its window's score and
the selection is the first min(budget, T) positions in the order (score
descending, position ascending), returned in increasing position order; a
trimmed cache may also be announced to the pool, which then forgets the
windows past the trim point (the windows wholly before it are still exact).
Plain float64 loops.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WINDOW = 4


def n_windows(T: int) -> int:
    """Windows covering T cached positions (the last one may be partial)."""
    return (int(T) + WINDOW - 1) // WINDOW


def pool_window(keys, w: int, T: int):
    """Mean of the cached key rows of window w (rows 4w .. min(4w+4, T) - 1)."""
    rows = [np.asarray(keys[t], dtype=np.float64) for t in range(WINDOW * w, min(WINDOW * w + WINDOW, T))]
    acc = np.zeros_like(rows[0])
    for r in rows:
        acc = acc + r
    return acc / len(rows)


def pool_all(keys, T: int):
    """Pooled keys of every window of a cache of T positions: [n_windows(T), d]."""
    return np.stack([pool_window(keys, w, T) for w in range(n_windows(T))]) if T > 0 else np.zeros((0, keys.shape[1]))


@dataclass
class PoolState:
    """What the pool remembers between steps (one per batch of sequences)."""
    valid: bool = False
    batch: int = 0
    d: int = 0
    lengths: list = field(default_factory=list)     # cache length per sequence the pool covers
    pooled: list = field(default_factory=list)      # per sequence: dict window -> pooled key


def guards_hold(state: PoolState, lengths_now, S: int, d: int, padded: bool) -> bool:
    """The four conditions under which only the tail is recomputed."""
    B = len(lengths_now)
    return (state.valid                                   # the cache has a pool
            and not padded                                # there is no padding
            and state.batch == B and state.d == d         # the batch shape matches
            and all(state.lengths[b] == lengths_now[b] - S for b in range(B)))   # length remembered


def pool_step(state: PoolState, keys_per_seq, S: int, padded: bool = False):
    """One step that appended S tokens to every sequence (their caches now hold
    keys_per_seq[b] rows).  Returns True if the incremental path was taken."""
    lengths_now = [len(k) for k in keys_per_seq]
    d = keys_per_seq[0].shape[1]
    B = len(keys_per_seq)
    incremental = guards_hold(state, lengths_now, S, d, padded)
    if not incremental:
        state.pooled = [dict() for _ in range(B)]
    for b in range(B):
        T = lengths_now[b]
        first = (T - S) // WINDOW if incremental else 0    # the old tail window and everything after
        for w in range(first, n_windows(T)):
            state.pooled[b][w] = pool_window(keys_per_seq[b], w, T)
    state.valid, state.batch, state.d = True, B, d
    state.lengths = list(lengths_now)
    return incremental


def pool_trim(state: PoolState, new_lengths):
    """The caches were cut back to new_lengths (positions at or past them were
    rejected): the pool forgets every window that held a rejected row (the one
    cut through included); the next step recomputes from there."""
    for b, n in enumerate(new_lengths):
        if n < state.lengths[b]:
            state.lengths[b] = int(n)
            for w in [w for w in state.pooled[b] if w >= int(n) // WINDOW]:
                del state.pooled[b][w]


def pooled_array(state: PoolState, b: int):
    T = state.lengths[b]
    return np.stack([state.pooled[b][w] for w in range(n_windows(T))])


def window_scores(pooled, q):
    """Score of every window: q . pooled key (reading of the pages' unnamed score)."""
    pooled = np.asarray(pooled, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    return np.array([float(np.dot(q, pooled[w])) for w in range(pooled.shape[0])])


def select_positions(window_score, T: int, budget: int):
    """The top min(budget, T) positions, each carrying its window's score, in the
    order (score descending, position ascending); returned increasing."""
    ws = np.asarray(window_score, dtype=np.float64)
    order = sorted(range(int(T)), key=lambda t: (-ws[t // WINDOW], t))
    return np.array(sorted(order[:min(int(budget), int(T))]), dtype=np.int64)


# ---- fixed-capacity update list ----------------------------------------------
# "Over 107 tok/s Qwen3.8-Flash-Next on M3 Ultra", section "Why doing eight rows
# can beat doing two" and its algorithm for constructing a fixed-capacity update
# list, read for this indexer: a block is a window of four positions, its
# destination is the window's own slot in the pooled array, the real updates of
# a step are the windows it must recompute (the old tail window and the new
# ones), and the complete blocks are the windows holding four rows.  Padding the
# real updates to P rows with complete, unchanged windows at destinations not
# yet in the list gives every step the same shape; each filler pools its own
# unchanged rows again, so its write reproduces the value already stored.

def update_list(delta, complete, P, m, streams=1, padding=True, fallback=None):
    """The ordered update list U and its capacity C.  delta: real updates in
    order; complete: the complete windows in order; P: target capacity (8 or
    16); m: tokens in the step (microbatch); fallback: the descriptor used when
    there is neither an update nor a complete window."""
    C = max(1, len(delta))
    U = list(delta)
    if padding and m <= 16 and streams == 1 and C <= P and len(complete) >= P:
        C = P
    if not U:
        U.append(complete[0] if complete else fallback)
    if padding and streams == 1:
        for b in complete:
            if len(U) == C:
                break
            if b not in U:          # destination of window b is its own slot
                U.append(b)
        assert len(U) == C
    else:
        while len(U) < C:           # the first row repeated
            U.append(U[0])
    return U, C


def pool_step_fixed(state: PoolState, keys_per_seq, S: int, P: int = 8, padded: bool = False):
    """pool_step, except that an incremental step recomputes the fixed-capacity
    update list of each sequence (real updates padded with idempotent fillers).
    Returns (incremental, lists): the list recomputed per sequence (None where
    every window was recomputed)."""
    lengths_now = [len(k) for k in keys_per_seq]
    d = keys_per_seq[0].shape[1]
    B = len(keys_per_seq)
    incremental = guards_hold(state, lengths_now, S, d, padded)
    if not incremental:
        state.pooled = [dict() for _ in range(B)]
    lists = []
    for b in range(B):
        T = lengths_now[b]
        if incremental:
            delta = list(range((T - S) // WINDOW, n_windows(T)))
            U, _ = update_list(delta, list(range(T // WINDOW)), P, S)
        else:
            U = None
        for w in (U if U is not None else range(n_windows(T))):
            state.pooled[b][w] = pool_window(keys_per_seq[b], w, T)
        lists.append(U)
    state.valid, state.batch, state.d = True, B, d
    state.lengths = list(lengths_now)
    return incremental, lists
