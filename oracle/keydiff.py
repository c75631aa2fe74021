"""fp64 CPU oracle of KeyDiff eviction -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may use this module; the product library never does and shares no code
with it.  Plain numpy in float64, written from course module 14, section
14.4 (KeyDiff: eviction by key similarity) and exercise 14.2 (KeyDiff
eviction on a needle toy):
  * a cache is held to a budget of B tokens per (sequence, KV head);
  * a token's importance is how far its key lies from the mean key of the
    cache's tokens (distinctive keys draw attention, a cloud of similar keys
    does not), measured by the Euclidean distance as in the exercise;
  * the least distinctive tokens are evicted, the first `sink` positions
    never (the attention-sink guard);
  * the sequence arrives in blocks and the cache is brought back to the
    budget after every block, so it never holds more than B + block tokens.

Readings (listed with the design notes):
  * one eviction takes the mean over every token the cache holds at that
    moment (the new block included) and keeps, besides the sink, the
    B - sink tokens farthest from it; the exercise removes one token at a
    time and recomputes the mean after each removal, which gives the same
    set when one token is evicted (pinned), and which a one-shot kernel
    replaces for larger evictions;
  * among equal distances the earlier position is evicted first (the
    exercise takes the first minimum), so the later one is kept;
  * kept tokens keep their order; the evicted cache holds them in slots
    0 .. count-1.
"""
from __future__ import annotations

import numpy as np

from .semantic import attend  # noqa: F401  (softmax attention over a token set)


def anchor(keys: np.ndarray) -> np.ndarray:
    """Mean key of the tokens the cache holds."""
    return np.asarray(keys, dtype=np.float64).mean(axis=0)


def distances(keys: np.ndarray) -> np.ndarray:
    """Euclidean distance of every key to the mean key."""
    k = np.asarray(keys, dtype=np.float64)
    return np.sqrt(np.sum((k - anchor(k)) ** 2, axis=1))


def keep(keys: np.ndarray, budget: int, sink: int) -> np.ndarray:
    """Positions (ascending) kept by one eviction of a cache holding `keys`
    down to `budget` tokens: every position below `sink`, then the farthest
    from the mean key among the others (ties: the later position)."""
    n = len(keys)
    if n <= budget:
        return np.arange(n, dtype=np.int32)
    s0 = min(sink, n)
    if budget < s0:
        raise ValueError("budget below the sink")
    d = distances(keys)
    cand = sorted(range(s0, n), key=lambda i: (-d[i], -i))
    return np.array(sorted(list(range(s0)) + cand[: budget - s0]), dtype=np.int32)


def evict_one_at_a_time(keys: np.ndarray, budget: int, keep_first: int) -> np.ndarray:
    """The exercise's rule: while the cache is over budget, recompute the mean
    of the kept keys and drop the candidate (position >= keep_first) closest
    to it, the first one on ties.  Returns the kept positions ascending."""
    k = np.asarray(keys, dtype=np.float64)
    kept = np.arange(len(k))
    while len(kept) > budget:
        m = k[kept].mean(axis=0)
        cands = kept[kept >= keep_first]
        if len(cands) == 0:
            raise ValueError("budget below the sink")
        dist = np.sqrt(np.sum((k[cands] - m) ** 2, axis=1))
        kept = kept[kept != cands[int(np.argmin(dist))]]  # argmin: the first minimum
    return kept.astype(np.int32)


def blockwise(keys: np.ndarray, block: int, budget: int, sink: int):
    """The sequence's keys arrive `block` tokens at a time; after each block
    the cache is evicted back to `budget`.  Returns the positions the cache
    holds after every block (ascending)."""
    held = np.zeros(0, dtype=np.int64)
    states = []
    for t0 in range(0, len(keys), block):
        held = np.concatenate([held, np.arange(t0, min(t0 + block, len(keys)))])
        held = held[keep(keys[held], budget, sink)]
        states.append(held.astype(np.int32))
    return states
