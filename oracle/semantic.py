"""fp64 CPU oracle of the semantic block index -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may use this module; the product library never does and shares no code
with it.  Plain numpy in float64, written from the semantic-blocks page
(rit.work blog, *semantic blocks sparse attention*): per request, layer and
KV head the normalised keys are grouped into semantic blocks by spherical
k-means; keys and values are laid out block by block; a query is compared
with the block centres, the best blocks are taken up to a token budget and
ordinary attention runs over the original keys and values inside them; the
current fragment and recent history are attended without selection.

Where the page leaves a step open this module takes the plainest reading
(each is listed with the design notes):
  * the index covers the positions [0, N) of a sequence (the prefix before
    the recent history), with C blocks (C = ceil(N / 2048) by default, the
    page's average block of 2048 tokens);
  * k-means starts from the unit keys at the evenly spaced positions
    floor(c * N / C) and runs a fixed number of iterations;
  * a key goes to the centre with the largest dot product (ties: the lower
    centre); a centre becomes the normalised sum of its unit keys; a centre
    with no keys (or a zero sum) keeps its previous value;
  * blocks are the final clusters; inside a block the tokens keep their
    position order;
  * a query row scores block c by the largest q_h . centre_c over the heads
    of its group; blocks are taken in order of score (ties: lower block)
    while the running token count stays within the budget, at least one;
    blocks without tokens are never taken;
  * the prompt is processed in chunks of rows over one index of the whole
    prompt (one index serves the prompt and the generation): a chunk's
    window (its own rows and the recent history) is attended causally
    without selection, and of the index it sees only the tokens before the
    window, so a block's size for the budget is its visible part.
"""
from __future__ import annotations

import numpy as np


def unit_keys(keys: np.ndarray) -> np.ndarray:
    """Each key divided by its length (a zero key stays zero)."""
    k = np.asarray(keys, dtype=np.float64)
    n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    return np.divide(k, n, out=np.zeros_like(k), where=n > 0)


def init_centres(u: np.ndarray, C: int) -> np.ndarray:
    """The unit keys at positions floor(c * N / C), c = 0 .. C-1."""
    N = u.shape[0]
    return u[(np.arange(C, dtype=np.int64) * N) // C].copy()


def assign(u: np.ndarray, centres: np.ndarray) -> np.ndarray:
    """Index of the centre with the largest dot product for every key
    (argmax returns the first, i.e. lower, index on ties)."""
    return np.argmax(u @ centres.T, axis=1).astype(np.int32)


def update(u: np.ndarray, a: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """Normalised sum of each cluster's unit keys; clusters without keys (or
    with a zero sum) keep their previous centre."""
    C = prev.shape[0]
    s = np.zeros_like(prev)
    np.add.at(s, a, u)
    n = np.sqrt(np.sum(s * s, axis=1, keepdims=True))
    return np.where(n > 0, np.divide(s, n, out=np.zeros_like(s), where=n > 0), prev)


def objective(u: np.ndarray, centres: np.ndarray, a: np.ndarray) -> float:
    """Sum over keys of the cosine to their centre."""
    return float(np.sum(np.einsum("nd,nd->n", u, centres[a])))


def spherical_kmeans(keys: np.ndarray, C: int, iters: int):
    """Returns (centres after `iters` updates, final assignment to them,
    objective after every update)."""
    u = unit_keys(keys)
    mu = init_centres(u, C)
    hist = []
    for _ in range(iters):
        a = assign(u, mu)
        mu = update(u, a, mu)
        hist.append(objective(u, mu, assign(u, mu)))
    return mu, assign(u, mu), hist


def block_layout(a: np.ndarray, C: int):
    """Tokens grouped block by block, position order inside a block:
    (perm[i] = position of row i of the blocked layout, offsets[C + 1])."""
    counts = np.bincount(a, minlength=C)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(a, kind="stable").astype(np.int32)
    return perm, offsets


def block_scores(qg: np.ndarray, centres: np.ndarray) -> np.ndarray:
    """Largest q_h . centre_c over the heads of the group, for every block."""
    return np.max(np.asarray(qg, dtype=np.float64) @ centres.T, axis=0)


def select_blocks(scores: np.ndarray, sizes: np.ndarray, budget: int, k_max: int) -> np.ndarray:
    """Blocks in order of (score desc, block asc), taken while the running
    token count stays <= budget (the first one always), at most k_max;
    empty blocks are skipped.  Returned ascending."""
    order = sorted((c for c in range(len(scores)) if sizes[c] > 0), key=lambda c: (-scores[c], c))
    taken, total = [], 0
    for c in order:
        if len(taken) >= k_max:
            break
        if taken and total + int(sizes[c]) > budget:
            break
        taken.append(c)
        total += int(sizes[c])
    return np.array(sorted(taken), dtype=np.int32)


def visible_sizes(perm: np.ndarray, offsets: np.ndarray, bound: int) -> np.ndarray:
    """Tokens of each block at positions before `bound` (the part of the
    index a prompt chunk may see: everything before its window)."""
    C = len(offsets) - 1
    return np.array([int(np.sum(perm[offsets[c]:offsets[c + 1]] < bound)) for c in range(C)], dtype=np.int64)


def prefill_chunk(K, V, qrows, centres, perm, offsets, c0: int, window: int, budget: int, k_max: int,
                  scale: float):
    """One chunk of a sparse prefill over an index of the whole prompt.  Rows
    i = 0 .. len(qrows)-1 sit at positions c0 + i; the chunk's window is
    [c0 + T - window, c0 + T) (T rows), attended causally and without
    selection; before it each row chooses blocks by centre score among their
    visible parts (positions before the window) under the token budget.
    qrows[i] is the [G][hd] query group of row i.  Returns, per row, the
    chosen blocks and the per-head (output, lse)."""
    T = len(qrows)
    bound = c0 + T - window
    vis = visible_sizes(perm, offsets, bound)
    res = []
    for i in range(T):
        pos = c0 + i
        qg = np.asarray(qrows[i], dtype=np.float64)
        blocks = select_blocks(block_scores(qg, centres), vis, budget, k_max)
        toks = np.concatenate([perm[offsets[x]:offsets[x + 1]][perm[offsets[x]:offsets[x + 1]] < bound]
                               for x in blocks] + [np.arange(max(0, bound), pos + 1)]).astype(np.int64)
        res.append((blocks, [attend(qg[h], K[toks], V[toks], scale) for h in range(len(qg))]))
    return res


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Softmax attention of one query over the given keys and values:
    (output, log-sum-exp)."""
    z = scale * (np.asarray(keys, dtype=np.float64) @ np.asarray(q, dtype=np.float64))
    m = np.max(z)
    w = np.exp(z - m)
    l = np.sum(w)
    return (w @ np.asarray(values, dtype=np.float64)) / l, float(m + np.log(l))
