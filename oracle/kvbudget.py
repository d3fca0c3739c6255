"""The Initial-Key KV cache, written out plainly over the oracle model.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and nothing else).  The GPU library never
imports, links or runs it; it shares no code with the HIP path.

What is computed, from the C17 engine article (5.3, Initial-Key Cache): when a sequence's
KV cache holds more positions than the budget, only three kinds of positions keep their
K/V -- the initial ones (the first positions of the sequence, where attention pools), the
recent ones (the last positions), and the most important of the rest, ranked by a running
sum of the attention they received in the last few layers -- and the others are evicted.
With a budget at least the sequence's length nothing is evicted and the result is the full
cache's.

Readings where the page leaves a step open:
  * initial = the sequence's first n_initial positions; recent = its last n_recent kept
    positions (the newest included); the middle keeps budget - n_initial - n_recent
    positions with the largest scores, equal scores going to the earlier position;
  * a position's score is the softmax probability it receives from each later query,
    summed over the query heads and over the last score_layers layers, accumulated while it
    is kept (an evicted position never comes back);
  * eviction runs after a token's step whenever more than `budget` positions are kept,
    and brings the count back to `budget`;
  * a prompt is run position by position without eviction; only its last position's query
    adds to the scores; eviction then runs once (the GPU prefills a prompt as batched chunks
    and scores the last position's attention the same way);
  * positions keep their RoPE rotation: a kept key stays rotated by its own position, and a
    new token is rotated by its true position, whatever was evicted before it.
"""
from __future__ import annotations

import numpy as np


def select_kept(positions, scores, budget: int, n_initial: int, n_recent: int):
    """The positions (sorted) that stay when `positions` (sorted, kept so far) exceed the
    budget: the sequence's first n_initial positions, the last n_recent, and the
    highest-scoring others (earlier position first on equal scores)."""
    positions = list(positions)
    if len(positions) <= budget:
        return positions
    init = [p for p in positions if p < n_initial]
    rest = [p for p in positions if p >= n_initial]
    recent = rest[len(rest) - n_recent:] if n_recent > 0 else []
    middle = rest[:len(rest) - n_recent] if n_recent > 0 else rest
    k = budget - len(init) - len(recent)
    ranked = sorted(middle, key=lambda p: (-scores[p], p))
    return sorted(init + recent + ranked[:max(k, 0)])


class BudgetedSeq:
    """One sequence of an oracle.Model under a KV budget."""

    def __init__(self, model, slot: int, budget: int, n_initial: int, n_recent: int, score_layers: int):
        assert budget >= n_initial + n_recent + 1
        self.m = model
        self.slot = slot
        self.budget, self.n_initial, self.n_recent, self.score_layers = budget, n_initial, n_recent, score_layers
        self.kept = []                      # kept positions, ascending
        self.scores = np.zeros(model.max_ctx)
        self.pos = 0                        # the next token's position

    def _run(self, token, score):
        keep = np.zeros(self.pos + 1, dtype=np.uint8)
        keep[self.kept] = 1
        keep[self.pos] = 1
        sc = self.scores if score else np.zeros(self.pos + 1)
        nxt, logits = self.m.step_kept(self.slot, token, self.pos, keep, self.score_layers if score else 0, sc)
        self.kept.append(self.pos)
        self.pos += 1
        return nxt, logits

    def _evict(self):
        keep = select_kept(self.kept, self.scores, self.budget, self.n_initial, self.n_recent)
        gone = sorted(set(self.kept) - set(keep))
        self.scores[gone] = 0.0
        self.kept = keep

    def prefill(self, tokens):
        out = None
        for i, t in enumerate(tokens):
            out = self._run(int(t), score=(i == len(tokens) - 1))
        self._evict()
        return out

    def step(self, token):
        out = self._run(int(token), score=True)
        self._evict()
        return out
