"""Stochastic next-token sampling, written out plainly in float64.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and nothing else).  The GPU library never
imports, links or runs it; it shares no code with the HIP sampler.

What is computed, from the pages' description of the sampler (the nxmr.cn C17 engine
article, 4.6; the smollm3.go walkthrough, "sampling: from logits to the next token"):

  temperature  T = 0 is greedy: the largest logit (the lowest index among equal ones).
               T > 0 divides the logits by T and takes their softmax.
  top-k        k > 0 keeps the k most probable tokens and renormalises (k = 0: off).
  top-p        0 < p < 1 walks the tokens from most to least probable, summing their
               probabilities, and keeps the shortest run whose sum reaches p, then
               renormalises (p = 1: off).
  min-p        m > 0 keeps the tokens whose probability is at least m and renormalises
               (m = 0: off).
  seeded RNG   the same seed gives the same draws.

Readings where the pages leave a step open:
  * the filters apply in the order listed (temperature, top-k, top-p, min-p), each on the
    renormalised distribution the one before it left;
  * "most probable" orders tokens by logit, largest first, and equal logits by index;
  * min-p compares against the probabilities of the distribution top-k and top-p left; the
    most probable token always survives it;
  * the draw takes u uniform in [0, 1) and returns the first token, in vocabulary order,
    whose cumulative probability exceeds u (inverse transform sampling);
  * u comes from Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as
    easy as 1, 2, 3", SC 2011), a counter-based generator: key (seed, 0), counter
    (c, 0, 0, 0) where c is the position of the token whose logits are sampled, u = the
    top 53 bits of the block's first 64-bit word times 2^-53.  Draws depend only on
    (seed, position), not on which other sequences share a batch.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_MASK = (1 << 64) - 1
# Philox4x64 multipliers and key increments (Salmon et al. 2011, table 2 and section 4)
_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B


def philox4x64(counter, key, rounds=10):
    """One Philox4x64 block: four 64-bit words from a 256-bit counter and a 128-bit key.

    Each round multiplies words 0 and 2 by the two constants, keeps the 128-bit products'
    high and low halves, and permutes: (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1,
    lo(M0*x0)); the key advances by the two Weyl increments between rounds."""
    x = [int(c) & _MASK for c in counter]
    k0, k1 = int(key[0]) & _MASK, int(key[1]) & _MASK
    for r in range(rounds):
        if r:
            k0, k1 = (k0 + _W0) & _MASK, (k1 + _W1) & _MASK
        p0, p1 = _M0 * x[0], _M1 * x[2]
        x = [(p1 >> 64) ^ x[1] ^ k0, p1 & _MASK, (p0 >> 64) ^ x[3] ^ k1, p0 & _MASK]
    return x


def uniform(seed: int, counter: int) -> float:
    """u in [0, 1): the top 53 bits of the first word of block (counter, 0, 0, 0) under key
    (seed, 0), scaled by 2^-53 (exact in float64)."""
    w = philox4x64((counter, 0, 0, 0), (seed, 0))[0]
    return (w >> 11) * 2.0 ** -53


@dataclass
class Sampler:
    temperature: float = 0.0
    top_k: int = 0
    top_p: float = 1.0
    min_p: float = 0.0
    seed: int = 0


@dataclass
class Draw:
    token: int
    probs: np.ndarray        # final distribution over the vocabulary (zeros where removed)
    u: float                 # the uniform the draw used (nan for greedy)
    cut_margins: list        # per active filter: relative distance of its decision from a tie


def greedy(logits) -> int:
    l = np.asarray(logits, np.float64)
    return int(np.flatnonzero(l == l.max())[0])


def _order(l):
    """token ids from most to least probable: logit descending, then index ascending"""
    return np.lexsort((np.arange(l.size), -l))


def filtered_probs(logits, s: Sampler):
    """The distribution the draw uses (float64), and for each filter that cut something the
    relative distance of its cut from flipping (used to tell rounding ties from errors)."""
    l = np.asarray(logits, np.float64)
    if l.ndim != 1 or l.size == 0:
        raise ValueError("logits must be a non-empty vector")
    z = (l - l.max()) / s.temperature
    p = np.exp(z)
    p /= p.sum()
    order = _order(l)
    keep = np.zeros(l.size, bool)
    keep[order] = True
    margins = []
    if 0 < s.top_k < l.size:
        keep[order[s.top_k:]] = False
        p = np.where(keep, p, 0.0)
        p /= p.sum()
    if 0 < s.top_p < 1:
        ranked = order[keep[order]]
        cs = np.cumsum(p[ranked])
        reach = np.flatnonzero(cs >= s.top_p)
        n = int(reach[0]) + 1 if reach.size else ranked.size
        keep[ranked[n:]] = False
        # the sums on either side of the cut, relative to p
        below = cs[n - 2] if n >= 2 else 0.0
        margins.append(min(abs(cs[n - 1] - s.top_p), abs(s.top_p - below)) / s.top_p)
        p = np.where(keep, p, 0.0)
        p /= p.sum()
    if s.min_p > 0:
        top = order[0]
        kept_before = keep.copy()
        keep &= p >= s.min_p
        keep[top] = True
        cand = p[kept_before]
        margins.append(float(np.min(np.abs(cand - s.min_p))) / s.min_p)
        p = np.where(keep, p, 0.0)
        p /= p.sum()
    return p, margins


def sample(logits, s: Sampler, counter: int) -> Draw:
    """The next token for these logits under sampler s, drawing with counter `counter`."""
    if s.temperature < 0 or not np.isfinite(s.temperature):
        raise ValueError("temperature must be finite and >= 0")
    if s.temperature == 0:
        l = np.asarray(logits, np.float64)
        t = greedy(l)
        p = np.zeros(l.size)
        p[t] = 1.0
        return Draw(t, p, float("nan"), [])
    p, margins = filtered_probs(logits, s)
    u = uniform(s.seed, counter)
    cdf = np.cumsum(p)
    t = int(np.searchsorted(cdf, u, side="right"))
    if t >= p.size:                      # u at or past a total that rounded below 1
        t = int(np.flatnonzero(p > 0)[-1])
    return Draw(t, p, u, margins)


def draw_margin(d: Draw) -> float:
    """Relative distance of u from the nearest cumulative-probability boundary of the draw
    (how far the draw is from picking a neighbouring token)."""
    cdf = np.cumsum(d.probs)
    edges = cdf[d.probs > 0]
    return float(np.min(np.abs(edges - d.u))) if edges.size else float("inf")
