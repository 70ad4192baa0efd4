"""Seeded sampling chain (test infrastructure; same rules of use as oracle.py).

The chain runs temperature -> top-k -> top-p -> renormalise -> draw, in that
order: "Coming back to Failed Star", section "Next: one complete
deterministic generation arc" (the sampling arc taken after greedy parity,
with an explicit filter order and known-answer tests); "Failed Star (fs)",
milestone M3 (temperature / top-k / top-p after greedy); "ferrite", section
"What it does" (greedy, temperature, top-k and top-p sampling).

The pages fix the order of the filters, not their rules.  Readings adopted
(each also listed in the design notes):

* temperature ``T > 0`` divides the logits before anything else; ``T == 0``
  is greedy selection (the argmax rule of oracle.greedy_argmax);
* only finite logits take part; a row with none gives -1;
* top-k keeps every token whose logit is >= the k-th largest finite logit
  (counted with multiplicity), so tokens tied with the k-th are all kept;
  ``k == 0`` means no limit;
* top-p works on the probabilities renormalised over the top-k set: with the
  tokens ranked by logit, it finds the first rank at which the cumulative
  mass reaches ``p`` and keeps every token at least as probable as the token
  at that rank (ties again all kept); ``p >= 1`` keeps the whole top-k set;
* the kept probabilities are renormalised, and one uniform ``u`` in [0, 1)
  (supplied by the caller, seeded) is mapped through the cumulative
  distribution taken in increasing token ID: the chosen token is the first
  whose cumulative probability exceeds ``u`` (the last kept token if rounding
  leaves ``u`` at or above the total).

Everything is float64 NumPy; the GPU computes in float32, so the test helper
``acceptable`` widens the comparison at boundaries that fall within a small
tolerance of the cut.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .oracle import greedy_argmax


def _finite_ids(x: np.ndarray) -> np.ndarray:
    return np.flatnonzero(np.isfinite(x))


def kth_largest(values: np.ndarray, k: int) -> float:
    """The k-th largest of ``values`` counted with multiplicity (1-based)."""
    srt = np.sort(values)[::-1]
    return float(srt[k - 1])


def kept_tokens(logits: np.ndarray, temperature: float, top_k: int, top_p: float
                ) -> Tuple[np.ndarray, np.ndarray]:
    """Token IDs kept by temperature -> top-k -> top-p, in increasing ID, and
    their renormalised probabilities (float64)."""
    x = np.asarray(logits, dtype=np.float64)
    ids = _finite_ids(x)
    if ids.size == 0:
        return ids, np.zeros(0)
    z = x[ids] / float(temperature)
    # top-k (tie-inclusive threshold on the scaled logits; T > 0 keeps the order)
    k = ids.size if top_k <= 0 else min(top_k, ids.size)
    tk = kth_largest(z, k)
    sel = z >= tk
    ids, z = ids[sel], z[sel]
    # probabilities over the top-k set
    w = np.exp(z - z.max())
    prob = w / w.sum()
    if top_p < 1.0:
        order = np.lexsort((ids, -z))          # rank: logit descending, ID ascending
        cum = np.cumsum(prob[order])
        r = int(np.searchsorted(cum, top_p, side="left"))
        r = min(r, order.size - 1)
        tp = z[order[r]]
        sel = z >= tp
        ids, prob = ids[sel], prob[sel]
    return ids, prob / prob.sum()


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float) -> int:
    """One draw of the chain for one row of logits (see the module notes)."""
    if temperature == 0.0:
        return greedy_argmax(np.asarray(logits))
    ids, q = kept_tokens(logits, temperature, top_k, top_p)
    if ids.size == 0:
        return -1
    cum = np.cumsum(q)
    j = int(np.searchsorted(cum, u, side="right"))
    return int(ids[min(j, ids.size - 1)])


def acceptable(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float,
               eps: float = 2e-5) -> List[int]:
    """Every token a correct float32 implementation may return for this draw.

    The result is unique unless the top-p cut or the draw lands within ``eps``
    (relative probability) of a boundary; then the neighbouring outcomes are
    also allowed.  Top-k decisions compare the given float32 logits exactly
    and need no slack.
    """
    if temperature == 0.0:
        return [greedy_argmax(np.asarray(logits))]
    x = np.asarray(logits, dtype=np.float64)
    ids0 = _finite_ids(x)
    if ids0.size == 0:
        return [-1]
    z0 = x[ids0] / float(temperature)
    k = ids0.size if top_k <= 0 else min(top_k, ids0.size)
    sel = z0 >= kth_largest(z0, k)
    ids, z = ids0[sel], z0[sel]
    w = np.exp(z - z.max())
    prob = w / w.sum()
    cuts = [None]
    if top_p < 1.0:
        order = np.lexsort((ids, -z))
        cum = np.cumsum(prob[order])
        cuts = sorted({int(np.searchsorted(cum, top_p - eps, side="left")),
                       int(np.searchsorted(cum, top_p, side="left")),
                       int(np.searchsorted(cum, top_p + eps, side="left"))})
        cuts = [z[order[min(r, order.size - 1)]] for r in cuts]
    out = set()
    for tp in cuts:
        keep = np.ones(ids.size, dtype=bool) if tp is None else (z >= tp)
        kid, q = ids[keep], prob[keep] / prob[keep].sum()
        cum = np.cumsum(q)
        for uu in (u - eps, u, u + eps):
            j = int(np.searchsorted(cum, min(max(uu, 0.0), np.nextafter(1.0, 0.0)), side="right"))
            out.add(int(kid[min(j, kid.size - 1)]))
    return sorted(out)
