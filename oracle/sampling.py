"""Per-node vocabulary distributions and sampling rules (oracle; test infrastructure only).

* Effective distribution: the acceptance test must use the distributions that
  are actually sampled from, temperature and top-k/top-p included ([P5] section
  on exact verification).  p = softmax(z / T); with top-p, keep the smallest
  set of most probable tokens whose mass reaches top_p and renormalise
  ([P3] section 4.2, generation config `temperature` / `top_p`).
* Greedy: the target's best token per position ([P1] section 3.1 item 3,
  greedy matching; [P5] section on exact verification).
* Sampling from a weight vector: inverse CDF in index order (our reading of the
  unspecified `torch.multinomial` in [P4] section "数学保证：无损输出质量").

All arithmetic is float64 on the stored fp32 logits.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def _nucleus_order(p: np.ndarray) -> np.ndarray:
    """Token order by (probability descending, index ascending)."""
    return np.lexsort((np.arange(p.shape[-1]), -p))


def effective_distribution(z: np.ndarray, temperature: float, top_p: float = 1.0) -> np.ndarray:
    """TopP(softmax(z / T)) for one logits row, float64."""
    s = np.asarray(z, dtype=np.float64) / float(temperature)
    e = np.exp(s - s.max())
    p = e / e.sum()
    if top_p >= 1.0:
        return p
    order = _nucleus_order(p)
    csum = np.cumsum(p[order])
    keep = min(int(np.searchsorted(csum, top_p, side="left")) + 1, p.size)
    kept = np.zeros(p.size, dtype=bool)
    kept[order[:keep]] = True
    out = np.where(kept, p, 0.0)
    return out / out.sum()


def nucleus_margin(z: np.ndarray, temperature: float, top_p: float) -> float:
    """Distance of top_p from the cumulative masses on either side of the nucleus cut.

    Returns min(|cum_before - top_p|, |cum_including - top_p|) for the crossing
    token (inf when top-p is off); used to flag decisions that sit within the
    rounding band of the cut.
    """
    if top_p >= 1.0:
        return float("inf")
    s = np.asarray(z, dtype=np.float64) / float(temperature)
    e = np.exp(s - s.max())
    p = e / e.sum()
    order = _nucleus_order(p)
    csum = np.cumsum(p[order])
    keep = min(int(np.searchsorted(csum, top_p, side="left")) + 1, p.size)
    before = csum[keep - 2] if keep >= 2 else 0.0
    including = csum[keep - 1]
    return float(min(abs(before - top_p), abs(including - top_p)))


def argmax_first(z: np.ndarray) -> np.ndarray:
    """Index of the largest logit along the last axis, smallest index on ties.

    np.argmax returns the first occurrence of the maximum.
    """
    return np.argmax(np.asarray(z), axis=-1)


def inverse_cdf(w: np.ndarray, u: float) -> Tuple[int, float]:
    """Draw from unnormalised weights w with one uniform u in [0,1).

    y = min{k : u * W < C_k}, C = inclusive prefix sums in index order, W = C[-1];
    if rounding leaves no such k, the last k with w_k > 0.  Also returns the
    margin min(|u - C_{y-1}/W|, |u - C_y/W|) used to flag near-ties.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    W = c[-1]
    hits = np.nonzero(float(u) * W < c)[0]
    if hits.size:
        y = int(hits[0])
    else:
        y = int(np.nonzero(w > 0)[0][-1])
    lo = c[y - 1] / W if y >= 1 else 0.0
    hi = c[y] / W
    return y, float(min(abs(float(u) - lo), abs(float(u) - hi)))


def inverse_cdf_rows(w: np.ndarray, u: np.ndarray):
    """`inverse_cdf` applied to every row of w [..., V] with its own uniform u [...]."""
    w = np.asarray(w, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    c = np.cumsum(w, axis=-1)
    W = c[..., -1]
    hit = (u * W)[..., None] < c
    any_hit = hit.any(axis=-1)
    V = w.shape[-1]
    last_pos = V - 1 - np.argmax((w > 0)[..., ::-1], axis=-1)
    y = np.where(any_hit, np.argmax(hit, axis=-1), last_pos)
    hi = np.take_along_axis(c, y[..., None], axis=-1)[..., 0] / W
    lo = np.where(y >= 1, np.take_along_axis(c, np.maximum(y - 1, 0)[..., None], axis=-1)[..., 0] / W, 0.0)
    margin = np.minimum(np.abs(u - lo), np.abs(u - hi))
    return y, margin
