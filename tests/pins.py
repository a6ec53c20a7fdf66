"""Independent references used to pin the oracle.

Nothing here calls the oracle or the HIP path: each helper computes its value
another way (exhaustive enumeration, high-precision decimal arithmetic, or a
library routine) so that a mistake in the oracle shows up as a mismatch.
"""
from __future__ import annotations

import itertools
from decimal import Decimal, getcontext

import numpy as np

getcontext().prec = 60


def f32_round_decimal(d: Decimal) -> np.float32:
    """Correctly rounded (to nearest, ties to even) fp32 value of a Decimal."""
    f = np.float32(float(d))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Decimal(float(cand)) - d)
        if best is None or err < best[0] or (
                err == best[0] and (int(np.float32(cand).view(np.uint32)) & 1) == 0):
            best = (err, np.float32(cand))
    return best[1]


def sigmoid_decimal(l: float) -> Decimal:
    return Decimal(1) / (Decimal(1) + (-Decimal(float(l))).exp())


def sigmoid_f32_exact(l: float) -> np.float32:
    """fp32 rounding of the exact sigmoid (60 significant digits)."""
    return f32_round_decimal(sigmoid_decimal(l))


def brute_topk(keys, k, allowed=None):
    """Exhaustive top-k: the index set S (|S| = k) whose every key is >= every
    key outside it; among several such sets the lexicographically smallest
    sorted index tuple (i.e. lower index wins ties).  Returned as a sorted tuple."""
    idx = [i for i in range(len(keys)) if allowed is None or allowed[i]]
    best = None
    for S in itertools.combinations(idx, k):
        inside = [keys[i] for i in S]
        outside = [keys[i] for i in idx if i not in S]
        if outside and min(inside) < max(outside):
            continue
        if best is None or S < best:
            best = S
    return best


def ordered_by_key(ids, keys) -> bool:
    """True when ids are listed by key descending, equal keys by index ascending."""
    for a, b in zip(ids[:-1], ids[1:]):
        if keys[a] < keys[b]:
            return False
        if keys[a] == keys[b] and a > b:
            return False
    return True


def brute_group_score(kappa, members):
    """max over pairs of fl32(kappa_i + kappa_j): the largest two-element sum."""
    best = None
    for i, j in itertools.combinations(members, 2):
        s = np.float32(np.float32(kappa[i]) + np.float32(kappa[j]))
        if best is None or s > best:
            best = s
    return best
