"""Pure-Python brute-force definitions for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring). These functions pin the
C oracle without sharing its method: the top-k here is the O(N^2) rank
definition with no sort at all, and the attention helpers are closed forms.
"""
from __future__ import annotations

import math


def rank_select(values, k):
    """Top-k by rank, no sorting. rank_j counts the entries that come before j
    in the order (value desc, index asc): those strictly greater, plus the
    equal ones with a smaller index. Position j is selected iff rank_j < k.
    Returns the selected indices ordered by rank."""
    n = len(values)
    ranks = []
    for j in range(n):
        r = 0
        for i in range(n):
            if values[i] > values[j] or (values[i] == values[j] and i < j):
                r += 1
        ranks.append(r)
    chosen = [j for j in range(n) if ranks[j] < k]
    return sorted(chosen, key=lambda j: ranks[j])


def softmax_weights_two_rows(z1, z2):
    """Softmax over two logits written as the logistic function of their gap."""
    a = 1.0 / (1.0 + math.exp(-(z1 - z2)))
    return a, 1.0 - a
