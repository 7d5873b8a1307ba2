"""Exact law of the walk's emitted tokens on tiny vocabularies.

[TreeSpark §3.3, Proposition 1]: for any node, any number of siblings and any
shaping policy, the walk emits tokens distributed exactly as the target p,
provided siblings are drawn from the stage proposals and never reordered by
value. This enumerator integrates the walk exactly: every sibling draw (from
the oracle's own stage proposal), every accept/reject outcome (probability
min(1, ratio) over u ~ U[0,1)) and every correction draw (the residual). It
uses the oracle's proposal_without, acceptance_ratio and residual_update, so
agreement with p pins those functions.
"""
from collections import defaultdict

import numpy as np

from .sampler import proposal_without, acceptance_ratio, residual_update


def enumerate_node_laws(target, draft, slots, vocab):
    """target(path) / draft(path): probability vectors at the node reached by
    the token path (a tuple); slots(path): number of child slots there.

    Returns {path: (P(walk reaches path), law of the next emitted token)} where
    the law is unnormalised (it sums to P(reach))."""
    reach = defaultdict(float)
    law = defaultdict(lambda: np.zeros(vocab))

    def visit(path, prob):
        reach[path] += prob
        p = np.asarray(target(path), dtype=np.float64)
        q = np.asarray(draft(path), dtype=np.float64)
        k = min(int(slots(path)), int((q > 0).sum()))
        stage(path, q, p, [], 0, k, prob)

    def stage(path, q, pres, drawn, j, k, prob):
        if j == k:
            law[path] += prob * pres / pres.sum()
            return
        qj = proposal_without(q, drawn)
        for x in range(vocab):
            if qj[x] <= 0:
                continue
            px = prob * qj[x]
            a = min(1.0, acceptance_ratio(pres[x], qj[x]))
            if a > 0:
                law[path][x] += px * a
                visit(path + (x,), px * a)
            if a < 1:
                new, _, _ = residual_update(pres, qj)
                stage(path, q, new, drawn + [x], j + 1, k, px * (1 - a))

    visit((), 1.0)
    return {pth: (reach[pth], law[pth]) for pth in reach}
