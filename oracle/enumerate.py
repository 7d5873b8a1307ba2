"""Exact law of the walk's emitted tokens on tiny vocabularies.

[TreeSpark §3.3, Proposition 1]: for any node, any number of siblings and any
shaping policy, the walk emits tokens distributed exactly as the target p,
provided siblings are drawn from the stage proposals and never reordered by
value. This enumerator integrates the walk exactly: every sibling draw (from
the oracle's own stage proposal), every accept/reject outcome (probability
min(1, ratio) over u ~ U[0,1)) and every correction draw (the residual). It
uses the oracle's proposal_without / proposal_with, acceptance_ratio and
residual_update, so agreement with p pins those functions.

The sibling draw scheme and the verification rule are separate arguments, so
the mismatched pairs and deterministic top-k siblings ([TreeSpark §5.4,
Table 9]: the top-k control is biased) can be integrated as well:
  draws "without": stage j draws from q without the tokens drawn so far;
  draws "with":    every stage draws from q (independent draws);
  draws "topk":    stage j takes the j-th most probable token of q (lowest id
                   on ties) with probability 1;
  rule "without" / "with": rules (c) / (b) of [survey, Taxonomy].
"""
from collections import defaultdict

import numpy as np

from .sampler import proposal_without, proposal_with, acceptance_ratio, residual_update


def enumerate_node_laws(target, draft, slots, vocab, rule="without", draws=None):
    """target(path) / draft(path): probability vectors at the node reached by
    the token path (a tuple); slots(path): number of child slots there;
    draws defaults to the scheme the rule is made for.

    Returns {path: (P(walk reaches path), law of the next emitted token)} where
    the law is unnormalised (it sums to P(reach))."""
    reach = defaultdict(float)
    law = defaultdict(lambda: np.zeros(vocab))

    draws = rule if draws is None else draws
    assert rule in ("without", "with") and draws in ("without", "with", "topk")

    def visit(path, prob):
        reach[path] += prob
        p = np.asarray(target(path), dtype=np.float64)
        q = np.asarray(draft(path), dtype=np.float64)
        k = int(slots(path))
        if draws != "with":  # distinct siblings: at most the support of q
            k = min(k, int((q > 0).sum()))
        stage(path, q, p, [], 0, k, prob)

    def draw_law(q, drawn):
        if draws == "with":
            return q
        if draws == "without":
            return proposal_without(q, drawn)
        order = np.lexsort((np.arange(vocab), -q))  # descending q, lowest id first
        one = np.zeros(vocab)
        one[order[len(drawn)]] = 1.0
        return one

    def stage(path, q, pres, drawn, j, k, prob):
        if j == k:
            law[path] += prob * pres / pres.sum()
            return
        qj = proposal_with(q, drawn) if rule == "with" else proposal_without(q, drawn)
        dj = draw_law(q, drawn)
        for x in range(vocab):
            if dj[x] <= 0:
                continue
            px = prob * dj[x]
            a = min(1.0, acceptance_ratio(pres[x], qj[x]))
            if a > 0:
                law[path][x] += px * a
                visit(path + (x,), px * a)
            if a < 1:
                new, _, _ = residual_update(pres, qj)
                stage(path, q, new, drawn + [x], j + 1, k, px * (1 - a))

    visit((), 1.0)
    return {pth: (reach[pth], law[pth]) for pth in reach}
