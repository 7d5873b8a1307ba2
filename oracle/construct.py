"""Dynamic draft-tree construction by expansion and rerank (EAGLE-2), in fp64.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module.

Source: [survey, Timeline] EAGLE-2 grows the draft tree by expanding the
top-k nodes by path-product value and reranking to keep the top-m nodes;
[survey, Taxonomy / construction policy] the signal is the cumulative draft
probability along the root path.

Readings of points the pages leave open:
  * a node's value is the sum of log q along its root path (the log of the
    path product), q = softmax of the node's draft row (temperature 1);
  * one expansion round gives every frontier node its k most probable
    children (the k largest draft logits, lowest token id first on ties),
    in that order;
  * candidates are numbered in generation order (round, then frontier slot,
    then child rank); the next frontier is the k best new candidates by
    value, best first (ties: lower id); frontier slot j of round d reads
    draft row j of that round (the drafter's output for that node);
  * the rerank keeps the m best of all candidates by value (ties: lower id).
    A child's value never exceeds its parent's and its id is larger, so the
    kept set is closed under ancestors;
  * the output tree lists the root, then the kept candidates in ascending id
    (topological, siblings in draw order), with request-local parents.
"""
import numpy as np


def log_softmax(row):
    """log softmax of one draft row in fp64 (max subtracted)."""
    x = np.asarray(row, dtype=np.float32).astype(np.float64)
    m = x.max()
    return x - (m + np.log(np.exp(x - m).sum()))


def topk_children(row, k):
    """The k largest draft logits of a row, largest first, lower id on ties."""
    x = np.asarray(row, dtype=np.float32)
    order = np.lexsort((np.arange(x.shape[0]), -x.astype(np.float64)))
    return order[:k].astype(np.int64)


def best(values, ids, n):
    """Positions of the n best (value descending, id ascending)."""
    order = np.lexsort((np.asarray(ids), -np.asarray(values, dtype=np.float64)))
    return order[:n]


def path_value(parent_value, child_logq):
    """Log path product: the parent's value plus the edge's log q."""
    return parent_value + child_logq


class Candidates:
    """Per-request candidate store in generation order."""

    def __init__(self):
        self.value, self.token, self.parent = [], [], []

    def add(self, value, token, parent):
        self.value.append(float(value))
        self.token.append(int(token))
        self.parent.append(int(parent))
        return len(self.value) - 1


def expand_round(cands, frontier, rows, k):
    """One round: frontier = candidate ids (-1 for the root), rows = their
    draft logit rows. Returns (new candidate ids, next frontier ids)."""
    new = []
    for f, row in zip(frontier, rows):
        base = 0.0 if f < 0 else cands.value[f]
        lq = log_softmax(row)
        for x in topk_children(row, k):
            new.append(cands.add(path_value(base, lq[x]), x, f))
    vals = [cands.value[i] for i in new]
    nxt = [new[j] for j in best(vals, new, k)]
    return new, nxt


def rerank(cands, m):
    """Root + the m best candidates in ascending id: (parent[], token[]),
    parent request-local (-1 at the root), token -1 at the root."""
    ids = np.arange(len(cands.value))
    keep = np.sort(ids[best(cands.value, ids, min(m, len(ids)))])
    pos = {-1: 0}
    for j, c in enumerate(keep):
        pos[int(c)] = j + 1
    if any(cands.parent[c] not in pos for c in keep):
        raise ValueError("kept set is not closed under ancestors")
    parent = [-1] + [pos[cands.parent[c]] for c in keep]
    token = [-1] + [cands.token[c] for c in keep]
    return np.asarray(parent, np.int32), np.asarray(token, np.int32), keep


def eagle2_tree(root_row, round_rows, k, m):
    """root_row [V]; round_rows[d] [k][V] for rounds d = 2..D (the drafter's
    rows for the frontier slots of that round). Returns (parent, token,
    candidates, frontiers) where frontiers[d] lists the frontier ids chosen
    after round d+1."""
    cands = Candidates()
    _, frontier = expand_round(cands, [-1], [root_row], k)
    frontiers = [frontier]
    for rows in round_rows:
        _, frontier = expand_round(cands, frontier, list(rows)[:len(frontier)], k)
        frontiers.append(frontier)
    parent, token, _ = rerank(cands, m)
    return parent, token, cands, frontiers


def near_gap(gap, eps):
    """A decision gap that rounding could flip: positive and below eps. An
    exact tie (gap 0: siblings with equal logits, identical arithmetic on any
    side) is broken by id the same way everywhere and does not count."""
    return 0.0 < float(gap) < eps


def order_gaps(vals, n):
    """Gaps between consecutive values among the n+1 best (descending): the
    order of the n best and the cut below them."""
    s = np.sort(np.asarray(vals, dtype=np.float64))[::-1][:n + 1]
    return s[:-1] - s[1:]


def cut_gap(vals, n):
    """The gap at the cut below the n best ([] when there are at most n)."""
    s = np.sort(np.asarray(vals, dtype=np.float64))[::-1]
    return s[n - 1:n] - s[n:n + 1] if len(s) > n else s[:0]


def round_ranges(k, rounds):
    """(start, count) of the candidate ids each round created: k for the
    root round, k * k for every later round."""
    out, start = [], 0
    for d in range(rounds):
        count = k if d == 0 else k * k
        out.append((start, count))
        start += count
    return out


def near_ties(cands, frontiers, k, m, eps):
    """True when a decision lies within eps of going the other way: the order
    of a round's k best values (the frontier's slot order decides which draft
    row each slot reads next) and its cut, or the rerank cut."""
    v = np.asarray(cands.value)
    for start, count in round_ranges(k, len(frontiers)):
        if any(near_gap(g, eps) for g in order_gaps(v[start:start + count], k)):
            return True
    return any(near_gap(g, eps) for g in cut_gap(v, m))
