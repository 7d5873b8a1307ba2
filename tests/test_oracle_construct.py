"""Pins for the oracle's EAGLE-2 construction (expansion + rerank)."""
import os

import numpy as np
import pytest
import scipy.special

import oracle.construct as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# The hand case's rows (tests/golden/eagle2_hand_case.txt): (q, offset).
ROOT = ((0.5, 0.3, 0.2), 0.0)
ROUND2 = [((0.1, 0.7, 0.2), 1.0), ((0.9, 0.05, 0.05), 2.0)]
ROUND3 = [((0.8, 0.1, 0.1), -0.5), ((0.5, 0.25, 0.25), 0.7)]


def _row(q, c):
    return (np.log(np.asarray(q)) + c).astype(np.float32)


def _hand_lines():
    out = []
    for line in open(os.path.join(GOLDEN, "eagle2_hand_case.txt")):
        if line.strip() and not line.startswith("#"):
            f = [s.strip() for s in line.split("|")]
            out.append((int(f[0]), int(f[1]), [int(x) for x in f[2].split()],
                        [int(x) for x in f[3].split()]))
    return out


def _hand(rounds, m):
    rows = [[_row(*r) for r in ROUND2], [_row(*r) for r in ROUND3]][:rounds - 1]
    return C.eagle2_tree(_row(*ROOT), rows, 2, m)


@pytest.mark.parametrize("case", _hand_lines(), ids=lambda c: f"rounds{c[0]}_m{c[1]}")
def test_hand_case(case):
    rounds, m, parent, token = case
    p, t, _, _ = _hand(rounds, m)
    assert p.tolist() == parent
    assert t.tolist() == token


def test_hand_case_values_are_path_products():
    _, _, cands, fr = _hand(3, 7)
    want = [0.5, 0.3, 0.35, 0.10, 0.27, 0.015, 0.28, 0.035, 0.135, 0.0675]
    np.testing.assert_allclose(np.exp(cands.value), want, rtol=1e-6)
    assert fr == [[0, 1], [2, 4], [6, 8]]


def test_planted_mistakes_fail_the_hand_case(monkeypatch):
    """An edge-only value, or log q without the row's normaliser, changes
    the tree."""
    for name, bad in (("path_value", lambda parent, lq: lq),
                      ("log_softmax", lambda row: np.asarray(row, np.float64))):
        monkeypatch.setattr(C, name, bad)
        for rounds, m, parent, token in _hand_lines():
            if (rounds, m) != (3, 4):
                continue
            try:
                p, t, _, _ = _hand(rounds, m)
                assert (p.tolist(), t.tolist()) != (parent, token), name
            except ValueError:  # the kept set also lost ancestor closure
                pass
        monkeypatch.undo()


def _random(seed, V=40, k=4, rounds=4, m=20):
    rng = np.random.default_rng(seed)
    root = (rng.standard_normal(V) * 2).astype(np.float32)
    rows = [(rng.standard_normal((k, V)) * 2).astype(np.float32) for _ in range(rounds - 1)]
    return root, rows, C.eagle2_tree(root, rows, k, m)


@pytest.mark.parametrize("seed", range(6))
def test_values_match_library_softmax_products(seed):
    """Each candidate's value is the log of the product of softmax
    probabilities (scipy) of its tokens along the path, each under the row
    of the node it extends."""
    root, rows, (_, _, cands, fr) = _random(seed)
    row_of = {-1: root}
    for d, frontier in enumerate(fr[:-1]):
        for j, f in enumerate(frontier):
            row_of[f] = rows[d][j]
    for i, (v, x, par) in enumerate(zip(cands.value, cands.token, cands.parent)):
        prob, node, tok = 1.0, par, x
        while True:
            prob *= scipy.special.softmax(row_of[node].astype(np.float64))[tok]
            if node < 0:
                break
            node, tok = cands.parent[node], cands.token[node]
        assert abs(np.exp(v) - prob) <= 1e-12 * max(prob, 1e-300) + 1e-300, i


@pytest.mark.parametrize("seed", range(6))
def test_invariants(seed):
    """Topological parents, ancestor closure, the rerank cut and each
    frontier cut, children only under frontier nodes, siblings in
    descending draft logit."""
    k, m = 4, 20
    root, rows, (parent, token, cands, fr) = _random(seed, k=k, m=m)
    n = len(parent)
    assert n == 1 + m and parent[0] == -1
    assert all(0 <= parent[i] < i for i in range(1, n))
    v = np.asarray(cands.value)
    ids = np.arange(len(v))
    _, _, keep = C.rerank(cands, m)
    dropped = np.setdiff1d(ids, keep)
    assert v[keep].min() >= v[dropped].max()
    for c in keep:  # closed under ancestors
        assert cands.parent[c] < 0 or cands.parent[c] in keep
    assert (v[np.asarray(cands.parent)[np.asarray(cands.parent) >= 0]] >=
            v[np.asarray(cands.parent) >= 0]).all()
    start = 0
    for d, frontier in enumerate(fr):
        cnt = k if d == 0 else k * k
        rnd = ids[start:start + cnt]
        rest = np.setdiff1d(rnd, frontier)
        if len(rest):
            assert v[frontier].min() >= v[rest].max()
        assert [v[f] for f in frontier] == sorted([v[f] for f in frontier], reverse=True)
        start += cnt
    expanded = {p for p in cands.parent if p >= 0}
    assert expanded <= set(sum(fr[:-1], []))
    # siblings appear in descending logit of the row they were drawn from
    row_of = {-1: root}
    for d, frontier in enumerate(fr[:-1]):
        for j, f in enumerate(frontier):
            row_of[f] = rows[d][j]
    for f, row in row_of.items():
        kids = [i for i in ids if cands.parent[i] == f]
        lg = [row[cands.token[i]] for i in kids]
        assert lg == sorted(lg, reverse=True)


def test_k1_is_the_greedy_chain():
    """k = 1: a chain of each round's argmax token."""
    rng = np.random.default_rng(3)
    root = rng.standard_normal(50).astype(np.float32)
    rows = [rng.standard_normal((1, 50)).astype(np.float32) for _ in range(5)]
    parent, token, _, _ = C.eagle2_tree(root, rows, 1, 10)
    assert parent.tolist() == [-1, 0, 1, 2, 3, 4, 5]
    assert token.tolist() == [-1, int(np.argmax(root))] + [int(np.argmax(r[0])) for r in rows]


def test_m_at_least_all_candidates_keeps_everything():
    k, rounds = 3, 3
    root, rows, (parent, _, cands, _) = _random(9, V=30, k=k, rounds=rounds, m=1000)
    assert len(parent) == 1 + k + (rounds - 1) * k * k == 1 + len(cands.value)


def test_topk_children_lowest_id_on_ties():
    row = np.array([1.0, 3.0, 3.0, 0.5, 3.0], dtype=np.float32)
    assert C.topk_children(row, 4).tolist() == [1, 2, 4, 0]
