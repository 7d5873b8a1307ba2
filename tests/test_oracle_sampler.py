"""Pins for the oracle's sampling walk and path selection."""
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.path import TwoAcceptedSiblings
from oracle.sampler import near_threshold
from workloads import random_tree, chain_tree, star_tree, gumbel_topk_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_softmax_T_matches_library():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(1000) * 3).astype(np.float32)
    for T in (0.25, 0.5, 1.0, 2.0):
        ref = scipy.special.softmax(x.astype(np.float64) / T)
        np.testing.assert_allclose(oracle.softmax_T(x, T), ref, rtol=1e-13, atol=0)


def _rand_dist(rng, V, zeros=0):
    w = rng.gamma(0.7, size=V)
    if zeros:
        w[rng.choice(V, zeros, replace=False)] = 0.0
    return w / w.sum()


@pytest.mark.parametrize("seed", range(8))
def test_exact_enumeration_law_equals_target(seed):
    """P6 (Proposition 1): the next emitted token after any reached node has
    law p_node exactly (<= 1e-12), for trees of depth <= 2, V <= 5, k <= 3."""
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 6))
    cache = {}

    def dist(kind, path):
        key = (kind, path)
        if key not in cache:
            cache[key] = _rand_dist(rng, V, zeros=int(rng.integers(0, 2)) if V > 2 else 0)
        return cache[key]

    k_by_depth = [int(rng.integers(1, 4)), int(rng.integers(0, 3)), 0]

    def slots(path):
        return k_by_depth[len(path)] if len(path) < 3 else 0

    laws = oracle.enumerate_node_laws(lambda pth: dist("p", pth), lambda pth: dist("q", pth), slots, V)
    assert abs(laws[()][0] - 1.0) < 1e-15
    for path, (reach, law) in laws.items():
        if reach < 1e-300:
            continue
        np.testing.assert_allclose(law / reach, dist("p", path), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_exact_enumeration_law_with_replacement_equals_target(seed):
    """Rule (b) (SpecInfer's MSS, MCSD Algorithm 1): with siblings drawn
    independently from q and the proposal kept at q, the next emitted token
    after any reached node has law p_node exactly, also with more siblings
    than tokens (repeats)."""
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(2, 5))
    cache = {}

    def dist(kind, path):
        key = (kind, path)
        if key not in cache:
            cache[key] = _rand_dist(rng, V, zeros=int(rng.integers(0, 2)) if V > 2 else 0)
        return cache[key]

    k_by_depth = [int(rng.integers(1, 5)), int(rng.integers(0, 3)), 0]
    laws = oracle.enumerate_node_laws(lambda pth: dist("p", pth), lambda pth: dist("q", pth),
                                      lambda pth: k_by_depth[len(pth)] if len(pth) < 3 else 0, V,
                                      rule="with")
    assert abs(laws[()][0] - 1.0) < 1e-15
    for path, (reach, law) in laws.items():
        if reach < 1e-300:
            continue
        np.testing.assert_allclose(law / reach, dist("p", path), rtol=0, atol=1e-12)


@pytest.mark.parametrize("rule,draws", [("without", "with"), ("with", "without"),
                                        ("without", "topk"), ("with", "topk")])
def test_mismatched_draws_and_rules_are_biased(rule, draws):
    """Each rule is exact only for its own draw scheme; deterministic top-k
    siblings ([TreeSpark §5.4, Table 9]) are biased under either rule."""
    rng = np.random.default_rng(7)
    p, q = _rand_dist(rng, 4), _rand_dist(rng, 4)
    laws = oracle.enumerate_node_laws(lambda _: p, lambda _: q, lambda pth: 2 if not pth else 0, 4,
                                      rule=rule, draws=draws)
    reach, law = laws[()]
    assert abs(reach - 1.0) < 1e-12
    assert 0.5 * np.abs(law - p).sum() > 1e-3


@pytest.mark.parametrize("rule", ["without", "with"])
def test_topk_siblings_with_q_equal_p_emit_only_the_argmax(rule):
    """[TreeSpark §5.4]: when q is close to p the first top-k candidate is
    almost always accepted. At q = p its ratio is 1, so the emitted token is
    the argmax with probability 1 (TV distance 1 - max p), while sampled
    siblings keep the law p."""
    p = np.array([0.344, 0.25, 0.2, 0.126, 0.08])
    laws = oracle.enumerate_node_laws(lambda _: p, lambda _: p, lambda pth: 3 if not pth else 0, 5,
                                      rule=rule, draws="topk")
    reach, law = laws[()]
    np.testing.assert_allclose(law, np.eye(5)[0], atol=1e-15)
    assert abs(0.5 * np.abs(law - p).sum() - (1 - p.max())) < 1e-12
    fair = oracle.enumerate_node_laws(lambda _: p, lambda _: p, lambda pth: 3 if not pth else 0, 5,
                                      rule=rule)[()][1]
    np.testing.assert_allclose(fair, p, atol=1e-12)


def test_enumeration_detects_a_planted_mistake(monkeypatch):
    """The enumeration pin fails when the residual forgets to subtract q."""
    import oracle.enumerate as en
    rng = np.random.default_rng(1)
    p, q = _rand_dist(rng, 4), _rand_dist(rng, 4)

    def bad_residual(pres, qj):
        return pres, pres.sum(), False
    monkeypatch.setattr(en, "residual_update", bad_residual)
    laws = en.enumerate_node_laws(lambda _: p, lambda _: q, lambda pth: 2 if not pth else 0, 4)
    reach, law = laws[()]
    assert np.abs(law / reach - p).max() > 1e-3


def _parse_hand_cases(name="sampler_hand_cases.txt"):
    cases = []
    for line in open(os.path.join(GOLDEN, name)):
        if not line.strip() or line.startswith("#"):
            continue
        f = [s.strip() for s in line.split("|")]
        vec = lambda s, t=float: [t(x) for x in s.split()]
        cases.append(dict(name=f[0], p=vec(f[1]), q=vec(f[2]), tokens=vec(f[3], int),
                          u_acc=vec(f[4]), u_res=float(f[5]), flags=vec(f[6], int),
                          nt=int(f[7])))
    return cases


_HAND = ([dict(c, replacement=False) for c in _parse_hand_cases()]
         + [dict(c, replacement=True) for c in _parse_hand_cases("sampler_hand_cases_with_replacement.txt")])


@pytest.mark.parametrize("case", _HAND, ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    k = len(case["tokens"])
    parent = star_tree(k + 1)
    V = len(case["p"])
    t = np.zeros((k + 1, V), dtype=np.float32)
    d = np.zeros((k + 1, V), dtype=np.float32)
    with np.errstate(divide="ignore"):
        t[0] = np.log(np.asarray(case["p"]))
        d[0] = np.log(np.asarray(case["q"]))
    tokens = np.asarray([0] + case["tokens"], dtype=np.int32)
    u = np.zeros((k + 1, 2), dtype=np.float32)
    u[1:, 0] = case["u_acc"]
    u[0, 1] = case["u_res"]
    u[1:, 1] = 0.5
    flag, nt, _ = oracle.walk_request(t, d, tokens, parent, 1.0, u, replacement=case["replacement"])
    assert list(flag[1:]) == case["flags"]
    assert nt[0] == case["nt"]


def _run_chain(rng, p, q, k, n):
    V = len(p)
    parent = chain_tree(k + 1)
    t = np.tile(np.log(p).astype(np.float32), (k + 1, 1))
    d = np.tile(np.log(q).astype(np.float32), (k + 1, 1))
    lens = []
    for _ in range(n):
        toks = np.concatenate([[0], rng.choice(V, size=k, p=q)]).astype(np.int32)
        u = rng.random((k + 1, 2), dtype=np.float32)
        flag, nt, _ = oracle.walk_request(t, d, toks, parent, 1.0, u)
        path, out, _ = oracle.accept_path_request(parent, toks, flag, nt, 0)
        lens.append(len(out))
    return np.asarray(lens)


def test_chain_expected_length_closed_form():
    """P7: a chain is standard speculative sampling; with constant per-node
    alpha = sum min(p, q), E[emitted] = (1 - alpha^(k+1)) / (1 - alpha)
    (survey page, Systems: the Leviathan chain formula)."""
    rng = np.random.default_rng(42)
    p = np.array([0.4, 0.25, 0.15, 0.1, 0.06, 0.04])
    q = np.array([0.2, 0.3, 0.1, 0.2, 0.1, 0.1])
    alpha = np.minimum(p, q).sum()
    k, n = 4, 6000
    lens = _run_chain(rng, p, q, k, n)
    expect = (1 - alpha ** (k + 1)) / (1 - alpha)
    ci = 2.576 * lens.std(ddof=1) / np.sqrt(n)
    assert abs(lens.mean() - expect) < ci, (lens.mean(), expect, ci)


def _first_token_tv(rng, p, q, k, n, deterministic=False):
    V = len(p)
    parent = star_tree(k + 1)
    t = np.tile(np.log(p).astype(np.float32), (k + 1, 1))
    d = np.tile(np.log(q).astype(np.float32), (k + 1, 1))
    counts = np.zeros(V)
    for _ in range(n):
        if deterministic:
            toks = np.argsort(-q, kind="stable")[:k]
        else:
            toks = gumbel_topk_tokens(rng, d[0], k, 1.0)
        toks = np.concatenate([[0], toks]).astype(np.int32)
        u = rng.random((k + 1, 2), dtype=np.float32)
        flag, nt, _ = oracle.walk_request(t, d, toks, parent, 1.0, u)
        _, out, _ = oracle.accept_path_request(parent, toks, flag, nt, 0)
        counts[out[0]] += 1
    return 0.5 * np.abs(counts / n - p).sum()


def _direct_tv_quantile(rng, p, n, reps=300, qtile=99):
    tvs = [0.5 * np.abs(rng.multinomial(n, p) / n - p).sum() for _ in range(reps)]
    return np.percentile(tvs, qtile)


def test_monte_carlo_tv_and_negative_control():
    """P10: the walk's first-token TV is within the 99th percentile of direct
    sampling's TV at equal n (TreeSpark §5.4, Table 9 method). P11: the
    deterministic top-k control must fail the same bound."""
    rng = np.random.default_rng(7)
    V, k, n = 8, 3, 4000
    logits = rng.standard_normal(V) * 0.8
    p = scipy.special.softmax(logits)
    q = scipy.special.softmax(logits + rng.standard_normal(V) * 0.3)
    bound = _direct_tv_quantile(rng, p, n)
    tv = _first_token_tv(rng, p, q, k, n)
    assert tv <= bound, (tv, bound)
    tv_ctrl = _first_token_tv(rng, p, q, k, n, deterministic=True)
    assert tv_ctrl > bound, (tv_ctrl, bound)


def test_q_equals_p_accepts_first_child():
    """P8a: with q = p every ratio is 1 (up to rounding) and u < 1 accepts."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        V = 7
        logits = rng.standard_normal(V).astype(np.float32)
        parent = star_tree(4)
        t = np.tile(logits, (4, 1))
        toks = np.concatenate([[0], gumbel_topk_tokens(rng, logits, 3, 1.0)]).astype(np.int32)
        u = rng.random((4, 2), dtype=np.float32) * np.float32(0.999)
        flag, nt, _ = oracle.walk_request(t, t.copy(), toks, parent, 1.0, u)
        assert flag[1] == 1 and flag[2] == 0 and flag[3] == 0


def test_disjoint_supports_reject_all_and_draw_from_p():
    """P8b: disjoint supports -> every child rejected; the stop draw has law p."""
    p = np.array([0.5, 0.3, 0.2, 0, 0, 0])
    q = np.array([0, 0, 0, 0.2, 0.3, 0.5])
    laws = oracle.enumerate_node_laws(lambda _: p, lambda _: q, lambda pth: 3 if not pth else 0, 6)
    reach, law = laws[()]
    np.testing.assert_allclose(law, p, atol=1e-15)
    assert set(laws) == {()}  # no child is ever accepted
    rng = np.random.default_rng(0)
    with np.errstate(divide="ignore"):
        t = np.tile(np.log(p).astype(np.float32), (4, 1))
        d = np.tile(np.log(q).astype(np.float32), (4, 1))
    for _ in range(20):
        toks = np.concatenate([[0], rng.permutation([3, 4, 5])]).astype(np.int32)
        u = rng.random((4, 2), dtype=np.float32)
        flag, nt, _ = oracle.walk_request(t, d, toks, star_tree(4), 1.0, u)
        assert flag[1:].sum() == 0 and nt[0] in (0, 1, 2)


def test_greedy_closed_form_path():
    """P8c: at T = 0 the path follows exact matches with the target argmax
    (TreeSpark §3.2 step 3, §5.1: greedy outputs are identical to target-only
    greedy decoding)."""
    parent = np.array([-1, 0, 0, 1, 1, 2, 3, 3])
    tokens = np.array([0, 4, 9, 2, 6, 1, 3, 8], dtype=np.int32)
    V = 10
    t = np.zeros((8, V), dtype=np.float32)
    want = {0: 9, 2: 1, 5: 7, 1: 6, 3: 3, 4: 0, 6: 5, 7: 2}  # argmax of each row
    for i, a in want.items():
        t[i, a] = 5.0
    flag, nt, _ = oracle.greedy_request(t, tokens, parent)
    np.testing.assert_array_equal(nt, [want[i] for i in range(8)])
    # root argmax 9 -> node 2; node 2's argmax 1 -> node 5; node 5's argmax 7 -> none
    path, out, keep = oracle.accept_path_request(parent, tokens, flag, nt, 100)
    assert path == [0, 2, 5] and out == [9, 1, 7] and keep == [100, 102, 105]


def test_greedy_walk_hand_case():
    """The T = 0 form that visits only the walk's nodes, on the tree of the
    case above: nodes 0, 2 and 5 are visited, so only their children (1, 2;
    5; none) are tested and only the visited rows carry a next token. The
    every-node form also flags 4 and 6, whose parents the walk never
    reaches; the accepted path is the same."""
    parent = np.array([-1, 0, 0, 1, 1, 2, 3, 3])
    tokens = np.array([0, 4, 9, 2, 6, 1, 3, 8], dtype=np.int32)
    t = np.zeros((8, 10), dtype=np.float32)
    for i, a in {0: 9, 2: 1, 5: 7, 1: 6, 3: 3, 4: 0, 6: 5, 7: 2}.items():
        t[i, a] = 5.0
    flag, nt, _ = oracle.greedy_walk_request(t, tokens, parent)
    np.testing.assert_array_equal(flag, [1, 0, 1, 0, 0, 1, 0, 0])
    np.testing.assert_array_equal(nt, [9, -1, 1, -1, -1, 7, -1, -1])
    ef, ent, _ = oracle.greedy_request(t, tokens, parent)
    np.testing.assert_array_equal(ef, [1, 0, 1, 0, 1, 1, 1, 0])
    assert oracle.accept_path_request(parent, tokens, flag, nt, 0) == \
        oracle.accept_path_request(parent, tokens, ef, ent, 0)


@pytest.mark.parametrize("planted", ["last_child_skipped", "rows_shifted"])
def test_greedy_walk_hand_case_catches_planted_mistakes(monkeypatch, planted):
    """A child scan that stops one short, or the rows read one node off (the
    child's row instead of the visited node's), fails the hand case."""
    import oracle.sampler as smp
    if planted == "last_child_skipped":
        real = smp.children
        monkeypatch.setattr(smp, "children", lambda par: [c[:-1] for c in real(par)])
    else:
        real = smp.greedy_walk_request
        monkeypatch.setattr(oracle, "greedy_walk_request",
                            lambda t, tok, par: real(np.roll(t, -1, axis=0), tok, par))
    with pytest.raises(AssertionError):
        test_greedy_walk_hand_case()


def _random_greedy_case(rng, n, V):
    parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)])
    t = rng.integers(-3, 4, size=(n, V)).astype(np.float32)  # integer logits: ties
    tokens = rng.integers(0, V, size=n).astype(np.int32)
    # plant matches so that walks go deep: a child often carries its parent's argmax
    for i in range(1, n):
        if rng.random() < 0.6:
            tokens[i] = int(np.argmax(t[parent[i]]))
    return parent, tokens, t


@pytest.mark.parametrize("seed", range(6))
def test_greedy_walk_agrees_with_every_node_form(seed):
    """Over random trees (integer logits with ties, planted matches, repeated
    sibling tokens allowed): the walk-only form gives the every-node form's
    accepted path, or the same two-flagged-siblings error; it flags exactly
    the children of the visited nodes, each as the every-node form does, and
    gives the every-node next token at the visited nodes only."""
    rng = np.random.default_rng(100 + seed)
    deep = 0
    for _ in range(60):
        n, V = int(rng.integers(1, 40)), int(rng.integers(2, 9))
        parent, tokens, t = _random_greedy_case(rng, n, V)
        wf, wnt, _ = oracle.greedy_walk_request(t, tokens, parent)
        ef, ent, _ = oracle.greedy_request(t, tokens, parent)
        try:
            want = oracle.accept_path_request(parent, tokens, ef, ent, 0)
        except TwoAcceptedSiblings:
            with pytest.raises(TwoAcceptedSiblings):
                oracle.accept_path_request(parent, tokens, wf, wnt, 0)
            continue
        got = oracle.accept_path_request(parent, tokens, wf, wnt, 0)
        assert got == want
        path = got[0]
        deep = max(deep, len(path))
        visited = set(path)
        for i in range(n):
            if i == 0:
                assert wf[i] == 1
            elif parent[i] in visited:
                assert wf[i] == ef[i]
            else:
                assert wf[i] == 0
            assert wnt[i] == (ent[i] if i in visited else -1)
    assert deep >= 4  # the planted matches made some walks deep


def test_alignment_probe():
    """Row i holds the logits of the token after node i (TreeSpark §3.1): a
    target row one-hot on the token that only one child carries makes that
    child accepted; reading the child's row instead does not."""
    V = 16
    parent = np.array([-1, 0, 0, 1])
    tokens = np.array([0, 5, 7, 3], dtype=np.int32)
    t = np.full((4, V), -30.0, dtype=np.float32)
    t[0, 7] = 30.0          # after the root the target wants token 7 (node 2)
    t[1:, 11] = 30.0
    d = np.zeros((4, V), dtype=np.float32)
    u = np.full((4, 2), 0.5, dtype=np.float32)
    flag, nt, _ = oracle.walk_request(t, d, tokens, parent, 1.0, u)
    assert flag[1] == 0 and flag[2] == 1
    shifted = np.roll(t, -1, axis=0)   # the off-by-one reading
    flag2, _, _ = oracle.walk_request(shifted, d, tokens, parent, 1.0, u)
    assert flag2[2] == 0


def _closed_form_stage_checks(p, q, toks, u):
    """P12 (a cross-check of the GPU's scalar form, not of the oracle): with
    p_j(y) = max(p - a_j q, 0)/B_j, a_1 = 0, B_1 = 1, a_{j+1} = a_j + B_j/S_j,
    B_{j+1} = sum max(p - a_{j+1} q, 0), S_j = 1 - sum_{i<j} q(x_i), the
    ratios and final residual equal the vector recursion's."""
    pres, drawn = p, []
    a, B, S = 0.0, 1.0, 1.0
    for x, uj in zip(toks, u):
        qj = oracle.proposal_without(q, drawn)
        r_vec = oracle.acceptance_ratio(pres[x], qj[x])
        r_cf = (max(p[x] - a * q[x], 0.0) / B) / (q[x] / S)
        assert abs(r_vec - r_cf) <= 1e-12 * max(1.0, r_vec)
        if uj < r_vec:
            return
        pres, _, _ = oracle.residual_update(pres, qj)
        a = a + B / S
        B = np.maximum(p - a * q, 0.0).sum()
        S = S - q[x]
        np.testing.assert_allclose(pres, np.maximum(p - a * q, 0.0) / B, atol=1e-13)
        drawn.append(x)


@pytest.mark.parametrize("seed", range(20))
def test_closed_form_identity(seed):
    rng = np.random.default_rng(seed)
    V = 12
    p, q = _rand_dist(rng, V), _rand_dist(rng, V)
    toks = rng.choice(V, size=6, replace=False, p=q)
    _closed_form_stage_checks(p, q, toks, np.ones(6))


@pytest.mark.parametrize("seed", range(10))
def test_walk_invariants(seed):
    """P9: exactly one accepted root path; emitted length = accepted depth + 1;
    next_token is set exactly at the stop node (T > 0) or everywhere (T = 0)."""
    rng = np.random.default_rng(seed)
    from workloads import make_sampler_inputs
    trees = [random_tree(rng, int(rng.integers(1, 30)), depth_cap=5) for _ in range(6)]
    temps = [0.0, 0.5, 1.0, 1.0, 2.0, 0.0]
    inp = make_sampler_inputs(rng, rng, rng, trees, 64, temps)
    flags, nts, logs = oracle.tree_spec_sample(inp)
    for r, parent in enumerate(trees):
        a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
        f, nt = flags[a:b], nts[a:b]
        path, out, keep = oracle.accept_path_request(parent, inp.tokens[a:b], f, nt, 10)
        d = oracle.depths(parent)
        assert len(out) == d[path[-1]] + 1
        if temps[r] > 0:
            on_path = set(path)
            assert all(f[i] == 0 for i in range(1, len(f)) if i not in on_path)
            assert [i for i in range(len(nt)) if nt[i] >= 0] == [path[-1]]
        else:
            assert (nt >= 0).all()


def test_inverse_cdf_closed_forms():
    """Uniform residual: y = floor(u V); one-hot: always that token; zero-mass
    tokens are never drawn."""
    V = 10
    uni = np.full(V, 0.1)
    for u in np.linspace(0, 0.999, 37):
        y, _ = oracle.inverse_cdf(uni, u)
        assert y == int(np.floor(np.float64(u) * V + 1e-12)) or abs(u * V - round(u * V)) < 1e-9
    oh = np.zeros(V)
    oh[6] = 1.0
    assert all(oracle.inverse_cdf(oh, u)[0] == 6 for u in (0.0, 0.3, 0.9999))
    sp = np.array([0, 0.5, 0, 0, 0.5, 0, 0, 0, 0, 0])
    assert {oracle.inverse_cdf(sp, u)[0] for u in np.linspace(0, 0.999, 50)} == {1, 4}


def test_two_accepted_siblings_is_an_error():
    from oracle.path import TwoAcceptedSiblings
    parent = np.array([-1, 0, 0])
    with pytest.raises(TwoAcceptedSiblings):
        oracle.accept_path_request(parent, [0, 1, 2], [1, 1, 1], [-1, -1, -1], 0)


def test_batched_accept_path_layout():
    parent = np.array([-1, 0, 1, -1, 0, 0])
    node_indptr = np.array([0, 3, 6])
    tokens = np.array([0, 11, 12, 0, 21, 22])
    flags = np.array([1, 1, 1, 1, 0, 1], dtype=np.int8)
    nts = np.array([-1, -1, 99, 77, -1, 88])
    pn, ot, ol, kk = oracle.tree_accept_path(node_indptr, parent, tokens, flags, nts, [5, 9], 3)
    np.testing.assert_array_equal(ol, [3, 2])
    np.testing.assert_array_equal(pn[0], [0, 1, 2, -1])
    np.testing.assert_array_equal(ot[0], [11, 12, 99, -1])
    np.testing.assert_array_equal(kk[1], [9, 11, -1, -1])
    np.testing.assert_array_equal(ot[1], [22, 88, -1, -1])
