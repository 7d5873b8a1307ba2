"""Pins for the oracle's TreeSpark construction (best-first by calibrated
path survival with the theta stop; TreeSpark §3.2, §3.4, §3.5).

* Brute force at T = 0: the keys fall along every path (p_hat < 1), so a
  best-first search with cap N and stop theta must return exactly the N best
  token sequences by sum of log p_hat whose key is at least log theta, among
  sequences whose every token lies within the top K of its parent's
  conditional. The enumeration scores every sequence of a tiny vocabulary
  directly, with no heap.
* The small-temperature limit: at T -> 0 the draws follow the logit order, so
  the sampled construction equals the greedy one.
* A hand case at T > 0 on three tokens: the admissible pre-draw bound admits a
  slot before its value is seen, and the calibrator reads q0, not q_T.
Planted mistakes in each must be caught.
"""
import itertools
import math

import numpy as np
import pytest

import oracle.treespark as TS
from workloads.bf16 import f32_to_bf16_bits


def _inputs(seed, V=4, r=3, depths=3, sigma=1.0):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, sigma, (depths, V)).astype(np.float32)
    W1 = f32_to_bf16_bits(rng.normal(0, 0.7, (V, r)).astype(np.float32))
    W2 = f32_to_bf16_bits(rng.normal(0, 0.7, (V, r)).astype(np.float32))
    return U, W1, W2


def _widen(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _paths(res):
    """Token sequence (root excluded) of every non-root node."""
    par, tok = res["parent"], res["token"]
    out = []
    for i in range(1, len(par)):
        seq, v = [], i
        while v > 0:
            seq.append(int(tok[v]))
            v = int(par[v])
        out.append(tuple(reversed(seq)))
    return out


def _brute(U, W1, W2, anchor, theta, N, K, a, b):
    """Every token sequence up to the depth cap, scored on its own: key =
    sum over its edges of log sigma(a logit(q0) + b), q0 = softmax of the
    parent's conditional logits U[d-1] + B(parent token, .) with B the full
    V x V table W1 W2^T. Sequences using a token outside the top K of its
    conditional are not reachable."""
    W1, W2 = _widen(W1), _widen(W2)
    Btab = W1 @ W2.T                                   # B[x, v] for every pair
    depths, V = U.shape
    scored = []
    for d in range(1, depths + 1):
        for seq in itertools.product(range(V), repeat=d):
            key, prev, ok = 0.0, anchor, True
            for i, x in enumerate(seq):
                l = U[i].astype(np.float64) + Btab[prev]
                rank = sorted(range(V), key=lambda y: (-l[y], y)).index(x)
                if rank >= K:
                    ok = False
                    break
                q = math.exp(l[x]) / sum(math.exp(t) for t in l)
                key += -math.log1p(math.exp(-(a * math.log(q / (1 - q)) + b)))
                prev = x
            if ok:
                scored.append((key, seq))
    scored.sort(key=lambda t: -t[0])
    lt = math.log(theta) if theta > 0 else -math.inf
    return [s for k, s in scored if k >= lt][:N], scored


CASES = [  # seed, V, depths, N, K, theta, a, b
    (0, 4, 3, 5, 4, 0.0, 0.67, -0.46),
    (1, 4, 3, 12, 4, 0.0, 1.0, 0.0),
    (2, 4, 3, 84, 4, 0.0, 0.67, -0.46),        # every sequence
    (3, 4, 3, 30, 2, 0.0, 0.67, -0.46),        # sibling cap
    (4, 5, 2, 30, 5, 0.05, 0.67, -0.46),       # theta stop
    (5, 4, 3, 40, 3, 0.02, 0.67, -0.46),
    (6, 3, 4, 64, 3, 0.01, 1.0, 0.0),          # path probability, theta stop
]


def _brute_misses(build, case):
    seed, V, depths, N, K, theta, a, b = case
    U, W1, W2 = _inputs(seed, V=V, depths=depths)
    anchor = seed % V
    res = build(U, W1, W2, anchor, 0.0, theta, N, K, a, b)
    want, _ = _brute(U, W1, W2, anchor, theta, N, K, a, b)
    got = _paths(res)
    miss = []
    if got != want:   # the same sequences, in the order they were popped
        miss.append((case, got[:6], want[:6]))
    return miss


@pytest.mark.parametrize("case", CASES)
def test_greedy_tree_is_the_top_n_sequences(case):
    assert _brute_misses(TS.build_tree, case) == []


def test_greedy_brute_force_catches_planted_mistakes(monkeypatch):
    def fails(label):
        return any(_brute_misses(TS.build_tree, c) for c in CASES), label

    # the base row of depth d read one depth too deep
    real = TS.child_logits
    with monkeypatch.context() as mp:
        mp.setattr(TS, "child_logits",
                   lambda U, W1, W2, d, t: real(U, W1, W2, min(d + 1, len(U)), t))
        assert fails("depth")[0]
    # the Markov head's factors exchanged (B(v, x) instead of B(x, v))
    with monkeypatch.context() as mp:
        mp.setattr(TS, "child_logits",
                   lambda U, W1, W2, d, t: np.asarray(U[d - 1], np.float64) + W1 @ W2[t])
        assert fails("factors")[0]
    # calibration sign mistake: sigma(a logit(q) - b)
    real_p = TS.log_p_hat
    with monkeypatch.context() as mp:
        mp.setattr(TS, "log_p_hat", lambda q, a, b: real_p(q, a, -b))
        assert fails("bias sign")[0]
    # raw log q as the key (an ablation on the page, not the method)
    with monkeypatch.context() as mp:
        mp.setattr(TS, "log_p_hat", lambda q, a, b: math.log(q) if q > 0 else -math.inf)
        assert fails("raw log q")[0]


def test_calibration_closed_forms():
    assert TS.log_p_hat(0.5) == pytest.approx(-math.log1p(math.exp(0.46)), abs=1e-15)
    for q in (1e-6, 0.01, 0.3, 0.7, 0.999):
        assert math.exp(TS.log_p_hat(q, 1.0, 0.0)) == pytest.approx(q, rel=1e-12)
    qs = np.linspace(0.001, 0.999, 200)
    vals = [TS.log_p_hat(q) for q in qs]
    assert all(x < y for x, y in zip(vals, vals[1:])) and vals[-1] < 0.0


@pytest.mark.parametrize("case", CASES[:5])
def test_small_temperature_limit_equals_greedy(case):
    seed, V, depths, N, K, theta, a, b = case
    U, W1, W2 = _inputs(seed, V=V, depths=depths)
    g = TS.build_tree(U, W1, W2, seed % V, 0.0, theta, N, K, a, b)
    s = TS.build_tree(U, W1, W2, seed % V, 1e-7, theta, N, K, a, b, seed=9)
    for k in ("parent", "token"):
        np.testing.assert_array_equal(s[k], g[k])
    np.testing.assert_allclose(s["logS"], g["logS"], rtol=0, atol=1e-12)


def _hand(T, theta, monkeypatch=None):
    """One depth, three tokens, no Markov term: q0 = (0.5, 0.3, 0.2). The
    root's draws come from the noise of row 0; the first draw is token 1 for
    the seed found below, so its slot is admitted on the bound p_hat(0.5)
    while its own value is p_hat(0.3)."""
    U = np.log(np.array([[0.5, 0.3, 0.2]], dtype=np.float64)).astype(np.float32)
    W = np.zeros((3, 1), np.uint16)
    return TS.build_tree(U, W, W, 0, T, theta, 3, 3, seed=_hand_seed(T))


def _hand_seed(T):
    """A seed whose draw order at the root starts with token 1."""
    l = np.log(np.array([0.5, 0.3, 0.2])).astype(np.float32).astype(np.float64)
    for seed in range(200):
        e = TS.Expansion(l, T, 0, 0, seed, 3)
        if int(e.draws[0]) == 1:
            return seed
    raise AssertionError("no seed")


def _ph(q, a=0.67, b=-0.46):
    return 1.0 / (1.0 + math.exp(-(a * math.log(q / (1 - q)) + b)))


def _hand_misses(build_hand):
    miss = []
    # theta between p_hat(0.3) and p_hat(0.5): the first slot is admitted on
    # its bound p_hat(0.5) although its token (1) has p_hat(0.3) < theta
    theta = 0.5 * (_ph(0.3) + _ph(0.5))
    res = build_hand(1.0, theta)
    if len(res["token"]) < 2 or res["token"][1] != 1:
        miss.append(("bound admits the first slot", res["token"]))
    elif abs(math.exp(res["logS"][1]) - _ph(0.3)) > 1e-6:   # fp32 logits
        miss.append(("survival of the drawn token", res["logS"]))
    # at T = 0.5, q_T = (0.658, 0.237, 0.105): a theta between p_hat(0.5)
    # and p_hat(0.658) admits nothing when the calibrator reads q0
    theta = 0.5 * (_ph(0.5) + _ph(0.25 / 0.38))
    res = build_hand(0.5, theta)
    if len(res["token"]) != 1:
        miss.append(("calibrator reads q0", res["token"]))
    return miss


def test_hand_case_pre_draw_bound_and_q0_calibration():
    assert _hand_misses(_hand) == []


def test_hand_case_catches_planted_mistakes(monkeypatch):
    # admission by the drawn token's own value (violates Proposition 1's
    # condition that a slot is admitted before its value is seen)
    with monkeypatch.context() as mp:
        real = TS.Expansion.max_unused_q0

        def own_value(self, used):
            return self.q0(int(self.draws[len(used)])) if len(used) < len(self.draws) else real(self, used)
        mp.setattr(TS.Expansion, "max_unused_q0", own_value)
        assert _hand_misses(_hand) != []
    # the calibrator fed q_T instead of q0 (the draws keep the true logits)
    with monkeypatch.context() as mp:
        real_init = TS.Expansion.__init__

        def scaled(self, logits, T, *args):
            real_init(self, logits, T, *args)
            if T > 0:
                self.l = logits / T
                m = self.l.max()
                self.lse = m + np.log(np.exp(self.l - m).sum())
        mp.setattr(TS.Expansion, "__init__", scaled)
        assert _hand_misses(_hand) != []


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_sampled_tree_invariants(T):
    """Valid topological trees within the caps; each node's children are
    distinct and are a prefix of that node's own draw order."""
    rng = np.random.default_rng(int(T * 10))
    V, depths, N, K = 64, 5, 40, 4
    U, W1, W2 = _inputs(int(T * 7), V=V, depths=depths, sigma=2.0)
    for req in range(4):
        anchor = int(rng.integers(V))
        res = TS.build_tree(U, W1, W2, anchor, T, 0.0, N, K, seed=3, request=req)
        par, tok, dep = res["parent"], res["token"], res["depth"]
        assert len(par) == N + 1 and par[0] == -1
        assert all(0 <= par[i] < i for i in range(1, len(par)))
        assert dep.max() <= depths
        for v in range(len(par)):
            kids = [i for i in range(1, len(par)) if par[i] == v]
            assert len(kids) <= K
            toks = [int(tok[i]) for i in kids]
            if kids:
                x_v = anchor if v == 0 else int(tok[v])
                e = TS.Expansion(TS.child_logits(U, _widen(W1), _widen(W2), int(dep[v]) + 1, x_v),
                                 T, req * (N + 1) + v, 0, 3, K)
                assert toks == [int(x) for x in e.draws[:len(toks)]]
