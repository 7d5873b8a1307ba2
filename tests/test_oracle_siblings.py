"""Pins for the oracle's sibling draw (Gumbel-top-k without replacement).

The law of the ordered k-tuple is checked against the product formula of k
sequential draws without replacement from softmax(d/T) (what RSD and TreeSpark
mean by drawing siblings without replacement), by a chi-square test over many
independent rows; planted mistakes in the noise must fail it. T = 0 is the
closed-form top-k with lowest-index ties. The generator itself is pinned to
the known-answer vectors its authors publish (tests/golden/philox4x32_10_kat.txt).
"""
import itertools
import pathlib

import numpy as np
import pytest
from scipy import stats

from oracle import siblings as S


def _batched_scores(d, T, rows, stream, seed, noise="gumbel"):
    """[n][V] scores for rows 0..n-1, vectorised over rows."""
    V = d.shape[0]
    y = np.arange(V, dtype=np.uint64)[None, :]
    r = np.asarray(rows, dtype=np.uint64)[:, None]
    words = S.philox4x32_10(np.broadcast_to(y >> np.uint64(2), (len(rows), V)),
                            np.broadcast_to(r, (len(rows), V)), np.full((len(rows), V), stream),
                            np.zeros((len(rows), V)), seed & 0xFFFFFFFF, seed >> 32)
    idx = np.broadcast_to((y & np.uint64(3)).astype(np.int64), (len(rows), V))
    w = np.choose(idx, words).astype(np.uint64)
    u = ((w >> np.uint64(8)).astype(np.float64) + 0.5) / float(1 << 24)
    if noise == "gumbel":
        g = -np.log(-np.log(u))
    elif noise == "exponential":      # planted mistake: -ln u is not Gumbel noise
        g = -np.log(u)
    else:                             # planted mistake: sign of the outer log flipped
        g = np.log(-np.log(u))
    return d[None, :] / T + g


def _law(d, T, k):
    q = np.exp(d / T - (d / T).max())
    q /= q.sum()
    law = {}
    for tup in itertools.permutations(range(len(d)), k):
        p, rest = 1.0, 1.0
        for x in tup:
            p *= q[x] / rest
            rest -= q[x]
        law[tup] = p
    return law


def _chi2_pvalue(d, T, k, n, noise="gumbel", seed=12345):
    sc = _batched_scores(d, T, np.arange(n), 7, seed, noise)
    top = np.argsort(-sc, axis=1, kind="stable")[:, :k]
    law = _law(d, T, k)
    keys = list(law)
    code = {t: i for i, t in enumerate(keys)}
    counts = np.zeros(len(keys))
    for row in map(tuple, top):
        counts[code[row]] += 1
    expected = np.array([law[t] for t in keys]) * n
    return stats.chisquare(counts, expected).pvalue


@pytest.mark.parametrize("T", [0.6, 1.0, 2.0])
def test_gumbel_topk_law_is_sequential_without_replacement(T):
    d = np.array([1.2, -0.3, 0.5, 2.0, 0.0])
    assert _chi2_pvalue(d, T, 3, 60000) > 1e-3


@pytest.mark.parametrize("noise", ["exponential", "flipped"])
def test_planted_noise_mistakes_fail_the_law(noise):
    d = np.array([1.2, -0.3, 0.5, 2.0, 0.0])
    assert _chi2_pvalue(d, 1.0, 3, 60000, noise=noise) < 1e-6


def test_batched_scores_match_the_row_function():
    d = np.random.default_rng(0).standard_normal(37).astype(np.float32)
    sc = _batched_scores(d.astype(np.float64), float(np.float32(0.8)), [3, 11], 5, 99)
    for i, r in enumerate([3, 11]):
        assert np.allclose(sc[i], S.scores(d, np.float32(0.8), r, 5, 99), rtol=0, atol=1e-12)


def test_greedy_is_topk_with_lowest_index_ties():
    d = np.array([0.5, 2.0, -1.0, 2.0, 0.5, 3.0, 0.5], dtype=np.float32)
    tok, _ = S.draw_children(d, 5, 0.0, 0, 0, 0)
    assert tok.tolist() == [5, 1, 3, 0, 4]


def test_batched_form_pads_and_reports_gaps():
    g = np.random.default_rng(1)
    logits = g.standard_normal((4, 50)).astype(np.float32)
    tokens, gap = S.tree_draw_siblings(logits, np.array([3, 0, 1, 5]), np.array([1.0, 1.0, 0.0, 0.5],
                                       dtype=np.float32), 2, 77, kmax=6)
    assert (tokens[1] == -1).all() and (tokens[0, 3:] == -1).all() and tokens[3, :5].min() >= 0
    assert np.isinf(gap[1]) and (gap[[0, 2, 3]] > 0).all()
    for r, k in enumerate([3, 0, 1, 5]):
        if k:
            assert len(set(tokens[r, :k].tolist())) == k


def test_philox_uniforms_are_uniform_and_keyed():
    u = S.uniforms(1 << 20, 3, 1, 2024)
    assert u.min() > 0 and u.max() < 1
    hist = np.histogram(u, bins=64, range=(0, 1))[0]
    assert stats.chisquare(hist).pvalue > 1e-3
    # consecutive words are not correlated
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 0.01
    # every counter and key word changes the stream
    base = S.uniforms(64, 3, 1, 2024)
    for other in (S.uniforms(64, 4, 1, 2024), S.uniforms(64, 3, 2, 2024),
                  S.uniforms(64, 3, 1, 2025), S.uniforms(64, 3, 1, 2024 + (1 << 32))):
        assert (other != base).mean() > 0.9


def _kat_vectors():
    path = pathlib.Path(__file__).parent / "golden" / "philox4x32_10_kat.txt"
    out = []
    for line in path.read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            c, k, w = (tuple(int(x, 16) for x in part.split()) for part in line.split("|"))
            out.append((c, k, w))
    return out


def test_philox_matches_the_published_known_answers():
    vectors = _kat_vectors()
    assert len(vectors) == 3
    for c, k, want in vectors:
        got = S.philox4x32_10(*c, *k)
        assert tuple(int(x) for x in got) == want


def test_philox_known_answers_catch_planted_round_mistakes():
    """Nine rounds, or a key schedule bumped before the first round, miss the vectors."""
    c, k, want = _kat_vectors()[2]

    def variant(rounds, bump_first):
        c0, c1, c2, c3 = (np.uint64(x) for x in c)
        k0, k1 = k
        for rnd in range(rounds):
            if rnd or bump_first:
                k0, k1 = (k0 + S.W0) & S.MASK, (k1 + S.W1) & S.MASK
            p0, p1 = np.uint64(S.M0) * c0, np.uint64(S.M1) * c2
            c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & np.uint64(S.MASK),
                              (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & np.uint64(S.MASK))
        return tuple(int(x) for x in (c0, c1, c2, c3))

    assert variant(10, False) == want   # the same construction, unplanted, meets the vector
    assert variant(9, False) != want
    assert variant(10, True) != want
