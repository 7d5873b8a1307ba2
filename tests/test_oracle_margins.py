"""Pins for the parts of the oracle that decide what is compared at all: the
exact widening of stored inputs, the near-threshold margins of the sampling
walk, and the near-tie test of the EAGLE-2 construction.

Every pin here is a value derived by hand (bit patterns, closed forms) or an
independent library routine (torch's own bfloat16 widening); each block ends
with planted mistakes that the pins must catch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.sampler as osamp
from oracle import construct

# random bf16 bit patterns include NaNs; widening them is expected to warn
pytestmark = pytest.mark.filterwarnings("ignore:invalid value encountered in cast")

# ---------------------------------------------------------------------------
# decode_values: bf16 bit patterns and fp32 values widened exactly to fp64.

# (bits, value) read off the bfloat16 format by hand: sign, 8 exponent bits
# (bias 127), 7 mantissa bits.
BF16_HAND = [
    (0x3F80, 1.0),
    (0xC000, -2.0),
    (0x0001, 2.0 ** -133),                       # smallest subnormal: 2^-126 * 2^-7
    (0x0080, 2.0 ** -126),                       # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),    # largest finite
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
    (0x3E20, 0.15625),                           # 2^-3 * 1.25
    (0x4049, 3.140625),                          # 2 * (1 + 73/128)
    (0xBF01, -(1.0 + 1.0 / 128.0) * 0.5),
]


def _decode_misses(fn):
    """Hand patterns, negative zero, NaN, and 4096 random patterns against
    torch's widening; returns the list of failures."""
    miss = []
    bits = np.array([b for b, _ in BF16_HAND], dtype=np.uint16)
    got = fn(bits, "bf16")
    for (b, want), g in zip(BF16_HAND, got):
        if not (g == want):
            miss.append(("hand", hex(b), g, want))
    nz = fn(np.array([0x8000], dtype=np.uint16), "bf16")[0]
    if not (nz == 0.0 and math.copysign(1.0, nz) < 0):
        miss.append(("-0", nz))
    if not np.isnan(fn(np.array([0x7FC0], dtype=np.uint16), "bf16")[0]):
        miss.append(("nan",))
    rng = np.random.default_rng(7)
    rb = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(rb.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    g = fn(rb, "bf16")
    ok = (g == ref) | (np.isnan(g) & np.isnan(ref))
    if not ok.all():
        miss.append(("torch", int((~ok).sum())))
    f = rng.normal(0, 3, 512).astype(np.float32)
    if not (fn(f, "fp32") == np.array([float(x) for x in f.tolist()])).all():
        miss.append(("fp32",))
    return miss


def test_decode_values_bf16_and_fp32():
    assert _decode_misses(oracle.decode_values) == []


def _shift15(a, dtype):
    if dtype != "bf16":
        return oracle.decode_values(a, dtype)
    return (np.asarray(a, np.uint32) << 15).view(np.float32).astype(np.float64)


def _no_sign(a, dtype):
    if dtype != "bf16":
        return oracle.decode_values(a, dtype)
    return oracle.decode_values(np.asarray(a, np.uint16) & np.uint16(0x7FFF), dtype)


def _byteswap(a, dtype):
    if dtype != "bf16":
        return oracle.decode_values(a, dtype)
    return oracle.decode_values(np.asarray(a, np.uint16).byteswap(), dtype)


def _via_fp16(a, dtype):
    if dtype != "bf16":
        return oracle.decode_values(a, dtype)
    return np.asarray(a, np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("planted", [_shift15, _no_sign, _byteswap, _via_fp16])
def test_decode_pins_catch_planted_mistakes(planted):
    assert _decode_misses(planted) != []


# ---------------------------------------------------------------------------
# inverse_cdf: the draw's token and its margin (distance of u * sum to the
# nearer boundary of the token's interval, over the sum).

# (weights, u, token, margin), derived by hand from the cumulative sums.
CDF_HAND = [
    ([1, 1, 2], 0.375, 1, 0.125),    # c = 1, 2, 4; u*S = 1.5: both boundaries 0.5 away
    ([1, 1, 2], 0.3, 1, 0.05),       # u*S = 1.2: 0.2 above c0 = 1
    ([1, 1, 2], 0.49, 1, 0.01),      # u*S = 1.96: 0.04 below c1 = 2
    ([1, 1, 2], 0.25, 1, 0.0),       # u*S = 1 = c0 exactly: the next token, on its boundary
    ([1, 1, 2], 0.9, 2, 0.1),        # u*S = 3.6: 0.4 below the end
    ([0, 3, 0, 1], 0.75, 3, 0.0),    # u*S = 3 = c1 = c2: zero-mass token 2 is skipped
    ([0, 3, 0, 1], 0.8, 3, 0.05),    # u*S = 3.2
    ([0, 3, 0, 1], 0.5, 1, 0.25),    # u*S = 2: 1 below c1 = 3, 2 above c0 = 0
    ([5], 0.7, 0, 0.3),
]


def _cdf_misses(fn):
    miss = []
    for w, u, y, mg in CDF_HAND:
        gy, gm = fn(np.asarray(w, dtype=np.float64), u)
        if gy != y or abs(gm - mg) > 1e-15:
            miss.append((w, u, gy, gm, y, mg))
    return miss


def test_inverse_cdf_margins():
    assert _cdf_misses(oracle.inverse_cdf) == []


def test_inverse_cdf_pins_catch_planted_mistakes(monkeypatch):
    # the farther boundary instead of the nearer one
    with monkeypatch.context() as mp:
        mp.setattr(osamp, "min", max, raising=False)
        assert _cdf_misses(oracle.inverse_cdf) != []
    # ties at a boundary resolved to the left (side="left")
    orig = np.searchsorted
    with monkeypatch.context() as mp:
        mp.setattr(osamp.np, "searchsorted", lambda a, v, side="right": orig(a, v, side="left"))
        assert _cdf_misses(oracle.inverse_cdf) != []
    # margin left in units of the unnormalised sum
    assert _cdf_misses(lambda w, u: (oracle.inverse_cdf(w, u)[0],
                                     oracle.inverse_cdf(w, u)[1] * np.sum(w))) != []


# ---------------------------------------------------------------------------
# The walk's decision log: ("accept", node, |u - ratio|) for every test whose
# ratio is below 1, ("draw", node, margin) for the final draw.
#
# Hand case (V = 3, T = 1): root target logits (0, 0, 1), draft logits
# (1, 0, 0), so p = (1, 1, e)/(2 + e) and q = (e, 1, 1)/(2 + e).
#  * a child with token 0 has ratio p(0)/q(0) = 1/e;
#  * a child with token 2 has ratio e >= 1 (always accepted, nothing logged);
#  * after rejecting token 0 the residual max(p - q, 0) is (0, 0, e - 1)/(2 + e)
#    (token 1's p and q are equal): a draw from it is token 2 with margin
#    min(u, 1 - u);
#  * the child's own row has uniform target logits: its bonus draw with
#    u = 0.5 is token 1, margin 1/6.
E = math.e


def _hand_walk(token, u_acc, u_root=0.25, u_child=0.5):
    t = np.array([[0, 0, 1], [0, 0, 0]], dtype=np.float32)
    d = np.array([[1, 0, 0], [0, 0, 0]], dtype=np.float32)
    uni = np.array([[0.0, u_root], [u_acc, u_child]], dtype=np.float32)
    return oracle.walk_request(t, d, np.array([-1, token]), np.array([-1, 0]), 1.0, uni)


def _log_misses(walk):
    miss = []
    r = 1.0 / E
    for delta, accept in ((-1e-7, True), (1e-7, False), (-0.2, True), (0.3, False)):
        u = np.float32(r + delta)
        flag, nt, log = walk(0, u)
        want_m = abs(float(u) - r)
        kinds = [k for k, _, _ in log]
        if kinds != ["accept", "draw"]:
            miss.append(("kinds", delta, kinds))
            continue
        if log[0][1] != 1 or abs(log[0][2] - want_m) > 1e-13:
            miss.append(("accept margin", delta, log[0], want_m))
        if bool(flag[1]) != accept:
            miss.append(("decision", delta, flag))
        if accept:
            if log[1][1] != 1 or nt[1] != 1 or abs(log[1][2] - 1 / 6) > 1e-13:
                miss.append(("bonus", delta, log[1], nt))
        elif log[1][1] != 0 or nt[0] != 2 or abs(log[1][2] - 0.25) > 1e-13:
            miss.append(("correction", delta, log[1], nt))
    # ratio e >= 1: accepted whatever u, and no acceptance margin logged
    flag, nt, log = walk(2, np.float32(0.999))
    if [k for k, _, _ in log] != ["draw"] or flag[1] != 1:
        miss.append(("ratio >= 1", log, flag))
    return miss


def test_walk_acceptance_log():
    assert _log_misses(_hand_walk) == []


def test_walk_log_pins_catch_planted_mistakes(monkeypatch):
    # a signed margin u - ratio instead of its size
    with monkeypatch.context() as mp:
        mp.setattr(osamp, "abs", lambda x: x, raising=False)
        assert _log_misses(_hand_walk) != []
    # the ratio inverted (q/p)
    with monkeypatch.context() as mp:
        mp.setattr(osamp, "acceptance_ratio", lambda px, qx: float(qx) / float(px))
        assert _log_misses(_hand_walk) != []
    # the complement 1 - ratio
    with monkeypatch.context() as mp:
        real = osamp.acceptance_ratio
        mp.setattr(osamp, "acceptance_ratio", lambda px, qx: 1.0 - real(px, qx))
        assert _log_misses(_hand_walk) != []


def test_near_threshold_reading():
    log = [("accept", 1, 0.5), ("draw", 1, 0.25)]
    assert not osamp.near_threshold(log, 0.2)
    assert osamp.near_threshold(log, 0.3)        # the draw is within 0.3
    assert osamp.near_threshold(log, 0.6)
    assert osamp.near_threshold([("draw", 0, 0.9), ("degenerate", 2, 0.0)], 1e-30)
    assert not osamp.near_threshold([], 1.0)
    # the hand walk at 1e-7 from its ratio is near at 1e-6 and not at 1e-8
    _, _, log = _hand_walk(0, np.float32(1.0 / E - 1e-7))
    m = log[0][2]
    assert osamp.near_threshold(log, 1e-6) and not osamp.near_threshold(log, m * 0.5)


# ---------------------------------------------------------------------------
# construct.near_ties on hand-built candidate sets: k = 2, so round 1 (the
# root) makes ids 0-1 and round 2 makes ids 2-5; eps = 1e-4.

NEAR_HAND = [
    # (round-1 values, round-2 values, m, expected, what it exercises)
    ([-0.1, -0.5], [-0.6, -0.7, -0.9, -1.2], 3, False, "all gaps >= eps"),
    ([-0.1, -0.5], [-0.6, -0.7, -0.70005, -1.2], 3, True, "round-2 cut gap 5e-5"),
    ([-0.1, -0.5], [-0.6, -0.60005, -0.9, -1.2], 4, True, "round-2 order gap 5e-5"),
    ([-0.1, -0.5], [-0.6, -0.6, -0.9, -1.2], 4, False, "exact sibling tie"),
    ([-0.1, -0.5], [-0.6, -0.7, -0.9, -0.90005], 5, True, "rerank cut gap 5e-5"),
    ([-0.1, -0.5], [-0.6, -0.7, -0.9, -0.90005], 4, False, "same values, cut elsewhere"),
    ([-0.1, -0.10005], [-0.6, -0.7, -0.9, -1.2], 3, True, "round-1 order gap"),
    ([-0.1, -0.5], [-0.6, -0.7, -0.8, -0.80005], 3, False, "a close pair below every cut"),
    ([-0.1, -0.5], [-0.6, -0.7, -0.70015, -1.2], 3, False, "cut gap 1.5e-4, above eps"),
]


def _near_case(r1, r2):
    c = construct.Candidates()
    for v in r1 + r2:
        c.add(v, 0, -1)
    return c, [[0, 1], [2, 3]]


def _near_misses(fn):
    miss = []
    for r1, r2, m, want, what in NEAR_HAND:
        c, fr = _near_case(r1, r2)
        if bool(fn(c, fr, 2, m, 1e-4)) != want:
            miss.append(what)
    return miss


def test_near_ties_hand_cases():
    assert _near_misses(construct.near_ties) == []


def test_near_ties_pins_catch_planted_mistakes(monkeypatch):
    # exact ties counted as near
    with monkeypatch.context() as mp:
        mp.setattr(construct, "near_gap", lambda g, eps: float(g) < eps)
        assert "exact sibling tie" in _near_misses(construct.near_ties)
    # only the cut of each round checked, not the order of its k best
    with monkeypatch.context() as mp:
        mp.setattr(construct, "order_gaps", lambda vals, n: construct.cut_gap(vals, n))
        assert "round-2 order gap 5e-5" in _near_misses(construct.near_ties)
    # the rerank cut forgotten
    with monkeypatch.context() as mp:
        mp.setattr(construct, "cut_gap", lambda vals, n: np.zeros(0))
        assert "rerank cut gap 5e-5" in _near_misses(construct.near_ties)
    # every round taken as k * k ids (the root round's k forgotten)
    with monkeypatch.context() as mp:
        mp.setattr(construct, "round_ranges", lambda k, r: [(i * k * k, k * k) for i in range(r)])
        assert _near_misses(construct.near_ties) != []
    # the order gaps taken among the n best only (the cut below them lost)
    with monkeypatch.context() as mp:
        real = construct.order_gaps
        mp.setattr(construct, "order_gaps", lambda vals, n: real(vals, n)[:max(n - 1, 0)])
        assert "round-2 cut gap 5e-5" in _near_misses(construct.near_ties)
