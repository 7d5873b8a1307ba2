"""Drawing a node's children without replacement: Gumbel-top-k.

[survey, Timeline]: Recursive Speculative Decoding draws tree siblings without
replacement via Gumbel-Top-k (and stochastic beam search); Sequoia also
switched to sampling without replacement. [TreeSpark §1, §3.3]: siblings are
drawn without replacement from the draft distribution q_T, and their draw
order is what the verifier replays.

Definition, for an expanded row with draft logits d[0..V-1], temperature T
and k children:
  T > 0:  score(y) = d[y] / T + g(y),  g(y) = -ln(-ln u(y)),
  T = 0:  score(y) = d[y];
the children are the k tokens of largest score, in descending score (ties:
lower token id first). At T > 0 this is k sequential draws without
replacement from softmax(d / T) (the Gumbel-max trick applied k times).

Noise: u(y) comes from the counter-based generator Philox4x32-10 (Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC
2011), counter (y // 4, row, stream, 0), key (seed mod 2^32, seed // 2^32),
output word y % 4; u = ((word >> 8) + 1/2) / 2^24, strictly inside (0, 1).
The draw is computed in fp64 here.

Pins: the law of the ordered draw (chi-square against the sequential
without-replacement product formula, with planted-mistake controls) and T = 0
as plain top-k. The generator is pinned to the known-answer vectors its
authors publish with their Random123 library (the pages print none), and
checked for uniformity and keying; the GPU side is compared bit-exact against
this implementation of the same published definition.
"""
import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57      # Philox4x32 multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85      # Weyl key increments
MASK = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on uint32 arrays (broadcasting); returns 4 words."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK for c in (c0, c1, c2, c3))
    k0 = np.uint64(k0 & MASK)
    k1 = np.uint64(k1 & MASK)
    for rnd in range(10):
        if rnd:
            k0 = np.uint64((int(k0) + W0) & MASK)
            k1 = np.uint64((int(k1) + W1) & MASK)
        p0 = np.uint64(M0) * c0
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def uniforms(V, row, stream, seed):
    """u(y) for y = 0..V-1 of one row, as fp64."""
    y = np.arange(V, dtype=np.uint64)
    words = philox4x32_10(y >> np.uint64(2), np.full(V, row), np.full(V, stream),
                          np.zeros(V), int(seed) & MASK, (int(seed) >> 32) & MASK)
    w = np.choose((y & np.uint64(3)).astype(np.int64), words).astype(np.uint64)
    return ((w >> np.uint64(8)).astype(np.float64) + 0.5) / float(1 << 24)


def scores(draft_row, temperature, row, stream, seed):
    d = np.asarray(draft_row, dtype=np.float32).astype(np.float64)
    if temperature <= 0:
        return d
    u = uniforms(d.shape[0], row, stream, seed)
    return d / float(np.float32(temperature)) - np.log(-np.log(u))


def draw_children(draft_row, k, temperature, row, stream, seed):
    """(tokens [k] in draw order, their scores)."""
    s = scores(draft_row, temperature, row, stream, seed)
    order = np.lexsort((np.arange(s.shape[0]), -s))[:k]
    return order.astype(np.int32), s[order]


def tree_draw_siblings(draft_logits, counts, temperature, stream, seed, kmax):
    """Batched form: tokens [R][kmax] (-1 padded) and, per row, the gap between
    consecutive scores among the first k+1 in draw order (for near-tie
    accounting)."""
    R = draft_logits.shape[0]
    tokens = np.full((R, kmax), -1, dtype=np.int32)
    min_gap = np.full(R, np.inf)
    for r in range(R):
        k = int(counts[r])
        if k <= 0:
            continue
        s = scores(draft_logits[r], float(temperature[r]), r, stream, seed)
        order = np.lexsort((np.arange(s.shape[0]), -s))[:k + 1]
        tokens[r, :min(k, len(order))] = order[:k]  # fewer tokens than k: the rest stay -1
        top = s[order]
        if len(top) > 1:
            min_gap[r] = float(np.min(top[:-1] - top[1:]))
    return tokens, min_gap
