"""TreeSpark's best-first draft-tree construction with the calibrated theta
stop, in fp64.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module.

Sources (TreeSpark: Markov-conditioned draft trees, paper 2609.22098):
  §3.1  the drafter: one backbone pass gives base logits U_1..U_b (one row per
        depth); a rank-r Markov head B(x, v) = <W1[x], W2[v]>.
  §3.2  step 1: a child at depth d of a parent with token x_p is drawn from
        q_{0,d}(. | x_p) = softmax(U_d + B(x_p, .)); step 2: a max-heap of
        candidate children keyed by calibrated path survival (the product of
        p_hat along the root path); at T = 0 the candidate is the most probable
        unused token under its parent's conditional, at T > 0 it is drawn
        without replacement; materialising a node opens a slot for its first
        child and, up to K siblings, one for its parent's next child; at T > 0
        a slot is keyed by the admissible pre-draw bound S(v) p_hat(max q0
        unused).
  §1, §3.4  p_hat = sigma(a logit(q0) + b) on the unscaled conditional q0
        (temperature 1 whatever the sampling temperature); deployed a/b =
        0.67/-0.46.
  §3.5  cumulative log p_hat orders the heap; expansion stops when the best
        remaining path survival falls below theta, with a node cap (64).
  §3.3  siblings are drawn without replacement from q_T and their draw order
        is what the verifier replays.

Readings of points the pages leave open:
  * node counts exclude the root: the cap N bounds the drafted nodes;
  * U[d-1] is the base row of depth d (d = 1..b); a node at depth b has no
    child slot;
  * a node's "slot" is its next child (the first, then the next sibling up to
    K); its key is log S(v) + log p_hat(m), m = the largest q0 of v's
    conditional among tokens not yet used as v's children. At T = 0 that
    token is the child (exact key); at T > 0 the child is v's next
    without-replacement draw and S(child) = S(v) p_hat(q0(child)) may fall
    below the key that admitted it;
  * draws without replacement are Gumbel-top-k on the conditional's logits
    over T: score(y) = l(y)/T - ln(-ln u(y)), u from Philox4x32-10 at
    counter (y // 4, node_row, stream, 0), key seed; node_row = request *
    (N + 1) + the node's index in materialisation order;
  * ties: larger key first, then the lower node index; token orders: larger
    logit (or score) first, then the lower token id;
  * the tree lists the root (token -1), then the nodes in materialisation
    order (parents before children, siblings in draw order).
"""
import heapq

import numpy as np

from .attention import decode_values
from .siblings import uniforms as philox_uniforms

CALIB_A, CALIB_B = 0.67, -0.46


def log_p_hat(q0, a=CALIB_A, b=CALIB_B):
    """log sigma(a logit(q0) + b) ([TreeSpark §1, §3.4])."""
    q0 = float(q0)
    if q0 <= 0.0:
        return -np.inf
    if q0 >= 1.0:
        return 0.0
    z = a * (np.log(q0) - np.log1p(-q0)) + b
    return -np.logaddexp(0.0, -z)


def child_logits(U, W1, W2, depth, token):
    """l(.) = U_depth + B(token, .) for the children at `depth` (1-based) of a
    node carrying `token` ([TreeSpark §3.1, §3.2 step 1]); W1, W2 fp64."""
    return np.asarray(U[depth - 1], dtype=np.float64) + W2 @ W1[token]


def top_order(values, n):
    """Indices of the n largest values, larger first, lower index on ties
    (every value tied with the n-th is considered before the cut)."""
    v = np.asarray(values, dtype=np.float64)
    if n >= len(v):
        return np.lexsort((np.arange(len(v)), -v))
    cut = np.partition(v, len(v) - n)[len(v) - n]
    cand = np.nonzero(v >= cut)[0]
    return cand[np.lexsort((cand, -v[cand]))][:n]


class Expansion:
    """A materialised node's conditional: logits, log-sum-exp, the token
    order by logit, and (T > 0) its without-replacement draw order."""

    def __init__(self, logits, T, node_row, stream, seed, K):
        self.l = logits
        m = logits.max()
        self.lse = m + np.log(np.exp(logits - m).sum())
        V = len(logits)
        self.order = top_order(logits, K + 1)   # no node has more than K children
        if T > 0:
            u = philox_uniforms(V, node_row, stream, seed)
            self.score = logits / float(np.float32(T)) - np.log(-np.log(u))
            self.draws = top_order(self.score, K)
        else:
            self.score = None
            self.draws = self.order[:K]

    def q0(self, y):
        return float(np.exp(self.l[y] - self.lse))

    def max_unused_q0(self, used):
        for y in self.order:
            if int(y) not in used:
                return self.q0(int(y))
        return 0.0


def build_tree(U, W1, W2, anchor, T, theta, N, K, a=CALIB_A, b=CALIB_B, seed=0, stream=0,
               request=0, log=None):
    """Best-first construction for one request.

    U [depths][V] fp32 base logits; W1, W2 [V][r] as fp64 (or bf16 bits,
    widened exactly); anchor = the root's token. Returns dict(parent, token,
    logS, depth) in materialisation order (root first). `log`, when a list,
    receives the decision margins: ("pop", gap to the runner-up key),
    ("theta", |best key - log theta|), ("order", smallest gap among the first
    K+1 logits or draw scores of an expanded node)."""
    W1 = np.asarray(W1)
    W2 = np.asarray(W2)
    if W1.dtype == np.uint16:
        W1 = decode_values(W1, "bf16")
    if W2.dtype == np.uint16:
        W2 = decode_values(W2, "bf16")
    depths = len(U)
    log_theta = np.log(theta) if theta > 0 else -np.inf
    parent, token, logS, depth = [-1], [-1], [0.0], [0]
    used = [set()]
    exps = {}

    def expand(i, tok):
        if depth[i] >= depths:
            return
        e = Expansion(child_logits(U, W1, W2, depth[i] + 1, tok), T,
                      request * (N + 1) + i, stream, seed, K)
        exps[i] = e
        if log is not None:
            s = e.score if e.score is not None else e.l
            top = s[top_order(s, K + 1)]
            if len(top) > 1:
                log.append(("order", i, float(np.min(top[:-1] - top[1:]))))

    def key(i):
        return logS[i] + log_p_hat(exps[i].max_unused_q0(used[i]), a, b)

    expand(0, anchor)
    heap = []  # (-key, node index): larger key first, lower index on ties
    if 0 in exps and K > 0:
        heapq.heappush(heap, (-key(0), 0))
    while len(parent) - 1 < N and heap:
        nk, v = heapq.heappop(heap)
        best = -nk
        if log is not None:
            if heap:
                log.append(("pop", v, best - (-heap[0][0])))
            if log_theta > -np.inf:
                log.append(("theta", v, abs(best - log_theta)))
        if best < log_theta:
            break
        e = exps[v]
        j = len(used[v])                       # this is v's (j+1)-th child
        x = int(e.draws[j])
        c = len(parent)
        parent.append(v)
        token.append(x)
        logS.append(logS[v] + log_p_hat(e.q0(x), a, b))
        depth.append(depth[v] + 1)
        used.append(set())
        used[v].add(x)
        if j + 1 < min(K, len(e.l)):           # v's next sibling slot
            heapq.heappush(heap, (-key(v), v))
        expand(c, x)                           # c's first-child slot
        if c in exps:
            heapq.heappush(heap, (-key(c), c))
    return dict(parent=np.asarray(parent, np.int32), token=np.asarray(token, np.int32),
                logS=np.asarray(logS), depth=np.asarray(depth, np.int32))


def build_batch(U, W1, W2, anchors, temperatures, thetas, N, K, a=CALIB_A, b=CALIB_B, seed=0,
                stream=0, requests=None):
    """U [B][depths][V]; returns a list of per-request results (with their
    decision logs under "log")."""
    W1 = decode_values(W1, "bf16") if np.asarray(W1).dtype == np.uint16 else np.asarray(W1)
    W2 = decode_values(W2, "bf16") if np.asarray(W2).dtype == np.uint16 else np.asarray(W2)
    out = []
    for r in (range(len(anchors)) if requests is None else requests):
        lg = []
        res = build_tree(U[r], W1, W2, int(anchors[r]), float(temperatures[r]),
                         float(thetas[r]), N, K, a, b, seed, stream, r, lg)
        res["log"] = lg
        out.append(res)
    return out


def near(log, eps):
    """True when a decision of the construction lies within eps of going the
    other way (a key against the runner-up or theta, or a token order)."""
    return any(m < eps for _, _, m in log)
