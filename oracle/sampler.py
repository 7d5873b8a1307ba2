"""The multi-step speculative-sampling walk over a draft tree, in fp64.

Sources:
  [survey, Timeline]   SpecInfer's multi-step speculative sampling: a
                       recursive, residual-renormalising rejection walk.
  [survey, Taxonomy]   rule (a) greedy exact match; rule (b) multi-draft
                       rejection sampling with replacement (SpecInfer's MSS,
                       MCSD Algorithm 1); rule (c) recursive rejection
                       sampling without replacement.
  [TreeSpark §1, §3.3] siblings drawn without replacement from the residual
                       q_T; each proposal is rebuilt from the shared logits and
                       the sibling draw order; accept child x with probability
                       min(1, p(x)/q(x)), and after a rejection subtract the
                       proposal from the target residual and renormalise
                       (Proposition 1 and its proof sketch).
  [TreeSpark §3.2 step 3] commit the longest surviving root path plus one
                       correction or bonus token from the target posterior;
                       greedy decoding uses exact target-token matching.
  [explainer, Red flags] exactly one path is accepted.

Readings of points the pages leave open:
  * row i of the logits is the distribution of the token after node i
    ([TreeSpark §3.1] LM-shifted alignment);
  * children of v are tested in ascending row index (= draw order);
  * rule (c): the stage-j proposal is q with the already-drawn siblings
    zeroed, divided by 1 - sum of their q mass; the residual subtracts that
    proposal;
  * rule (b): siblings are independent draws from q, so every stage's
    proposal is q itself (a repeated token meets a residual that is already 0
    there and is rejected);
  * accept iff u < ratio (ratio >= 1 always accepts); u_acc = uniforms[c][0]
    for node c's own test, u_res = uniforms[v][1] for the draw if the walk
    stops at v;
  * the correction/bonus draw is the inverse CDF over ascending token id:
    the smallest y with cumsum(res)[y] > u * sum(res);
  * a residual whose sum is exactly 0 (probability zero in exact arithmetic)
    is left unchanged and the event is logged as near-threshold;
  * p = softmax(t / T), q = softmax(d / T); T == 0 means greedy exact match.
"""
import numpy as np

from .tree import children, check_tree


def softmax_T(logits, T):
    """softmax(logits / T) in fp64 with the max subtracted ([TreeSpark §3.4]:
    the temperature-scaled conditional q_T)."""
    x = np.asarray(logits, dtype=np.float32).astype(np.float64) / float(T)
    e = np.exp(x - x.max())
    return e / e.sum()


def proposal_without(q, drawn):
    """Stage proposal: q restricted to tokens not yet drawn, renormalised
    ([TreeSpark §1]: 'without replacement from the residual q_T')."""
    qj = np.array(q, dtype=np.float64, copy=True)
    if drawn:
        idx = np.asarray(drawn, dtype=np.int64)
        mass = q[idx].sum()
        qj[idx] = 0.0
        qj /= (1.0 - mass)
    return qj


def proposal_with(q, drawn):
    """Stage proposal of rule (b): the siblings are independent draws from q
    ([survey, Taxonomy] rule (b): SpecInfer's MSS, MCSD Algorithm 1), so the
    proposal stays q whatever was drawn before."""
    return np.array(q, dtype=np.float64, copy=True)


def residual_update(pres, qj):
    """After a rejection: max(p_j - q_j, 0) renormalised ([TreeSpark §3.3]).
    Returns (new residual, sum before normalising, degenerate flag)."""
    r = np.maximum(pres - qj, 0.0)
    s = r.sum()
    if s > 0:
        return r / s, s, False
    return pres, 0.0, True


def acceptance_ratio(p_x, q_x):
    """p_j(x) / q_j(x); +inf when q_j(x) == 0 < p_j(x), 0 when both are 0."""
    if q_x > 0:
        return float(p_x) / float(q_x)
    return float("inf") if p_x > 0 else 0.0


def inverse_cdf(pres, u):
    """Smallest y with cumsum(pres)[y] > u * sum(pres); returns (y, margin)
    where margin is the distance of u*sum to the nearer boundary of y's
    interval, divided by the sum."""
    c = np.cumsum(pres)
    total = c[-1]
    thr = float(u) * total
    y = int(np.searchsorted(c, thr, side="right"))
    if y >= len(c):  # only reachable through rounding: take the last token with mass
        y = int(np.nonzero(pres > 0)[0][-1])
    lo = c[y - 1] if y > 0 else 0.0
    margin = min(thr - lo, c[y] - thr) / total
    return y, margin


def greedy_request(t_rows, tokens, parent):
    """T == 0 ([survey, Taxonomy] rule (a); [TreeSpark §3.2 step 3]):
    next_token[i] = argmax t_i (lowest index on ties) for every node;
    flag[i] = (token[i] == next_token[parent[i]]); flag[root] = 1."""
    check_tree(parent)
    n = len(parent)
    nt = np.asarray([int(np.argmax(t_rows[i])) for i in range(n)], dtype=np.int32)
    flag = np.zeros(n, dtype=np.int8)
    flag[0] = 1
    for i in range(1, n):
        flag[i] = 1 if int(tokens[i]) == int(nt[parent[i]]) else 0
    return flag, nt, []


def greedy_walk_request(t_rows, tokens, parent):
    """T == 0 along the walk only ([survey, Taxonomy] rule (a); [TreeSpark
    §3.2 step 3]: greedy decoding matches target tokens exactly; the rows the
    walk never reaches are not needed for the accepted path). From the root:
    next_token[v] = argmax t_v (lowest index on ties) at every visited node;
    every child c of v is tested, flag[c] = (token[c] == next_token[v]); the
    walk moves to the first flagged child in draw order and stops at a node
    with none. flag[root] = 1; untested nodes keep flag 0 and next_token -1.
    The accepted path (and the error of two flagged siblings) is the one the
    every-node form gives."""
    check_tree(parent)
    n = len(parent)
    ch = children(parent)
    flag = np.zeros(n, dtype=np.int8)
    flag[0] = 1
    nt = np.full(n, -1, dtype=np.int32)
    v = 0
    while True:
        y = int(np.argmax(t_rows[v]))
        nt[v] = y
        hits = [c for c in ch[v] if int(tokens[c]) == y]
        for c in ch[v]:
            flag[c] = 1 if c in hits else 0
        if not hits:
            return flag, nt, []
        v = hits[0]


def walk_request(t_rows, d_rows, tokens, parent, T, uniforms, replacement=False):
    """T > 0: the recursive rejection walk, without replacement (rule (c)) or,
    with replacement=True, with replacement (rule (b)).

    Returns (flag[n] int8, next_token[n] int32, log) where log lists
    (kind, node, margin) for every acceptance test with ratio < 1 ('accept'),
    every final draw ('draw') and every degenerate residual ('degenerate').
    """
    check_tree(parent)
    n = len(parent)
    ch = children(parent)
    flag = np.zeros(n, dtype=np.int8)
    flag[0] = 1
    nt = np.full(n, -1, dtype=np.int32)
    log = []
    v = 0
    while True:
        p = softmax_T(t_rows[v], T)
        q = softmax_T(d_rows[v], T)
        pres = p
        drawn = []
        accepted = None
        for c in ch[v]:
            x = int(tokens[c])
            qj = proposal_with(q, drawn) if replacement else proposal_without(q, drawn)
            ratio = acceptance_ratio(pres[x], qj[x])
            u = float(uniforms[c][0])
            if ratio < 1.0:
                log.append(("accept", c, abs(u - ratio)))
            if u < ratio:
                flag[c] = 1
                accepted = c
                break
            pres, s, degenerate = residual_update(pres, qj)
            if degenerate:
                log.append(("degenerate", c, 0.0))
            drawn.append(x)
        if accepted is not None:
            v = accepted
            continue
        y, margin = inverse_cdf(pres, float(uniforms[v][1]))
        log.append(("draw", v, margin))
        nt[v] = y
        return flag, nt, log


def tree_spec_sample(inp, replacement=False, greedy_path=False):
    """Whole batch. Returns accept_flag [T] int8, next_token [T] int32 and a
    per-request list of decision logs. replacement selects rule (b) for the
    T > 0 requests (rule (c) otherwise); greedy_path selects the T == 0 form
    that visits only the walk's nodes (greedy_walk_request) instead of every
    node (greedy_request)."""
    T_total = int(inp.node_indptr[-1])
    flags = np.zeros(T_total, dtype=np.int8)
    nts = np.full(T_total, -1, dtype=np.int32)
    logs = []
    for r in range(inp.batch):
        a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
        par = inp.parent[a:b]
        temp = float(inp.temperature[r])
        if temp == 0.0 and greedy_path:
            f, nt, log = greedy_walk_request(inp.target_logits[a:b], inp.tokens[a:b], par)
        elif temp == 0.0:
            f, nt, log = greedy_request(inp.target_logits[a:b], inp.tokens[a:b], par)
        else:
            f, nt, log = walk_request(inp.target_logits[a:b], inp.draft_logits[a:b],
                                      inp.tokens[a:b], par, temp, inp.uniforms[a:b],
                                      replacement=replacement)
        flags[a:b] = f
        nts[a:b] = nt
        logs.append(log)
    return flags, nts, logs


def near_threshold(log, eps):
    """True when any logged decision of a request lies within eps of its
    threshold (or a residual was degenerate)."""
    return any(kind == "degenerate" or m < eps for kind, _, m in log)
