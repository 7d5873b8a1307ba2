"""GPU parity: tree_spec_sample + tree_accept_path (HIP, via the C ABI)
against the fp64 oracle. Decisions are bit-exact; a request whose oracle log
holds a decision within EPS of its threshold (or a degenerate residual) is
excluded from the bit-exact comparison and counted. EPS is the specification's
band, 1e-6: the GPU sums the vocabulary from fp32 exps (fp64 arguments and
accumulation, ~1.5e-7 relative per term) and takes every single decision
value in fp64, so its decision values lie within ~1e-7 of the oracle's."""
import numpy as np
import pytest

import oracle
from oracle.sampler import near_threshold
from workloads import make_config, make_sampler_inputs, random_tree, chain_tree, star_tree

pytestmark = pytest.mark.gpu

EPS = 1e-6   # the near-threshold band of the specification


def _run(inp, **kw):
    from gpu_run import run_sampler
    return run_sampler(inp, **kw)


def near_kind(log, eps):
    """How a request's decisions sit against the band: "accept" when an
    acceptance test lies within eps of its ratio (or a residual degenerated),
    "draw" when only the final draw lies within eps of a boundary, None."""
    if any(k == "degenerate" or (k == "accept" and m < eps) for k, _, m in log):
        return "accept"
    if any(k == "draw" and m < eps for k, _, m in log):
        return "draw"
    return None


def compare_walk(inp, got, flags, nts, logs, pn, ot, ol, kk):
    """Bit-exact comparison; a request with a near acceptance test is skipped
    whole, one whose only near decision is the final draw is compared on
    everything upstream of the draw (flags, path, keep-list, emitted tokens
    but the last). Returns (skipped, draw_only)."""
    skipped = draw_only = 0
    for r in range(inp.batch):
        a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
        kind = near_kind(logs[r], EPS)
        if kind == "accept":
            skipped += 1
            continue
        np.testing.assert_array_equal(got["flag"][a:b], flags[a:b], err_msg=f"request {r}")
        assert got["out_len"][r] == ol[r], r
        np.testing.assert_array_equal(got["path_nodes"][r], pn[r])
        np.testing.assert_array_equal(got["kv_keep"][r], kk[r])
        n = int(ol[r])
        if kind == "draw":
            draw_only += 1
            stop = int(pn[r][n - 1])
            keep = np.ones(b - a, bool)
            keep[stop] = False
            np.testing.assert_array_equal(got["next_token"][a:b][keep], nts[a:b][keep], err_msg=f"request {r}")
            np.testing.assert_array_equal(got["out_tokens"][r][:n - 1], ot[r][:n - 1])
            assert 0 <= got["out_tokens"][r][n - 1] < inp.vocab
        else:
            np.testing.assert_array_equal(got["next_token"][a:b], nts[a:b], err_msg=f"request {r}")
            np.testing.assert_array_equal(got["out_tokens"][r], ot[r])
    return skipped, draw_only


def _compare(inp, got, prefix_lens=None, allow_near=0, replacement=False, draw_near=None,
             greedy_path=False):
    """allow_near: requests with a near acceptance test (skipped); draw_near:
    the expected number whose only near decision is the draw (None: any)."""
    assert got["status"] == 0, (got["status"], got["bits"])
    flags, nts, logs = oracle.tree_spec_sample(inp, replacement=replacement, greedy_path=greedy_path)
    md = got["max_depth"]
    B = inp.batch
    prefix_lens = prefix_lens if prefix_lens is not None else [0] * B
    pn, ot, ol, kk = oracle.tree_accept_path(inp.node_indptr, inp.parent, inp.tokens, flags,
                                             nts, prefix_lens, md)
    skipped, draw_only = compare_walk(inp, got, flags, nts, logs, pn, ot, ol, kk)
    assert skipped <= allow_near, skipped
    if draw_near is not None:
        assert draw_only == draw_near, draw_only
    return skipped


def test_tiny():
    cfg = make_config("tiny", attention=False)
    _compare(cfg.sampler, _run(cfg.sampler, max_depth=5, prefix_lens=cfg.prefix_lens),
             cfg.prefix_lens)


# draw_near: requests whose final draw lands within the band of a boundary
# (tail tokens of probability below ~2e-6); counted by the oracle alone.
@pytest.mark.parametrize("temp,draw_near", [("mixed", 2), (0.0, 0), (0.5, 1), (1.0, 9)])
def test_highload_full_vocab(temp, draw_near):
    cfg = make_config("highload", attention=False, temperature=temp)
    _compare(cfg.sampler, _run(cfg.sampler, max_depth=8, prefix_lens=cfg.prefix_lens),
             cfg.prefix_lens, draw_near=draw_near)


# Greedy requests along the walk only (TV_GREEDY_PATH): every output the
# walk writes is compared, and the untouched nodes' defaults too.
@pytest.mark.parametrize("temp", [0.0, "mixed"])
def test_highload_greedy_path(temp):
    cfg = make_config("highload", attention=False, temperature=temp)
    got = _run(cfg.sampler, max_depth=8, prefix_lens=cfg.prefix_lens, greedy_path=True)
    _compare(cfg.sampler, got, cfg.prefix_lens, draw_near=None, greedy_path=True)
    if temp == 0.0:
        # the walk tests only the children of visited nodes: most rows untouched
        assert (got["next_token"] == -1).sum() > cfg.sampler.node_indptr[-1] // 2


@pytest.mark.parametrize("V", [7, 64, 1000, 4099])
@pytest.mark.parametrize("batch", [1, 5, 40])
def test_greedy_path_random_small(V, batch):
    """Random trees, mostly greedy requests, children drawn from correlated
    draft rows so that walks go deep; V = 7 and 4099 take the unvectorised
    loads."""
    rng = np.random.default_rng(1000 + V + batch)
    trees = [random_tree(rng, int(rng.integers(1, min(25, V + 1) + 1)),
                         depth_cap=int(rng.integers(1, 6)))
             for _ in range(batch)]
    temps = rng.choice([0.0, 0.0, 0.0, 0.5, 1.0], size=batch)
    inp = make_sampler_inputs(rng, rng, rng, trees, V, temps, mode="correlated")
    _compare(inp, _run(inp, max_depth=6, greedy_path=True), greedy_path=True)


def test_greedy_path_ties_and_a_bad_parent():
    """Ties take the lowest index along the walk, as in the every-node form;
    a parent link that breaks the order is reported (status TV_DEV_TREE)."""
    V = 50
    trees = [star_tree(6), chain_tree(4)]
    rng = np.random.default_rng(0)
    inp = make_sampler_inputs(rng, rng, rng, trees, V, [0.0, 0.0])
    inp.target_logits[:] = 0.0
    inp.target_logits[:, 7] = 3.0
    inp.target_logits[:, 31] = 3.0   # tie with 7: argmax must be 7
    inp.tokens[:] = [0, 9, 31, 7, 2, 5, 0, 7, 7, 1]
    got = _run(inp, max_depth=6, greedy_path=True)
    _compare(inp, got, greedy_path=True)
    assert list(got["out_len"]) == [2, 3]
    inp.parent[8] = 2   # node 2 of the chain names itself
    got = _run(inp, max_depth=6, greedy_path=True)
    assert got["bits"] & 1, got["bits"]   # TV_DEV_TREE


def test_highload_independent_logits():
    """The literal independent N(0,2) reading: short walks, many rejections."""
    cfg = make_config("highload", attention=False, temperature=1.0, mode="independent", batch=16)
    _compare(cfg.sampler, _run(cfg.sampler, max_depth=8))


def test_sequoia_sampler():
    cfg = make_config("sequoia", attention=False)
    _compare(cfg.sampler, _run(cfg.sampler, max_depth=12, prefix_lens=cfg.prefix_lens),
             cfg.prefix_lens)


@pytest.mark.parametrize("V", [7, 64, 1000, 4099])
@pytest.mark.parametrize("batch", [1, 5, 40])
def test_random_small(V, batch):
    rng = np.random.default_rng(V + batch)
    # at most V children per node: a node cannot have more distinct siblings than tokens
    trees = [random_tree(rng, int(rng.integers(1, min(25, V + 1) + 1)),
                         depth_cap=int(rng.integers(1, 6)))
             for _ in range(batch)]
    temps = rng.choice([0.0, 0.25, 0.5, 1.0, 2.0], size=batch)
    mode = "independent" if V < 100 else "correlated"
    inp = make_sampler_inputs(rng, rng, rng, trees, V, temps, mode=mode)
    _compare(inp, _run(inp, max_depth=6))


def test_greedy_ties_take_lowest_index():
    V = 50
    trees = [star_tree(6), chain_tree(4)]
    rng = np.random.default_rng(0)
    inp = make_sampler_inputs(rng, rng, rng, trees, V, [0.0, 0.0])
    inp.target_logits[:] = 0.0
    inp.target_logits[:, 7] = 3.0
    inp.target_logits[:, 31] = 3.0   # tie with 7: argmax must be 7
    inp.tokens[:] = [0, 9, 31, 7, 2, 5, 0, 7, 7, 1]
    got = _run(inp, max_depth=4)
    assert (got["next_token"] == 7).all()
    _compare(inp, got)


def test_alignment_probe():
    """Row i is the distribution after node i: a one-hot target row on the
    token only one child carries makes that child accepted."""
    V = 128
    trees = [np.array([-1, 0, 0, 1, 2])]
    rng = np.random.default_rng(1)
    inp = make_sampler_inputs(rng, rng, rng, trees, V, [1.0])
    inp.tokens[:] = [0, 5, 7, 3, 9]
    inp.target_logits[:] = -30.0
    inp.target_logits[0, 7] = 30.0
    inp.target_logits[2, 9] = 30.0
    inp.target_logits[[1, 3, 4], 11] = 30.0
    got = _run(inp, max_depth=3)
    assert list(got["flag"]) == [1, 0, 1, 0, 1]
    assert got["out_len"][0] == 3
    _compare(inp, got)


def test_q_equals_p_accepts_first_child():
    rng = np.random.default_rng(2)
    trees = [random_tree(rng, 20, depth_cap=4) for _ in range(10)]
    inp = make_sampler_inputs(rng, rng, rng, trees, 512, [1.0] * 10)
    inp.draft_logits = inp.target_logits.copy()
    inp.uniforms = (inp.uniforms * np.float32(0.999)).astype(np.float32)
    got = _run(inp, max_depth=4)
    _compare(inp, got)
    for r, t in enumerate(trees):
        a = int(inp.node_indptr[r])
        for v in range(len(t)):
            ch = [i for i in range(len(t)) if t[i] == v]
            if ch and got["flag"][a + v] == 1:
                assert got["flag"][a + ch[0]] == 1


def test_two_accepted_siblings_reported():
    """tree_accept_path flags a node with two accepted children (host-forced flags)."""
    import torch
    import tree_verification_verify_amd as tv
    ni = torch.tensor([0, 3, 6], dtype=torch.int32, device="cuda")
    par = torch.tensor([-1, 0, 0, -1, 0, 1], dtype=torch.int32, device="cuda")
    tok = torch.tensor([0, 4, 5, 0, 6, 7], dtype=torch.int32, device="cuda")
    flag = torch.tensor([1, 1, 1, 1, 1, 1], dtype=torch.int8, device="cuda")
    nt = torch.tensor([-1, 11, 12, -1, -1, 13], dtype=torch.int32, device="cuda")
    pre = torch.tensor([10, 20], dtype=torch.int32, device="cuda")
    desc = tv.sample_desc(2, 16, 3, 2)
    ws = tv.alloc_workspace(tv.sample_workspace_size(desc))
    pn = torch.empty(6, dtype=torch.int32, device="cuda")
    ot, kk = torch.empty_like(pn), torch.empty_like(pn)
    ol = torch.empty(2, dtype=torch.int32, device="cuda")
    tv.tree_accept_path(2, 2, ni, par, tok, flag, nt, pre, pn, ot, ol, kk, ws)
    st, bits = tv.device_status(ws)
    assert st == 9 and bits & 8
    assert ol.cpu().tolist() == [-1, 3]
    assert ot.cpu().tolist()[3:] == [6, 7, 13]
    assert kk.cpu().tolist()[3:] == [20, 21, 22]


def test_monte_carlo_tv_on_gpu():
    """P10 on the GPU path: 3000 independent one-level walks (root with 3
    children drawn without replacement); the first emitted token's TV to p is
    within the 99th percentile of direct sampling's TV at equal n."""
    rng = np.random.default_rng(11)
    V, k, n = 16, 3, 3000
    logits = (rng.standard_normal(V) * 1.2).astype(np.float32)
    dl = (logits + rng.standard_normal(V).astype(np.float32) * 0.4).astype(np.float32)
    trees = [star_tree(k + 1)] * n
    inp = make_sampler_inputs(rng, rng, rng, trees, V, [1.0] * n)
    inp.target_logits[:] = logits
    inp.draft_logits[:] = dl
    from workloads import gumbel_topk_tokens
    for r in range(n):
        inp.tokens[r * (k + 1) + 1:(r + 1) * (k + 1)] = gumbel_topk_tokens(rng, dl, k, 1.0)
    got = _run(inp, max_depth=1)
    first = got["out_tokens"][:, 0]
    p = np.exp(logits.astype(np.float64) - logits.max())
    p /= p.sum()
    tv_walk = 0.5 * np.abs(np.bincount(first, minlength=V) / n - p).sum()
    tvs = [0.5 * np.abs(rng.multinomial(n, p) / n - p).sum() for _ in range(300)]
    assert tv_walk <= np.percentile(tvs, 99), (tv_walk, np.percentile(tvs, 99))
    _compare(inp, got)


def _subset(inp, idx):
    """Requests idx of a batch, in that order (repeats allowed)."""
    from workloads.inputs import SamplerInputs
    rows, ind = [], [0]
    for r in idx:
        a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
        rows.append(np.arange(a, b))
        ind.append(ind[-1] + b - a)
    rr = np.concatenate(rows)
    return SamplerInputs(vocab=inp.vocab, target_logits=inp.target_logits[rr],
                         draft_logits=None if inp.draft_logits is None else inp.draft_logits[rr],
                         tokens=inp.tokens[rr], node_indptr=np.asarray(ind, np.int32),
                         parent=inp.parent[rr], temperature=inp.temperature[list(idx)],
                         uniforms=inp.uniforms[rr])


def test_workspace_reused_across_calls():
    """One workspace, calls of different batch sizes (so different team
    sizes and request-to-slot maps) back to back: the team exchange must
    never take a word left by an earlier call for a current one."""
    import tree_verification_verify_amd as tv
    cfg = make_config("highload", attention=False)
    big = cfg.sampler
    rng = np.random.default_rng(5)
    trees = [random_tree(rng, int(rng.integers(2, 20)), depth_cap=5) for _ in range(200)]
    many = make_sampler_inputs(rng, rng, rng, trees, 2048, rng.choice([0.5, 1.0], size=200))
    desc = tv.sample_desc(200, big.vocab, big.max_nodes, 8)
    ws = tv.alloc_workspace(tv.sample_workspace_size(desc))
    for inp in [big, _subset(big, [46, 19, 3]), many, big, big, _subset(big, list(range(63, -1, -1)))]:
        _compare(inp, _run(inp, max_depth=8, ws=ws))
    # both greedy forms and the walk, alternating on the same workspace
    for gp in (True, False, True, True, False):
        for inp in (big, _subset(big, [5, 60, 33, 2])):
            _compare(inp, _run(inp, max_depth=8, ws=ws, greedy_path=gp), greedy_path=gp)


def test_streamed_slices():
    """A vocabulary whose per-member slice exceeds the resident capacity
    (the streamed passes), with 4-aligned rows."""
    rng = np.random.default_rng(9)
    trees = [random_tree(rng, n, depth_cap=4) for n in (9, 14, 5)]
    inp = make_sampler_inputs(rng, rng, rng, trees, 262144, [1.0, 0.5, 1.0], noise=1.0)
    _compare(inp, _run(inp, max_depth=4))


def test_more_children_than_listed():
    """A root with 150 children: the per-visit child list holds 64, the rest
    are found by scanning; independent logits force long rejection runs."""
    rng = np.random.default_rng(12)
    inp = make_sampler_inputs(rng, rng, rng, [star_tree(151), star_tree(90)], 4096, [1.0, 2.0],
                              mode="independent")
    _compare(inp, _run(inp, max_depth=1))


@pytest.mark.parametrize("V", [8192, 8196, 151936])
def test_greedy_split_rows_and_ties(V):
    """T = 0 with rows split over team members (trees with fewer rows than the
    team): equal maxima in different chunks and members resolve to the lowest
    index, and the last logit of a partial final chunk can win."""
    rng = np.random.default_rng(V)
    trees = [chain_tree(1), chain_tree(2), random_tree(rng, 5, depth_cap=3), random_tree(rng, 23, depth_cap=6)]
    inp = make_sampler_inputs(rng, rng, rng, trees, V, [0.0] * 4)
    t = inp.target_logits
    t[0, [100, V // 2 + 3, V - 5]] = 40.0          # ties: lowest index wins
    t[1, V - 1] = 40.5                              # last logit of the row
    t[2, [V - 1, V - 2]] = 40.0                     # tie at the row end
    t[3:, [17, V - 17]] = 40.0
    got = _run(inp, max_depth=6)
    assert got["next_token"][0] == 100
    assert got["next_token"][1] == V - 1
    _compare(inp, got)


# ---- the with-replacement rule (survey page, Taxonomy rule (b)) ----------


@pytest.mark.parametrize("temp,draw_near", [("mixed", 0), (1.0, 8)])
def test_highload_with_replacement(temp, draw_near):
    cfg = make_config("highload", attention=False, temperature=temp, draws="with")
    inp = cfg.sampler
    _compare(inp, _run(inp, max_depth=8, prefix_lens=cfg.prefix_lens, replacement=True),
             cfg.prefix_lens, replacement=True, draw_near=draw_near)


@pytest.mark.parametrize("V", [3, 7, 64, 1000])
def test_random_small_with_replacement(V):
    """Small vocabularies make repeated siblings common, and more children
    than tokens possible (so no T = 0 request here: greedy exact match needs
    distinct siblings)."""
    rng = np.random.default_rng(300 + V)
    trees = [random_tree(rng, int(rng.integers(1, 25)), depth_cap=int(rng.integers(1, 6)))
             for _ in range(40)]
    temps = rng.choice([0.25, 0.5, 1.0, 2.0], size=40)
    inp = make_sampler_inputs(rng, rng, rng, trees, V, temps,
                              mode="independent" if V < 100 else "correlated", draws="with")
    repeats = 0
    for r in range(inp.batch):
        a, b = int(inp.node_indptr[r]), int(inp.node_indptr[r + 1])
        par, tok = inp.parent[a:b], inp.tokens[a:b]
        for v in range(b - a):
            kids = tok[par == v]
            repeats += len(set(kids.tolist())) < len(kids)
    assert repeats > 0  # the repeated-token case is exercised
    _compare(inp, _run(inp, max_depth=6, replacement=True), replacement=True)


def test_rules_differ_on_the_same_draws():
    """The same without-replacement draws under both rules on a vocabulary
    small enough that the drawn siblings hold much of q's mass (on a large
    vocabulary the two proposals nearly coincide): the kernel follows the rule
    it is given (each side against its own oracle rule)."""
    rng = np.random.default_rng(21)
    trees = [random_tree(rng, int(rng.integers(4, 25)), depth_cap=4) for _ in range(64)]
    inp = make_sampler_inputs(rng, rng, rng, trees, 8, [1.0] * 64, mode="independent")
    a = _run(inp, max_depth=4, replacement=False)
    b = _run(inp, max_depth=4, replacement=True)
    _compare(inp, a, replacement=False)
    _compare(inp, b, replacement=True)
    assert (a["flag"] != b["flag"]).any() or (a["next_token"] != b["next_token"]).any()


def test_more_children_than_listed_with_replacement():
    """150 independent draws at the root (past the per-visit list of 64)."""
    rng = np.random.default_rng(13)
    inp = make_sampler_inputs(rng, rng, rng, [star_tree(151), star_tree(90)], 4096, [1.0, 2.0],
                              mode="independent", draws="with")
    _compare(inp, _run(inp, max_depth=1, replacement=True), replacement=True)


def test_monte_carlo_tv_with_replacement_on_gpu():
    """Rule (b) on the GPU path: 3000 one-level walks, root with 3 independent
    draws from q; the first emitted token's TV to p is within the 99th
    percentile of direct sampling's TV at equal n."""
    rng = np.random.default_rng(17)
    V, k, n = 16, 3, 3000
    logits = (rng.standard_normal(V) * 1.2).astype(np.float32)
    dl = (logits + rng.standard_normal(V).astype(np.float32) * 0.4).astype(np.float32)
    inp = make_sampler_inputs(rng, rng, rng, [star_tree(k + 1)] * n, V, [1.0] * n)
    inp.target_logits[:] = logits
    inp.draft_logits[:] = dl
    from workloads import independent_draw_tokens
    for r in range(n):
        inp.tokens[r * (k + 1) + 1:(r + 1) * (k + 1)] = independent_draw_tokens(rng, dl, k, 1.0)
    got = _run(inp, max_depth=1, replacement=True)
    first = got["out_tokens"][:, 0]
    p = np.exp(logits.astype(np.float64) - logits.max())
    p /= p.sum()
    tv_walk = 0.5 * np.abs(np.bincount(first, minlength=V) / n - p).sum()
    tvs = [0.5 * np.abs(rng.multinomial(n, p) / n - p).sum() for _ in range(300)]
    assert tv_walk <= np.percentile(tvs, 99), (tv_walk, np.percentile(tvs, 99))
    _compare(inp, got, replacement=True)


@pytest.mark.parametrize("replacement", [False, True])
def test_topk_siblings_are_biased_on_gpu(replacement):
    """The biased control ([TreeSpark §5.4, Table 9]): siblings fixed to the
    top 3 of q instead of drawn. With q = p on a diffuse target, the first
    candidate is always accepted, so the walk emits the argmax: its TV to p
    is far above direct sampling's at equal n (and the GPU still matches the
    oracle decision for decision)."""
    rng = np.random.default_rng(23)
    V, k, n = 16, 3, 3000
    logits = (rng.standard_normal(V) * 0.5).astype(np.float32)
    inp = make_sampler_inputs(rng, rng, rng, [star_tree(k + 1)] * n, V, [1.0] * n)
    inp.target_logits[:] = logits
    inp.draft_logits[:] = logits
    top = np.argsort(-logits.astype(np.float64), kind="stable")[:k].astype(np.int32)
    for r in range(n):
        inp.tokens[r * (k + 1) + 1:(r + 1) * (k + 1)] = top
    got = _run(inp, max_depth=1, replacement=replacement)
    p = np.exp(logits.astype(np.float64) - logits.max())
    p /= p.sum()
    first = got["out_tokens"][:, 0]
    tv_walk = 0.5 * np.abs(np.bincount(first, minlength=V) / n - p).sum()
    tvs = [0.5 * np.abs(rng.multinomial(n, p) / n - p).sum() for _ in range(300)]
    print(f"top-k control TV {tv_walk:.3f}, direct sampling 99th percentile "
          f"{np.percentile(tvs, 99):.3f}, 1 - max p {1 - p.max():.3f}")
    assert tv_walk > 5 * np.percentile(tvs, 99)
    assert abs(tv_walk - (1 - p.max())) < 1e-9  # the argmax every time
    _compare(inp, got, replacement=replacement)


@pytest.mark.parametrize("temp,greedy_path", [(1.0, False), (0.0, False), (0.0, True)])
def test_team_wait_gives_up_when_forced_from_the_host(temp, greedy_path, monkeypatch):
    """A team wait limit of 0 (set from the host for these launches only)
    makes the exchange (T > 0, and the greedy walk's argmax exchange) and the
    greedy barrier (T = 0, every node) give up at once: the kernel still ends
    normally and reports TV_DEV_TIMEOUT (status 10). Each run uses a fresh
    workspace."""
    cfg = make_config("highload", attention=False, batch=32, vocab=8192, temperature=temp)
    monkeypatch.setenv("TREEVERIFY_TEAM_WAIT_US", "0")
    got = _run(cfg.sampler, max_depth=8, greedy_path=greedy_path)
    monkeypatch.delenv("TREEVERIFY_TEAM_WAIT_US")
    assert got["bits"] & (1 << 4) and got["status"] == 10, (got["bits"], got["status"])
    # the default limit again: a fresh workspace verifies normally
    _compare(cfg.sampler, _run(cfg.sampler, max_depth=8, greedy_path=greedy_path), greedy_path=greedy_path)
