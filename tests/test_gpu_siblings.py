"""GPU parity: tree_draw_siblings (HIP, via the C ABI) against the oracle.

The kernel scores in fp32 (the oracle in fp64), so a row whose oracle scores
among the first k+1 differ by less than EPS is excluded and counted; every
other row must match token for token (T = 0 rows always: no noise)."""
import numpy as np
import pytest

import oracle
from workloads import make_config

pytestmark = pytest.mark.gpu
EPS = 1e-4
KMAX = 16


def _run(logits, counts, temps, stream_id, seed):
    import torch
    import tree_verification_verify_amd as tv
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to("cuda")
    c = torch.from_numpy(np.asarray(counts, dtype=np.int32)).to("cuda")
    t = torch.from_numpy(np.asarray(temps, dtype=np.float32)).to("cuda")
    out = torch.full((logits.shape[0], KMAX), -7, dtype=torch.int32, device="cuda")
    ws = tv.alloc_workspace(4096)
    tv.tree_draw_siblings(lg, c, t, out, stream_id=stream_id, seed=seed, status_workspace=ws)
    st, bits = tv.device_status(ws)
    return out.cpu().numpy(), st, bits


def _compare(logits, counts, temps, stream_id, seed, max_excluded_frac=0.02):
    got, st, bits = _run(logits, counts, temps, stream_id, seed)
    assert st == 0, bits
    ref, gap = oracle.tree_draw_siblings(logits, counts, temps, stream_id, seed, KMAX)
    near = (gap < EPS) & (np.asarray(temps) > 0)
    ok = near | (got == ref).all(axis=1)
    assert ok.all(), np.nonzero(~ok)[0][:10]
    assert near.mean() <= max_excluded_frac, near.mean()
    return int(near.sum())


def test_highload_expansions():
    cfg = make_config("highload")
    s = cfg.sampler
    rows, counts, temps = [], [], []
    for r in range(s.batch):
        a, b = int(s.node_indptr[r]), int(s.node_indptr[r + 1])
        ch = np.bincount(s.parent[a + 1:b], minlength=b - a)
        for i in np.nonzero(ch)[0][:4]:  # a few expanded nodes per request
            rows.append(a + int(i))
            counts.append(int(ch[i]))
            temps.append(float(s.temperature[r]))
    logits = s.draft_logits[rows]
    _compare(logits, counts, temps, stream_id=3, seed=0x1234_5678_9ABC)


def test_scalar_path_ties_and_padding():
    g = np.random.default_rng(5)
    V = 1001  # not a multiple of 4: the scalar path
    logits = np.round(g.standard_normal((12, V)) * 2, 1).astype(np.float32)  # many ties
    counts = [0, 1, 2, 3, 5, 8, 16, 16, 4, 7, 1, 16]
    temps = [1.0, 0.0, 0.0, 0.5, 1.0, 0.0, 0.0, 2.0, 0.7, 0.0, 1.3, 1.0]
    _compare(logits, counts, temps, stream_id=9, seed=77)


def test_fewer_tokens_than_children():
    logits = np.array([[0.5, 2.0, -1.0], [1.0, 1.0, 1.0]], dtype=np.float32)
    logits = np.pad(logits, ((0, 0), (0, 1)), constant_values=-np.inf)[:, :3]
    got, st, _ = _run(np.ascontiguousarray(logits), [5, 3], [0.0, 0.0], 0, 0)
    assert st == 0
    assert got[0].tolist() == [1, 0, 2] + [-1] * 13
    assert got[1].tolist() == [0, 1, 2] + [-1] * 13


def test_vector_path_rows_of_many_sizes():
    g = np.random.default_rng(6)
    V = 4096 + 8
    logits = (g.standard_normal((40, V)) * 2).astype(np.float32)
    counts = g.integers(0, 17, size=40)
    temps = g.choice([0.0, 0.5, 1.0, 1.5], size=40)
    _compare(logits, counts, temps, stream_id=1, seed=2 ** 40 + 5)


@pytest.mark.parametrize("bad,bit", [("count", 32), ("temp", 4)])
def test_bad_rows_are_reported(bad, bit):
    logits = np.zeros((3, 64), dtype=np.float32)
    counts = [2, 2, 2]
    temps = [1.0, 1.0, 1.0]
    if bad == "count":
        counts[1] = 17
    else:
        temps[1] = -1.0
    got, st, bits = _run(logits, counts, temps, 0, 0)
    assert bits & bit
    assert (got[1] == -1).all()
    assert (got[0, :2] >= 0).all() and (got[2, :2] >= 0).all()
