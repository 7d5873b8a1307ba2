"""Host-side checks of the figures bench.py reports (no GPU needed): the
algorithmic byte counts it divides by kernel time, the rule that keeps a
stale HBM traffic figure out of its line, and the one-GPU guard."""
import hashlib
import json
import os
import re
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_config  # noqa: E402

HIGHLOAD_ATTN_BYTES = 1_238_102_016  # 1.238 GB per launch, the figure the roofline uses


def test_attention_bytes_of_the_highload_batch():
    inp = make_config("highload", sampler=False).attn
    assert inp.dtype == "bf16" and (inp.num_q_heads, inp.num_kv_heads, inp.head_dim) == (32, 8, 128)
    # counted from the request arrays: every key of every request (prefix and
    # tree rows) read once per kv head as K and V, every tree row's Q read and
    # O written, two bytes each
    nodes = np.diff(inp.node_indptr.astype(np.int64))
    keys = inp.prefix_len.astype(np.int64) + nodes
    kv = int(keys.sum()) * 8 * 128 * 2 * 2
    qo = int(nodes.sum()) * 32 * 128 * 2 * 2
    assert kv + qo == HIGHLOAD_ATTN_BYTES
    assert bench.attn_algorithmic_bytes(inp) == HIGHLOAD_ATTN_BYTES
    assert int(nodes.sum()) == 1216 and inp.batch == 64


def test_sampler_bytes_hand_case():
    V = 1000
    s = SimpleNamespace(vocab=V, batch=3, node_indptr=np.array([0, 5, 9, 12]),
                        temperature=np.array([0.0, 1.0, 0.5], np.float32))
    out_len = np.array([2, 3, 1])
    # T = 0: every target row (5) or the two visited; T > 0: both rows of
    # each visited node (3 and 1)
    assert bench.sampler_algorithmic_bytes(s, out_len) == (5 + 2 * 3 + 2 * 1) * V * 4
    assert bench.sampler_algorithmic_bytes(s, out_len, greedy_path=True) == (2 + 2 * 3 + 2 * 1) * V * 4


def test_traffic_is_reported_only_for_the_measured_kernel_source():
    text = open(bench.PROFILE_COUNTERS).read()
    recorded = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text).group(1)
    current = hashlib.sha256(open(bench.ATTN_SOURCE, "rb").read()).hexdigest()
    traffic = bench.read_traffic()
    assert (traffic is not None) == (recorded == current)
    if traffic is not None:
        # the counters' bytes per launch sit a few percent above the
        # algorithmic bytes (partial pages, merge partials)
        assert 1.0 <= traffic / HIGHLOAD_ATTN_BYTES <= 1.1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
