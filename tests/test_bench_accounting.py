"""The benchmark's count of the distinct rows one decode call reads, checked against the union of
what the oracle's descent reads, query by query (keys of the candidates of every scored level,
values of the candidates a query did not keep, keys and values of the token candidates)."""
from types import SimpleNamespace

import numpy as np
import pytest

import bench
from oracle import decode, level_counts


@pytest.mark.parametrize("L,f,k,nq", [
    (300, 4, [2, 2, 2, 2], 6),        # four levels, orphans at every level, trailing tokens
    (1024, 4, [3, 1, 4, 8, 9], 5),    # mixed k; the top level is kept whole
    (37, 4, [1, 8], 4),               # level 2 kept whole
    (64, 4, [0, 2, 2], 3),            # k = 0 at level 1: its candidates are all entries
    (3, 4, [], 3),                    # fewer tokens than the fanout: dense
])
def test_unique_rows_match_the_oracle_union(L, f, k, nq):
    B, Hkv, G, d = 2, 2, 2, 8
    rng = np.random.default_rng(L + nq)
    K = rng.standard_normal((B, Hkv, L, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, L, d)).astype(np.float32)
    q = rng.standard_normal((B, nq, Hkv * G, d)).astype(np.float32)
    W = (np.eye(d) + 0.05 * rng.standard_normal((d, d))).astype(np.float32)
    res = decode(K, V, W, q, L, f, k, "f32", theta=1.0e4)
    T = len(level_counts(L, f))
    sel = -np.ones((B, nq, Hkv, T, max(k + [1])), np.int32)
    keys, vals, toks = {}, {}, {}
    for (b, j, h), u in res.items():
        for lv in range(1, T + 1):
            kept = u.sel.get(lv, [])
            sel[b, j, h, lv - 1, :len(kept)] = kept
            ents = {i for (l, i) in u.entries if l == lv}
            if min(k[lv - 1], u.C[lv]) < u.C[lv]:
                keys.setdefault((b, h, lv), set()).update(kept, ents)
            vals.setdefault((b, h, lv), set()).update(ents)
        toks.setdefault((b, h), set()).update(i for (l, i) in u.entries if l == 0)
    rows = sum(map(len, keys.values())) + sum(map(len, vals.values())) + 2 * sum(map(len, toks.values()))
    w = SimpleNamespace(f=f, L=L, d=d, elem_bytes=4)
    assert bench.decode_unique_bytes(w, k, sel) == rows * d * 4


def test_bench_refuses_more_than_one_gpu():
    """--gpus above 1 ends with a message and exit status 2 before any GPU work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
