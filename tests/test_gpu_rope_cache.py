"""The RoPE table cache: calls that take their table from the library's per-device cache give bit
for bit what calls that fill their own table give.

The cache holds the first (head size, theta) that a call uses on the GPU; these tests use the
benchmark workloads' (d = 128, theta = 1e6). Each call runs with the cache allowed and with it
turned off (RECSA_ROPE_CACHE=0: every call fills its own table), on a workspace filled with NaN
(a call that reads the cache never looks at it; one that fills its own table overwrites it), and
decoding is also compared with recsa_decode_noalloc, which always fills its own table."""
import os

import numpy as np
import pytest
import torch

from gpu_util import dev_tensor
from long_context_hierarchical_amd import recsa as R
from synthetic import Workload, gen_decode_inputs

pytestmark = pytest.mark.gpu


class _cache:
    def __init__(self, on):
        self.on = on

    def __enter__(self):
        self.old = os.environ.get("RECSA_ROPE_CACHE")
        os.environ["RECSA_ROPE_CACHE"] = "1" if self.on else "0"

    def __exit__(self, *exc):
        if self.old is None:
            del os.environ["RECSA_ROPE_CACHE"]
        else:
            os.environ["RECSA_ROPE_CACHE"] = self.old


def _setup(L, n_q, seed, B=2):
    w = Workload("rope_cache", B=B, Hq=8, Hkv=2, d=128, dtype="bf16", L=L, f=16, k=8, n_queries=n_q, mode="decode",
                 std=128 ** -0.5, seed=seed)
    inp = gen_decode_inputs(w)
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
    K, V, W, q = (dev_tensor(inp[x], w.dtype) for x in ("K", "V", "W", "q"))
    tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device="cuda")
    R.recsa_build_tree(sh, K, V, W, 0, w.L, tree)
    return w, sh, K, V, W, q, tree


def _nan_ws(sh, n, k):
    nbytes = max(R.recsa_workspace_bytes(sh, n, k), 16)
    return torch.full((nbytes // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")


def _outs(B, n_q, Hq, d):
    out = torch.full((B, n_q, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, n_q, Hq), float("nan"), dtype=torch.float32, device="cuda")
    return out, lse


def _np(*ts):
    # bf16 tensors (the caches) as their bits
    torch.cuda.synchronize()
    return tuple((t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy() for t in ts)


def test_decode_cached_table_matches_own_table():
    w, sh, K, V, W, q, tree = _setup(16 ** 3 * 3 + 201, 5, 71)
    for n, kk in ((w.L, 8), (2000, 4), (w.L - 1, 16)):
        k = [kk] * R.recsa_num_levels(n, w.f)
        res = []
        for mode in ("on", "off", "noalloc"):
            out, lse = _outs(w.B, w.n_queries, w.Hq, w.d)
            with _cache(mode == "on"):
                if mode == "noalloc":
                    R.recsa_decode_noalloc(sh, q, K, V, tree, n, k, out, lse, None, 0)
                else:
                    R.recsa_decode(sh, q, K, V, tree, n, k, out, lse, None, 0, _nan_ws(sh, n, k))
            res.append(_np(out, lse))
        assert np.isfinite(res[0][0]).all() and np.isfinite(res[0][1]).all(), n
        for other in res[1:]:
            assert np.array_equal(res[0][0], other[0]) and np.array_equal(res[0][1], other[1]), n


def test_prefill_cached_table_matches_own_table():
    w, sh, K, V, W, q, tree = _setup(9000, 9000, 72)
    k = [8] * R.recsa_num_levels(w.L, w.f)
    n_q = 300
    q_start = w.L - n_q
    qs = q[:, q_start:].contiguous()
    res = []
    for on in (True, False, True):
        out, lse = _outs(w.B, n_q, w.Hq, w.d)
        with _cache(on):
            R.recsa_prefill(sh, qs, q_start, K, V, tree, k, out, lse, None, 0, _nan_ws(sh, w.L, k))
        res.append(_np(out, lse))
    assert np.isfinite(res[0][0]).all()
    for other in res[1:]:
        assert np.array_equal(res[0][0], other[0]) and np.array_equal(res[0][1], other[1])


def test_decode_step_cached_table_matches_own_table():
    """Eight decoding steps from the same cache contents, with the cache allowed and turned off:
    caches, tree and outputs bit for bit."""
    w, sh, K, V, W, q, tree = _setup(16 ** 3 + 16 * 5 - 4, 8, 73, B=1)
    n0 = w.L - 8
    # the tree as it stands at n0 tokens, on a copy of the caches
    runs = []
    for on in (True, False):
        Kc, Vc = K.clone(), V.clone()
        tr = torch.zeros_like(tree)
        R.recsa_build_tree(sh, Kc, Vc, W, 0, n0, tr)
        outs = []
        for t in range(n0, w.L):
            k = [8] * R.recsa_num_levels(t + 1, w.f)
            out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
            lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
            with _cache(on):
                R.recsa_decode_step(sh, q[:, t - n0].contiguous(), K[:, :, t].contiguous(), V[:, :, t].contiguous(),
                                    Kc, Vc, W, tr, t, k, out, lse, None, 0, _nan_ws(sh, t + 1, k))
            outs.append(_np(out, lse))
        runs.append((outs, _np(Kc, Vc, tr)))
    for (a, b) in zip(runs[0][0], runs[1][0]):
        assert np.isfinite(a[0]).all()
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for x, y in zip(runs[0][1], runs[1][1]):
        assert np.array_equal(x, y)


_TWO_STREAMS = r'''
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[1] + "/tests")
from long_context_hierarchical_amd import recsa as R
from gpu_util import dev_tensor
from synthetic import Workload, gen_decode_inputs
w = Workload("rope_cache_streams", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", L=16 ** 3 * 2 + 33, f=16, k=8,
             n_queries=3, mode="decode", std=128 ** -0.5, seed=74)
inp = gen_decode_inputs(w)
sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
K, V, W, q = (dev_tensor(inp[x], w.dtype) for x in ("K", "V", "W", "q"))
tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device="cuda")
R.recsa_build_tree(sh, K, V, W, 0, w.L, tree)
k = [8] * R.recsa_num_levels(w.L, w.f)
nb = max(R.recsa_workspace_bytes(sh, w.L, k), 16)
torch.cuda.synchronize()
s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
outs = []
for _ in range(2):
    ws = torch.full((nb // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    o = torch.full((w.B, w.n_queries, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((w.B, w.n_queries, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
    outs.append((o, l, ws))
torch.cuda.synchronize()
# the first call fills the process's cache on s1; the second, issued at once on s2, must wait for
# that fill (or find it complete)
for s, (o, l, ws) in zip((s1, s2), outs):
    R.recsa_decode(sh, q, K, V, tree, w.L, k, o, l, None, 0, ws, stream=s)
torch.cuda.synchronize()
ref_o = torch.full_like(outs[0][0], float("nan")); ref_l = torch.full_like(outs[0][1], float("nan"))
R.recsa_decode_noalloc(sh, q, K, V, tree, w.L, k, ref_o, ref_l, None, 0)
torch.cuda.synchronize()
for o, l, _ in outs:
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
print("ok", flush=True)
'''


def test_first_fill_on_one_stream_and_a_call_on_another(tmp_path):
    """In a fresh process: the first call fills the cache on one stream and a call issued right
    after on another stream reads it; both give bit for bit what a call filling its own table
    gives."""
    import subprocess
    import sys
    script = tmp_path / "two_streams.py"
    script.write_text(_TWO_STREAMS)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    env.pop("RECSA_ROPE_CACHE", None)
    r = subprocess.run([sys.executable, str(script), root], capture_output=True, text=True, timeout=180, env=env)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


def test_decode_captured_in_a_graph_reads_the_cache():
    """A decode captured in a HIP graph once the cache is complete: every replay (with eager work
    and synchronisations between them) equals the eager call bit for bit."""
    w, sh, K, V, W, q, tree = _setup(16 ** 3 * 2 + 77, 4, 75)
    k = [8] * R.recsa_num_levels(w.L, w.f)
    ws = _nan_ws(sh, w.L, k)
    out, lse = _outs(w.B, w.n_queries, w.Hq, w.d)
    R.recsa_decode(sh, q, K, V, tree, w.L, k, out, lse, None, 0, ws)
    ref = _np(out, lse)
    g = torch.cuda.CUDAGraph()
    gout, glse = _outs(w.B, w.n_queries, w.Hq, w.d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        R.recsa_decode(sh, q, K, V, tree, w.L, k, gout, glse, None, 0, ws)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        R.recsa_decode(sh, q, K, V, tree, w.L, k, gout, glse, None, 0, ws)
    for rep in range(3):
        gout.fill_(float("nan"))
        glse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _np(gout, glse)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), rep
        # eager work between the replays
        R.recsa_decode(sh, q, K, V, tree, w.L, k, out, lse, None, 0, ws)
        torch.cuda.synchronize()
