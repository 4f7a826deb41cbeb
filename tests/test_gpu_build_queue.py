"""The tree build's two launch forms and its tile queue. A build call whose level-1 launch has at
most one tile per CU runs every launch as one 1024-thread workgroup per tile; any other runs the
persistent kernel, which hands a launch's later tiles out through a counter, in the order the
workgroups ask for them. Which workgroup builds a tile does
not change how it is built, so a tree built through the queue must equal, bit for bit, the tree
built with the tiles in the static order (RECSA_BUILD_QUEUE=0), whatever the increments, and
with builds running at once on several streams (more of them than there are queues) or replayed
from a HIP graph. The full-size tests compare queue-built trees of 131K-2M tokens with the
oracle; here one slice of each shape is compared with the oracle too, and trees built in small
increments (every launch in the one-tile form) are compared with one-shot builds.

Inputs are seeded normal rows generated on the device (K, V at scale d^-1/2, W = I + noise)."""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import storage_bits
from long_context_hierarchical_amd import recsa as R

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


class _queue:
    def __init__(self, on):
        self.on = on

    def __enter__(self):
        self.old = os.environ.get("RECSA_BUILD_QUEUE")
        os.environ["RECSA_BUILD_QUEUE"] = "1" if self.on else "0"

    def __exit__(self, *exc):
        if self.old is None:
            del os.environ["RECSA_BUILD_QUEUE"]
        else:
            os.environ["RECSA_BUILD_QUEUE"] = self.old


# (B, H_kv, d, dtype, f, L): every shape's level-1 launch has more tiles (32 nodes at d = 128,
# 64 at d = 64) than the 512 workgroups of the persistent grid
SHAPES = [
    (1, 8, 128, "bf16", 16, 16 ** 4 * 2 + 16 ** 2 * 3 + 7),   # levels 1+2 and 3+4 fused
    (2, 3, 128, "bf16", 32, 32 ** 3 * 3 + 32 * 5 + 1),        # f = 32: pairs fused
    (2, 4, 64, "f32", 16, 16 ** 4 + 16 ** 3 + 9),             # float32: node rows re-read
    (2, 4, 128, "bf16", 5, 5 ** 7 * 2 + 3),                   # f = 5: one level per launch
]


def _inputs(B, Hkv, d, dtype, L, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = d ** -0.5
    K = (torch.randn(B, Hkv, L, d, device="cuda", generator=g) * s).to(td)
    V = (torch.randn(B, Hkv, L, d, device="cuda", generator=g) * s).to(td)
    W = (torch.eye(d, device="cuda") + 0.05 * s * torch.randn(d, d, device="cuda", generator=g)).to(td)
    return K, V, W


def _tree(sh):
    return torch.full((R.recsa_tree_bytes(sh),), 0xA5, dtype=torch.uint8, device="cuda")


def _levels(sh, tree, L, f):
    """Every level's node rows [B][H_kv][nodes][d] as storage bits (rows past the last complete
    node are not part of the tree)."""
    out = []
    for lv in range(1, R.recsa_num_levels(L, f) + 1):
        n = L // f ** lv
        NK, NV = R.tree_level_views(sh, tree, lv)
        out.append((storage_bits(NK[:, :, :n]), storage_bits(NV[:, :, :n])))
    return out


def _same(a, b, what):
    for lv, ((ka, va), (kb, vb)) in enumerate(zip(a, b), start=1):
        assert np.array_equal(ka, kb), f"{what}: keys differ at level {lv}"
        assert np.array_equal(va, vb), f"{what}: values differ at level {lv}"


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_H{s[1]}_d{s[2]}_{s[3]}_f{s[4]}")
def test_queue_order_builds_the_static_order_tree(shape):
    B, Hkv, d, dtype, f, L = shape
    _say(f"build queue {shape}")
    K, V, W = _inputs(B, Hkv, d, dtype, L, seed=11 + f)
    sh = R.Shape(B, Hkv, 8 * Hkv, d, f, dtype, L, 0.0, 1.0e6)
    trees = {}
    for on in (False, True):
        tree = _tree(sh)
        with _queue(on):
            R.recsa_build_tree(sh, K, V, W, 0, L, tree)
        torch.cuda.synchronize()
        trees[on] = _levels(sh, tree, L, f)
    _same(trees[True], trees[False], "one-shot build")
    # built in increments through the queue
    tree = _tree(sh)
    cuts = [0, f ** 2 + 1, L // 3, L // 3 + f - 1, L - 5, L]
    with _queue(True):
        for a, b in zip(cuts[:-1], cuts[1:]):
            R.recsa_build_tree(sh, K, V, W, a, b, tree)
    torch.cuda.synchronize()
    _same(_levels(sh, tree, L, f), trees[False], "build in increments")
    # one slice against the oracle
    b, h = B - 1, Hkv - 1
    Kf = oracle.from_storage(storage_bits(K[b, h]).view(np.uint16 if dtype == "bf16" else np.float32), dtype)
    Vf = oracle.from_storage(storage_bits(V[b, h]).view(np.uint16 if dtype == "bf16" else np.float32), dtype)
    Wf = oracle.from_storage(storage_bits(W).view(np.uint16 if dtype == "bf16" else np.float32), dtype)
    want = oracle.build_slice(Kf, Vf, Wf, f, dtype, n_new=L)
    for lv, (nk, nv) in enumerate(trees[True], start=1):
        wk = oracle.to_storage(want[lv - 1][0], dtype).view(nk.dtype)
        wv = oracle.to_storage(want[lv - 1][1], dtype).view(nv.dtype)
        assert np.array_equal(nk[b, h], wk), f"keys differ from the oracle at level {lv}"
        assert np.array_equal(nv[b, h], wv), f"values differ from the oracle at level {lv}"


def test_builds_on_many_streams_at_once():
    """Twelve builds issued back to back on twelve streams (more than the eight queues), twice:
    every tree equals the static-order tree."""
    B, Hkv, d, dtype, f, L = 1, 8, 128, "bf16", 16, 16 ** 4 + 16 ** 2 * 9 + 3
    _say("build queue: 12 streams")
    K, V, W = _inputs(B, Hkv, d, dtype, L, seed=21)
    sh = R.Shape(B, Hkv, 32, d, f, dtype, L, 0.0, 1.0e6)
    ref = _tree(sh)
    with _queue(False):
        R.recsa_build_tree(sh, K, V, W, 0, L, ref)
    torch.cuda.synchronize()
    want = _levels(sh, ref, L, f)
    streams = [torch.cuda.Stream() for _ in range(12)]
    trees = [_tree(sh) for _ in streams]
    torch.cuda.synchronize()
    for rep in range(2):
        with _queue(True):
            for s, t in zip(streams, trees):
                R.recsa_build_tree(sh, K, V, W, 0, L, t, stream=s)
        torch.cuda.synchronize()
        for i, t in enumerate(trees):
            _same(_levels(sh, t, L, f), want, f"stream {i}, pass {rep}")
            t.fill_(0x5A)
        torch.cuda.synchronize()


def test_build_replayed_from_a_graph():
    """A build captured in a HIP graph (it takes the static order) and replayed three times,
    with queue-ordered builds between the replays: every tree equals the eager one."""
    B, Hkv, d, dtype, f, L = 1, 8, 128, "bf16", 16, 16 ** 4 + 16 * 3 + 1
    _say("build queue: graph")
    K, V, W = _inputs(B, Hkv, d, dtype, L, seed=31)
    sh = R.Shape(B, Hkv, 32, d, f, dtype, L, 0.0, 1.0e6)
    ref = _tree(sh)
    with _queue(True):
        R.recsa_build_tree(sh, K, V, W, 0, L, ref)
    torch.cuda.synchronize()
    want = _levels(sh, ref, L, f)
    gt = _tree(sh)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        R.recsa_build_tree(sh, K, V, W, 0, L, gt)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        R.recsa_build_tree(sh, K, V, W, 0, L, gt)
    other = _tree(sh)
    for rep in range(3):
        gt.fill_(0x33)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(_levels(sh, gt, L, f), want, f"replay {rep}")
        with _queue(True):
            R.recsa_build_tree(sh, K, V, W, 0, L, other)
        torch.cuda.synchronize()
        _same(_levels(sh, other, L, f), want, f"eager build after replay {rep}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2]], ids=lambda s: f"d{s[2]}_{s[3]}")
def test_small_launches_build_the_one_shot_tree(shape):
    """Built 4096 (d = 128) or 2048 (d = 64) tokens at a time (at most 65 tiles per launch: the
    one-tile form) against a one-shot build (the persistent form)."""
    B, Hkv, d, dtype, f, L = shape
    _say(f"build small launches {shape}")
    K, V, W = _inputs(B, Hkv, d, dtype, L, seed=41)
    sh = R.Shape(B, Hkv, 8 * Hkv, d, f, dtype, L, 0.0, 1.0e6)
    one = _tree(sh)
    R.recsa_build_tree(sh, K, V, W, 0, L, one)
    step = 4096 if d == 128 else 2048
    inc = _tree(sh)
    cuts = list(range(0, L, step)) + [L]
    for a, b in zip(cuts[:-1], cuts[1:]):
        R.recsa_build_tree(sh, K, V, W, a, b, inc)
    torch.cuda.synchronize()
    _same(_levels(sh, inc, L, f), _levels(sh, one, L, f), "4096-token increments")


def test_builds_from_several_host_threads():
    """Four host threads, each building its own tree on its own stream six times (the library
    call releases the interpreter lock, so the calls overlap on the host and on the GPU): every
    tree equals the static-order tree."""
    import threading
    B, Hkv, d, dtype, f, L = 1, 8, 128, "bf16", 16, 16 ** 4 + 16 ** 2 * 7 + 5
    _say("build queue: 4 host threads")
    K, V, W = _inputs(B, Hkv, d, dtype, L, seed=51)
    sh = R.Shape(B, Hkv, 32, d, f, dtype, L, 0.0, 1.0e6)
    ref = _tree(sh)
    with _queue(False):
        R.recsa_build_tree(sh, K, V, W, 0, L, ref)
    torch.cuda.synchronize()
    want = _levels(sh, ref, L, f)
    trees = [_tree(sh) for _ in range(4)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            for _ in range(6):
                R.recsa_build_tree(sh, K, V, W, 0, L, trees[i], stream=streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below
            errors.append(repr(e))

    with _queue(True):
        threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, t in enumerate(trees):
        _same(_levels(sh, t, L, f), want, f"thread {i}")
