"""The C-ABI library without a GPU: it loads, exports every declared entry point, sizes
buffers as documented, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

from long_context_hierarchical_amd import recsa as R
from oracle import INT32_MAX, level_counts, plan_counts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "recsa.h")).read()
    return sorted(set(re.findall(r"\b(recsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = R.lib()
    names = _declared()
    assert set(names) == set(R.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert R.recsa_abi_version() == 3


def _shape(**kw):
    base = dict(batch=2, n_kv_heads=8, n_q_heads=32, head_dim=128, fanout=16, dtype="bf16",
                capacity=1 << 20, rope_theta=1.0e6)
    base.update(kw)
    return R.Shape(**base)


def test_levels_and_tree_layout():
    for n, f in [(0, 16), (15, 16), (16, 16), (4096, 16), (4095, 16), (131072, 16), (2 ** 21, 32), (1000, 3)]:
        assert R.recsa_num_levels(n, f) == len(level_counts(n, f))
    sh = _shape()
    T = R.recsa_num_levels(sh.capacity, sh.fanout)
    total, off = 0, 0
    for lv in range(1, T + 1):
        rows = sh.capacity // sh.fanout ** lv
        blk = sh.batch * sh.n_kv_heads * rows * sh.head_dim * 2
        assert R.recsa_level_offset(sh, lv, 0) == off
        assert R.recsa_level_offset(sh, lv, 1) == off + blk
        off += 2 * blk
    assert R.recsa_tree_bytes(sh) == off


@pytest.mark.parametrize("n,f,k", [(4096, 16, 4), (131072, 16, 8), (2 ** 21, 32, 16), (5000, 16, 8), (777, 4, 3)])
def test_sel_width_matches_closed_form(n, f, k):
    sh = _shape(fanout=f, capacity=max(n, 1))
    T = R.recsa_num_levels(n, f)
    ks = [k] * T
    C, s, _ = plan_counts(n, f, ks)
    assert R.recsa_sel_width(sh, n, n, ks) == max(s.values(), default=0)
    lo = max(1, n - 300)
    want = 0
    for m in range(lo, n + 1):
        _, sm, _ = plan_counts(m, f, ks + [k] * 4)
        want = max(want, max(sm.values(), default=0))
    assert R.recsa_sel_width(sh, lo, n, ks) == want


@pytest.mark.parametrize("seed", range(12))
def test_sel_width_over_ranges_matches_every_prefix(seed):
    """recsa_sel_width(n_min, n_max) = the largest kept count over every prefix in the range, with
    per-level k that make the kept counts rise and fall with n (orphans, levels kept whole)."""
    rng = np.random.default_rng(seed)
    f = int(rng.choice([2, 3, 4, 16]))
    n_max = int(rng.integers(1, 3000))
    n_min = int(rng.integers(0, n_max + 1))
    T = R.recsa_num_levels(n_max, f)
    ks = [int(rng.choice([0, 1, 2, 3, 5, 17, INT32_MAX])) for _ in range(max(T, 1))]
    sh = _shape(fanout=f, capacity=n_max)
    want = 0
    for m in range(n_min, n_max + 1):
        _, sm, _ = plan_counts(m, f, ks + [ks[-1]] * 4)
        want = max(want, max(sm.values(), default=0))
    assert R.recsa_sel_width(sh, n_min, n_max, ks) == want


def test_workspace_holds_the_rope_table():
    sh = _shape(head_dim=128)
    k = [8] * 4
    nb = R.recsa_workspace_bytes(sh, 131072, k)
    # positions 0..max candidates (f*k + f - 1 = 143) of (cos, sin) float32 pairs, 256-byte aligned
    assert nb == ((143 + 1) * 64 * 8 + 255) // 256 * 256
    assert R.recsa_workspace_bytes(_shape(rope_theta=0.0), 131072, k) == 0


def _status(fn, *args, **kw):
    with pytest.raises(R.RecsaError) as e:
        fn(*args, **kw)
    return e.value.code


class _FakeTensor:
    """A pointer-only stand-in: validation must reject the call before touching it."""

    def __init__(self, addr=0x1000, shape=(1, 1, 1, 1)):
        self._addr, self.shape = addr, shape

    def data_ptr(self):
        return self._addr

    def numel(self):
        return 1 << 30

    def element_size(self):
        return 1


class _NoStream:
    cuda_stream = 0


def test_error_paths_return_status_before_launch():
    t = _FakeTensor()
    ns = _NoStream()
    sh = _shape(capacity=4096)
    k = [8] * 3
    bad_heads = _shape(n_q_heads=30)
    assert _status(R.recsa_build_tree, bad_heads, t, t, t, 0, 16, t, ns) == -1
    assert _status(R.recsa_build_tree, _shape(head_dim=96), t, t, t, 0, 16, t, ns) == -3
    assert _status(R.recsa_build_tree, _shape(fanout=1), t, t, t, 0, 16, t, ns) == -3
    assert _status(R.recsa_build_tree, sh, t, t, t, 0, 5000, t, ns) == -2
    assert _status(R.recsa_build_tree, sh, t, t, t, 20, 10, t, ns) == -1
    assert _status(R.recsa_build_tree, sh, None, t, t, 0, 4096, t, ns) == -1
    assert _status(R.recsa_build_tree, sh, _FakeTensor(0x1008), t, t, 0, 4096, t, ns) == -1
    q = _FakeTensor(shape=(2, 4, 32, 128))
    assert _status(R.recsa_decode, sh, q, t, t, t, 5000, k, t, None, None, 0, t, ns) == -2
    assert _status(R.recsa_decode, sh, q, t, t, t, 4096, [8, 8], t, None, None, 0, t, ns) == -1
    assert _status(R.recsa_decode, sh, q, t, t, t, 4096, [8, -1, 8], t, None, None, 0, t, ns) == -1
    assert _status(R.recsa_decode, sh, q, t, t, t, 4096, k, t, None, t, 1, t, ns) == -1  # sel_width too small
    small_ws = _FakeTensor()
    small_ws.numel = lambda: 16
    assert _status(R.recsa_decode, sh, q, t, t, t, 4096, k, t, None, None, 0, small_ws, ns) == -5
    assert _status(R.recsa_prefill, sh, q, 4094, t, t, t, k, t, None, None, 0, t, ns) == -2
    assert _status(R.recsa_prefill, sh, q, -1, t, t, t, k, t, None, None, 0, t, ns) == -1
    assert _status(R.recsa_decode, _shape(capacity=1 << 20), q, t, t, t, 1 << 20, [1 << 30] * 5, t, None, None, 0,
                   t, ns) == -3                                                          # lists beyond LDS
    assert "capacity" in R.lib().recsa_last_error().decode() or R.lib().recsa_last_error()
    # one decoding step: the new row must fit, its inputs must lie outside the caches, the
    # pooler is needed, and the attention checks apply -- all before anything is written
    kn = _FakeTensor(0x10000000)
    q1 = _FakeTensor(shape=(2, 32, 128))
    step = R.recsa_decode_step
    assert _status(step, sh, q1, kn, kn, t, t, t, t, 4096, k, t, workspace=t, stream=ns) == -2
    assert _status(step, sh, q1, t, kn, t, t, t, t, 100, k, t, workspace=t, stream=ns) == -1
    assert "overlap" in R.lib().recsa_last_error().decode()
    assert _status(step, sh, q1, kn, kn, t, t, None, t, 100, k, t, workspace=t, stream=ns) == -1
    assert _status(step, sh, q1, kn, kn, t, t, t, t, 4095, [8, 8], t, workspace=t, stream=ns) == -1
    assert _status(step, sh, q1, kn, kn, t, t, t, t, 100, k, t, None, None, 0, small_ws, stream=ns) == -5
    assert _status(step, sh, q1, kn, kn, t, t, t, t, 100, k, t, None, t, 0, t, stream=ns) == -1  # sel_width
    # gradients: mode, capacity, the forward's selections, their width and the workspace are checked first
    bwd = R.recsa_backward
    w8 = R.recsa_sel_width(sh, 4096, 4096, k)
    args = (t, t, t, t, k, t, t, t, w8, t, t, t, t, t)
    assert _status(bwd, sh, False, q, 0, 5000, *args, workspace=t, stream=ns) == -2
    assert _status(bwd, sh, True, q, 4094, 0, *args, workspace=t, stream=ns) == -2
    assert _status(bwd, sh, False, q, 0, 4096, t, t, t, t, k, t, t, None, w8, t, t, t, t, t, workspace=t,
                   stream=ns) == -1
    assert _status(bwd, sh, False, q, 0, 4096, t, t, t, t, k, t, t, t, 1, t, t, t, t, t, workspace=t,
                   stream=ns) == -1
    assert _status(bwd, sh, False, q, 0, 4096, *args, workspace=small_ws, stream=ns) == -5
    assert R.recsa_backward_workspace_bytes(sh, 4096, k) > R.recsa_workspace_bytes(sh, 4096, k)
    # heads selecting in groups smaller than their KV head: a divisor of G; gradients need whole groups
    alone = _shape(capacity=4096, select_heads=1)
    assert _status(bwd, alone, False, q, 0, 4096, *args, workspace=t, stream=ns) == -3
    assert _status(R.recsa_decode, _shape(capacity=4096, select_heads=3), q, t, t, t, 4096, k, t, None, None, 0, t,
                   ns) == -1


def test_two_stage_sizes_and_error_paths():
    """Workspace = RoPE table (rows 0..C0) + queries rotated at two positions + rotated block keys
    (unless given) + the per-slab candidate lists + the kept block ids; bad arguments are rejected
    before any launch."""
    sh = _shape(batch=4, capacity=1 << 19)
    n, nq, kb, kt = 1 << 19, 256, 128, 512
    n1 = n // 16
    C0 = 16 * kb
    SB = 1024                                   # blocks per slab for 4 query heads per KV head
    slabs = -(-n1 // SB)
    al = lambda x: (x + 255) // 256 * 256
    want = (al((C0 + 1) * 64 * 8) + 2 * al(4 * nq * 32 * 128 * 2) + al(4 * 8 * n1 * 128 * 2)
            + al(4 * 8 * nq * slabs * kb * 8) + al(4 * 8 * nq * kb * 4))
    assert R.recsa_two_stage_workspace_bytes(sh, n, nq, kb, kt) == want
    assert R.recsa_two_stage_workspace_bytes(sh, n, nq, kb, kt, blocks_rotated=True) == want - al(4 * 8 * n1 * 128 * 2)
    t = _FakeTensor()
    ns = _NoStream()
    q = _FakeTensor(shape=(4, nq, 32, 128))
    ts = R.recsa_two_stage_decode
    assert _status(ts, sh, q, t, t, t, n + 1, kb, kt, t, workspace=t, stream=ns) == -2
    assert _status(ts, sh, q, t, t, t, n, -1, kt, t, workspace=t, stream=ns) == -1
    assert _status(ts, sh, q, t, t, t, n, kb, -1, t, workspace=t, stream=ns) == -1
    assert _status(ts, _shape(batch=4, capacity=n, select_heads=1), q, t, t, t, n, kb, kt, t, workspace=t,
                   stream=ns) == -3
    assert _status(ts, sh, q, t, t, t, n, 4096, kt, t, workspace=t, stream=ns) == -3        # lists beyond LDS
    sb = _FakeTensor(shape=(4, nq, 8, kb - 1))
    assert _status(ts, sh, q, t, t, t, n, kb, kt, t, sel_blocks=sb, workspace=t, stream=ns) == -1
    st = _FakeTensor(shape=(4, nq, 8, kt - 1))
    assert _status(ts, sh, q, t, t, t, n, kb, kt, t, sel_tokens=st, workspace=t, stream=ns) == -1
    small_ws = _FakeTensor()
    small_ws.numel = lambda: 1024
    assert _status(ts, sh, q, t, t, t, n, kb, kt, t, workspace=small_ws, stream=ns) == -5
    assert _status(ts, sh, q, None, t, t, n, kb, kt, t, workspace=t, stream=ns) == -1
    rb = R.recsa_two_stage_rotate_blocks
    assert _status(rb, sh, t, 10, 5, t, ns) == -1
    assert _status(rb, sh, t, 0, n + 16, t, ns) == -2
    assert _status(rb, sh, None, 0, 4096, t, ns) == -1
    assert _status(rb, sh, t, 0, 4096, t, ns) == -1                                        # block_keys = tree
