"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on seeded inputs.

Selections must be identical level by level (a flagged near tie, relative score gap below
1e-5, may split either way); outputs within 2e-3 (bf16 storage) or 1e-5 (float32).
"""
import numpy as np
import pytest
import torch

import oracle
import gpu_util
from gpu_util import TOL, Gpu, check_unit, oracle_replayer, storage_bits
from long_context_hierarchical_amd import recsa as R
from synthetic import WORKLOADS, Workload, gen_decode_inputs, with_overrides

pytestmark = pytest.mark.gpu
INT32_MAX = oracle.INT32_MAX


def _say(msg):
    print(msg, flush=True)


def _check_units(w, inp, res, k, units, mode, n_tokens=None, q_start=0):
    """Every unit's selections, outputs and lse against the oracle; a near-tie split is followed
    by forced-selection replay, so no unit goes unchecked."""
    out, lse, sel, _ = res
    cache = oracle.TreeCache(inp["K"], inp["V"], inp["W"], w.f, w.dtype)
    if mode == "decode":
        qs = inp["q"]
        ref = oracle.decode(inp["K"], inp["V"], inp["W"], qs, n_tokens, w.f, k, w.dtype, w.theta, units=units,
                            cache=cache)
    else:
        qs = inp["q"][:, q_start:q_start + out.shape[1]]
        ref = oracle.prefill(inp["K"], inp["V"], inp["W"], qs, q_start, w.f, k, w.dtype, w.theta, units=units,
                             cache=cache)
    G = w.G
    stats = {"match": 0, "replayed": 0}
    for (b, j, h), r in ref.items():
        n = n_tokens if mode == "decode" else q_start + j + 1
        rep = oracle_replayer(cache, qs, w, k, b, j, h, n, mode != "decode")
        st = check_unit(r, sel[b, j, h], out[b, j, h * G:(h + 1) * G], lse[b, j, h * G:(h + 1) * G],
                        TOL[w.dtype], where=f"{w.name} unit {(b, j, h)}", replay=rep)
        stats[st] += 1
    if stats["replayed"]:
        _say(f"{w.name}: {stats}")
    return stats


def _w(name="t", B=1, Hq=4, Hkv=1, d=64, dtype="f32", L=4096, f=16, k=4, n_queries=4, **kw):
    std = kw.pop("std", 1.0 if dtype == "f32" else d ** -0.5)
    return Workload(name, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, L=L, f=f, k=k, n_queries=n_queries,
                    mode="decode", std=std, **kw)


# ------------------------------------------------------------------ tree build

BUILD_CASES = [
    _w("b_f32_d64_f16", L=4096 + 77, seed=1),
    _w("b_bf16_d128_f16", Hq=8, Hkv=2, d=128, dtype="bf16", L=16 ** 3 * 3 + 250, seed=2),
    _w("b_bf16_d128_f32", Hq=4, Hkv=1, d=128, dtype="bf16", L=32 ** 2 * 5 + 31, f=32, seed=3),
    _w("b_f32_d64_f3", L=3 ** 7 + 5, f=3, seed=4),
    _w("b_bf16_d64_f5", B=2, Hq=2, Hkv=2, d=64, dtype="bf16", L=5 ** 5 + 9, f=5, seed=5),
    # fanouts dividing the pool kernel's tile (d=128: 32 nodes, d=64: 64): level pairs built in one pass
    _w("b_bf16_d64_f32_fused", Hq=2, Hkv=1, d=64, dtype="bf16", L=32 ** 3 + 32 * 7 + 5, f=32, seed=7),
    _w("b_f32_d64_f32_fused", Hq=2, Hkv=2, d=64, dtype="f32", L=32 ** 2 * 3 + 40, f=32, seed=8),
    _w("b_bf16_d128_f16_deep", Hq=8, Hkv=2, d=128, dtype="bf16", L=16 ** 4 + 16 ** 2 * 5 + 3, f=16, seed=9),
]


@pytest.mark.parametrize("w", BUILD_CASES, ids=lambda w: w.name)
def test_tree_build_bitwise(w):
    """Every node key and value equals the oracle's bit for bit, built in several increments."""
    _say(f"build {w.name}")
    inp = gen_decode_inputs(w, n_q=1)
    g = Gpu(w, inp, build=False)
    cuts = [0, 1, w.f - 1, w.f ** 2 + 3, w.L // 2, w.L - 1, w.L]
    for a, b in zip(cuts[:-1], cuts[1:]):
        from long_context_hierarchical_amd import recsa as R
        R.recsa_build_tree(g.shape, g.K, g.V, g.W, a, b, g.tree)
    torch.cuda.synchronize()
    from long_context_hierarchical_amd import recsa as R
    Wf = oracle.from_storage(inp["W"], w.dtype)
    T = oracle.level_counts(w.L, w.f)
    for b in range(w.B):
        for h in range(w.Hkv):
            Kf = oracle.from_storage(inp["K"][b, h], w.dtype)
            Vf = oracle.from_storage(inp["V"][b, h], w.dtype)
            tree = oracle.build_slice(Kf, Vf, Wf, w.f, w.dtype, n_new=w.L)
            for lv in range(1, len(T) + 1):
                NK, NV = R.tree_level_views(g.shape, g.tree, lv)
                want_k = oracle.to_storage(tree[lv - 1][0], w.dtype)
                want_v = oracle.to_storage(tree[lv - 1][1], w.dtype)
                got_k = storage_bits(NK[b, h])
                got_v = storage_bits(NV[b, h])
                wk = want_k.view(got_k.dtype)
                wv = want_v.view(got_v.dtype)
                assert np.array_equal(got_v, wv), f"values differ at level {lv}: {np.sum(got_v != wv)} elements"
                assert np.array_equal(got_k, wk), f"keys differ at level {lv}: {np.sum(got_k != wk)} elements"


def test_rope_table_bitwise(monkeypatch):
    """The (cos, sin) table the kernels read equals the oracle's bit for bit. With the library's
    RoPE table cache turned off the call fills its table in its workspace, where it is read back;
    the cache is filled by the same kernel (a row does not depend on the table's length), and
    test_gpu_rope_cache checks that cached and uncached calls agree bit for bit."""
    monkeypatch.setenv("RECSA_ROPE_CACHE", "0")
    w = _w("tab", Hq=32, Hkv=8, d=128, dtype="bf16", L=16 ** 4 + 100, f=16, k=8, n_queries=1, seed=6)
    inp = gen_decode_inputs(w, n_q=1, heads=[0])
    g = Gpu(w, inp)
    k = [8] * 4
    _, _, _, ws = g.decode(k, w.L)
    P = 16 * 8 + 16 - 1
    got = ws[:(P + 1) * 64 * 8].view(torch.float32).view(P + 1, 64, 2).cpu().numpy()
    c, s = oracle.rope_table(P, 128, w.theta)
    assert np.array_equal(got[..., 0].view(np.uint32), c.view(np.uint32))
    assert np.array_equal(got[..., 1].view(np.uint32), s.view(np.uint32))


# ------------------------------------------------------------------ decode

def test_decode_tiny_workload_full():
    """The 4K-token float32 workload: every query, every unit."""
    w = WORKLOADS["c0"]
    _say("decode c0")
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    k = [w.k] * 3
    res = g.decode(k, w.L)
    units = [(0, j, 0) for j in range(w.n_queries)]
    _check_units(w, inp, res, k, units, "decode", n_tokens=w.L)


DECODE_CASES = [
    # (workload, k per level, n_tokens offset from L)
    (_w("d_bf16_G4_f16_ragged", Hq=8, Hkv=2, d=128, dtype="bf16", L=5000, k=8, n_queries=3, seed=11), [8] * 3),
    (_w("d_bf16_G8_f32", Hq=16, Hkv=2, d=128, dtype="bf16", L=40000, f=32, k=16, n_queries=2, seed=12), [16] * 3),
    (_w("d_f32_G1_f3", Hq=2, Hkv=2, d=64, dtype="f32", L=1000, f=3, k=2, n_queries=3, seed=13), [2, 3, 1, 2, 2, 4]),
    (_w("d_bf16_G2_f4_mixedk", B=2, Hq=4, Hkv=2, d=64, dtype="bf16", L=777, f=4, n_queries=2, seed=14),
     [0, 3, 1, 5]),
    (_w("d_f32_norope", d=64, L=3000, k=4, n_queries=3, theta=0.0, seed=15), [4, 4]),
    (_w("d_f32_T0", d=64, L=13, k=4, n_queries=2, seed=16), [4]),
    (_w("d_bf16_nopruning", Hq=8, Hkv=2, d=128, dtype="bf16", L=3000, k=4, n_queries=2, seed=17), [INT32_MAX] * 2),
    (_w("d_f32_k0", d=64, L=4096 + 300, k=0, n_queries=2, seed=18), [0, 0, 0]),
    (_w("d_bf16_G4_f16_big_k", Hq=4, Hkv=1, d=128, dtype="bf16", L=16 ** 3 * 4, k=20, n_queries=2, seed=19),
     [20, 20, 20]),
]


@pytest.mark.parametrize("w,k", DECODE_CASES, ids=lambda x: getattr(x, "name", ""))
def test_decode_variants(w, k):
    _say(f"decode {w.name}")
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    res = g.decode(k, w.L)
    units = [(b, j, h) for b in range(w.B) for j in range(w.n_queries) for h in range(w.Hkv)]
    _check_units(w, inp, res, k, units, "decode", n_tokens=w.L)


def test_decode_on_a_shorter_prefix_and_empty_cache():
    """The tree holds more nodes than the visible prefix; nodes beyond it must be ignored.
    With no visible token, out = 0 and lse = -inf."""
    w = _w("prefix", Hq=8, Hkv=2, d=128, dtype="bf16", L=9000, k=8, n_queries=2, seed=21)
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    for n in (8191, 4096, 300, 16, 15, 1):
        k = [8] * max(1, oracle.level_counts(n, 16).__len__())
        res = g.decode(k, n)
        units = [(0, j, h) for j in range(2) for h in range(2)]
        _check_units(w, inp, res, k, units, "decode", n_tokens=n)
    out, lse, sel, _ = g.decode([8], 0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_decode_is_deterministic():
    w = _w("det", Hq=32, Hkv=8, d=128, dtype="bf16", L=70000, k=8, n_queries=8, seed=22)
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    k = [8] * 4
    a = g.decode(k, w.L)
    b = g.decode(k, w.L)
    assert np.array_equal(a[2], b[2])
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))


def test_decode_launch_shapes_agree_bitwise():
    """Calls with many units run one wave per (sequence, query, KV head); calls with few run
    several waves per unit. Both accumulate every output element in the same order, so the
    same query gives bitwise-identical results either way."""
    w = _w("shapes", B=2, Hq=32, Hkv=8, d=128, dtype="bf16", L=70000, k=8, n_queries=150, seed=23)
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    k = [8] * 4
    big = g.decode(k, w.L)                      # 2 x 150 x 8 = 2400 units: one wave each
    for j in (0, 77, 149):
        one = g.decode(k, w.L, q=g.q[:, j:j + 1].contiguous())   # 16 units: several waves each
        assert np.array_equal(one[2][:, 0], big[2][:, j]), j
        assert np.array_equal(one[0][:, 0].view(np.uint32), big[0][:, j].view(np.uint32)), j
        assert np.array_equal(one[1][:, 0].view(np.uint32), big[1][:, j].view(np.uint32)), j


ONE_WAVE_CASES = [
    # (workload with >= 2048 (sequence, query, KV head) units per call, k per level)
    (_w("w1_f32_d64_G1_f3", Hq=2, Hkv=2, d=64, dtype="f32", L=1000, f=3, k=2, n_queries=1100, seed=41),
     [2, 3, 1, 2, 2, 4]),
    (_w("w1_bf16_d64_G2_f4", B=2, Hq=4, Hkv=2, d=64, dtype="bf16", L=777, f=4, k=3, n_queries=520, seed=42),
     [0, 3, 1, 5]),
    (_w("w1_bf16_d128_G8_f32", Hq=16, Hkv=2, d=128, dtype="bf16", L=40000, f=32, k=16, n_queries=1030, seed=43),
     [16] * 3),
    (_w("w1_f32_d128_G4_f16", Hq=8, Hkv=2, d=128, dtype="f32", L=5000, k=8, n_queries=1030, seed=44), [8] * 3),
    # bf16 without the rotation (the unrotated score passes next to the matrix-core tile)
    (_w("w1_bf16_d128_G4_norope", Hq=8, Hkv=2, d=128, dtype="bf16", L=5000, k=8, n_queries=1030, theta=0.0,
        seed=45), [8] * 3),
    # bf16 with one query head per KV head (the tile, then the fmaf value sums)
    (_w("w1_bf16_d128_G1_f16", Hq=2, Hkv=2, d=128, dtype="bf16", L=6000, k=8, n_queries=1030, seed=46), [8] * 3),
]


@pytest.mark.parametrize("w,k", ONE_WAVE_CASES, ids=lambda x: getattr(x, "name", ""))
def test_decode_one_wave_per_unit_variants(w, k):
    """Calls large enough for one wave per unit, for each storage type, head size and group
    size: sampled units against the oracle, and every sampled query bitwise equal to the same
    query decoded alone (several waves per unit)."""
    _say(f"decode one-wave {w.name}")
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    big = g.decode(k, w.L)
    js = [0, 1, w.n_queries // 2, w.n_queries - 1]
    units = [(b, j, h) for b in range(w.B) for j in js for h in range(w.Hkv)]
    _check_units(w, inp, big, k, units, "decode", n_tokens=w.L)
    for j in js:
        one = g.decode(k, w.L, q=g.q[:, j:j + 1].contiguous())
        assert np.array_equal(one[2][:, 0], big[2][:, j]), j
        assert np.array_equal(one[0][:, 0].view(np.uint32), big[0][:, j].view(np.uint32)), j


# ------------------------------------------------------------------ prefill

def test_prefill_matches_oracle_and_chunking():
    """Causal prefill: sampled positions (edges of blocks and levels included) against the
    oracle, and the same positions computed in uneven chunks give bitwise-identical results."""
    w = _w("pf", Hq=8, Hkv=2, d=128, dtype="bf16", L=5000, k=8, n_queries=5000, seed=31)
    _say("prefill")
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    k = [8] * 3
    full = g.prefill(k, 0, w.L)
    rng = np.random.default_rng(0)
    pos = sorted(set([0, 1, 14, 15, 16, 17, 255, 256, 257, 4095, 4096, 4097, w.L - 1] +
                     rng.integers(0, w.L, 40).tolist()))
    units = [(0, int(p), h) for p in pos for h in range(w.Hkv)]
    _check_units(w, inp, full, k, units, "prefill", q_start=0)
    cuts = [0, 1000, 1001, 3333, w.L]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = g.prefill(k, a, b - a)
        assert np.array_equal(part[2], full[2][:, a:b]), (a, b)
        assert np.array_equal(part[0].view(np.uint32), full[0][:, a:b].view(np.uint32)), (a, b)


def test_prefill_with_incremental_tree():
    """Chunked prefill where the tree is extended chunk by chunk, as a serving loop does."""
    w = _w("pf_inc", Hq=8, Hkv=2, d=64, dtype="f32", L=3000, f=4, k=3, n_queries=3000, seed=32)
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp, build=False)
    from long_context_hierarchical_amd import recsa as R
    k = [3] * 6
    outs = []
    for a in range(0, w.L, 700):
        b = min(w.L, a + 700)
        R.recsa_build_tree(g.shape, g.K, g.V, g.W, a, b, g.tree)
        outs.append(g.prefill(k, a, b - a))
    sel = np.concatenate([o[2] for o in outs], axis=1)
    out = np.concatenate([o[0] for o in outs], axis=1)
    lse = np.concatenate([o[1] for o in outs], axis=1)
    pos = [0, 3, 4, 15, 16, 63, 64, 699, 700, 701, 2047, 2048, 2999] + list(range(1200, 1230))
    units = [(0, p, h) for p in pos for h in range(2)]
    _check_units(w, inp, (out, lse, sel, None), k, units, "prefill", q_start=0)


def test_prefill_two_sequences_bf16_eight_head_groups():
    """bf16 prefill of two sequences with 8 query heads per KV head, tree and queries in two
    uneven calls: both sequences against the oracle at block edges and random positions."""
    w = _w("pf_b2_g8", B=2, Hq=16, Hkv=2, d=128, dtype="bf16", L=3000, f=16, k=8, n_queries=3000, seed=33)
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp, build=False)
    from long_context_hierarchical_amd import recsa as R
    k = [8] * 2
    outs = []
    for a, b in ((0, 1777), (1777, w.L)):
        R.recsa_build_tree(g.shape, g.K, g.V, g.W, a, b, g.tree)
        outs.append(g.prefill(k, a, b - a))
    sel = np.concatenate([o[2] for o in outs], axis=1)
    out = np.concatenate([o[0] for o in outs], axis=1)
    lse = np.concatenate([o[1] for o in outs], axis=1)
    rng = np.random.default_rng(3)
    pos = sorted(set([0, 15, 16, 255, 256, 1776, 1777, 2047, 2048, 2999] + rng.integers(0, w.L, 12).tolist()))
    units = [(b, p, h) for b in range(w.B) for p in pos for h in range(w.Hkv)]
    _check_units(w, inp, (out, lse, sel, None), k, units, "prefill", q_start=0)



# ------------------------------------------------------------------ heads selecting in smaller groups

@pytest.mark.parametrize("Gs", [1, 2])
@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_heads_selecting_in_smaller_groups(Gs, mode):
    """select_heads = Gs < G: groups of Gs query heads each descend on their own summed logit over
    their KV head's tree; every group against the oracle's."""
    w = _w("sel_heads", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", L=16 ** 3 + 100, f=16, k=4, n_queries=3, seed=71)
    inp = gen_decode_inputs(w)
    dev = "cuda:0"
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta, select_heads=Gs)
    K, V, W, q = (gpu_util.dev_tensor(inp[x], w.dtype) for x in ("K", "V", "W", "q"))
    tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device=dev)
    R.recsa_build_tree(sh, K, V, W, 0, w.L, tree)
    T = R.recsa_num_levels(w.L, w.f)
    k = [w.k] * T
    n_q = q.shape[1]
    groups = w.Hq // Gs
    q_start = w.L - n_q
    n_min, n_max = (q_start + 1, w.L) if mode == "prefill" else (w.L, w.L)
    width = R.recsa_sel_width(sh, n_min, n_max, k)
    ws = torch.zeros(R.recsa_workspace_bytes(sh, n_max, k), dtype=torch.uint8, device=dev)
    out = torch.empty(w.B, n_q, w.Hq, w.d, dtype=torch.float32, device=dev)
    lse = torch.empty(w.B, n_q, w.Hq, dtype=torch.float32, device=dev)
    sel = torch.full((w.B, n_q, groups, T, width), -7, dtype=torch.int32, device=dev)
    cache = oracle.TreeCache(inp["K"], inp["V"], inp["W"], w.f, w.dtype)
    if mode == "prefill":
        R.recsa_prefill(sh, q, q_start, K, V, tree, k, out, lse, sel, width, ws)
        ref = oracle.prefill(inp["K"], inp["V"], inp["W"], inp["q"], q_start, w.f, k, w.dtype, w.theta, select_heads=Gs,
                             cache=cache)
    else:
        R.recsa_decode(sh, q, K, V, tree, w.L, k, out, lse, sel, width, ws)
        ref = oracle.decode(inp["K"], inp["V"], inp["W"], inp["q"], w.L, w.f, k, w.dtype, w.theta, select_heads=Gs,
                            cache=cache)
    torch.cuda.synchronize()
    out, lse, sel = out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()
    stats = {"match": 0, "replayed": 0}
    for (b, j, g), r in ref.items():
        n = q_start + j + 1 if mode == "prefill" else w.L
        rep = oracle_replayer(cache, inp["q"], w, k, b, j, g, n, mode == "prefill", Gs=Gs)
        st = check_unit(r, sel[b, j, g], out[b, j, g * Gs:(g + 1) * Gs], lse[b, j, g * Gs:(g + 1) * Gs],
                        TOL[w.dtype], where=f"select_heads {Gs} unit {(b, j, g)}", replay=rep)
        stats[st] += 1
    _say(f"select_heads {Gs} {mode}: {stats}")


# ------------------------------------------------------------------ exact ties

def _tie_inputs(kind, B, Hkv, Hq, d, L, dtype, seed, n_q):
    """Inputs whose group scores tie exactly at the selection boundary of every level.
    'zero': every key is 0, so every logit is 0 (the lowest-index candidates must be kept).
    'blocks': rotation off; the keys repeat whole f^2-token blocks drawn from three vectors, so
    every level-1 node under such a block has the same key and the level-2 nodes take three
    values: runs of equal scores straddle the k-th place at levels 1 and 2."""
    rng = np.random.default_rng(seed)
    std = 1.0 if dtype == "f32" else d ** -0.5

    def store(x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        if dtype == "bf16":
            from synthetic import bf16_bits
            return bf16_bits(x)
        return x
    if kind == "zero":
        K = np.zeros((B, Hkv, L, d), np.float32)
    else:
        base = rng.standard_normal((B, Hkv, 3, d)).astype(np.float32) * std
        pick = rng.integers(0, 3, (B, Hkv, -(-L // 256)))
        K = np.take_along_axis(base, np.repeat(pick, 256, axis=2)[..., :L, None].repeat(d, 3), axis=2)
    V = rng.standard_normal((B, Hkv, L, d)).astype(np.float32) * std
    q = rng.standard_normal((B, n_q, Hq, d)).astype(np.float32) * std
    W = (np.eye(d) + 0.05 / np.sqrt(d) * rng.standard_normal((d, d))).astype(np.float32)
    return {"K": store(K), "V": store(V), "q": store(q), "W": store(W)}


TIE_CASES = [
    # (kind, dtype, d, G, f, L, k per level)
    ("zero", "bf16", 128, 4, 16, 16 ** 3 * 2 + 77, [8, 8, 8]),
    ("zero", "f32", 64, 4, 16, 16 ** 3 + 300, [3, 20, 1]),
    ("zero", "bf16", 128, 8, 32, 32 ** 3 + 32 ** 2 + 50, [16, 20, 2]),  # level 1: 640 candidates
    ("zero", "bf16", 64, 2, 16, 4500, [0, 8, 16]),
    ("blocks", "bf16", 128, 4, 16, 16 ** 3 * 3 + 5, [8, 5, 8]),
    ("blocks", "f32", 64, 4, 16, 16 ** 3 + 19, [4, 7, 2]),
    ("blocks", "bf16", 128, 8, 16, 16 ** 3 * 2, [12, 20, 3]),
]


@pytest.mark.parametrize("case", TIE_CASES, ids=lambda c: f"{c[0]}_{c[1]}_d{c[2]}_G{c[3]}_f{c[4]}")
@pytest.mark.parametrize("mode", ["decode", "prefill", "prefill_wide"])
def test_exact_ties_keep_lowest_indices(case, mode):
    """Equal group scores at the k-th place: the kept sets must be exactly the oracle's (equal
    scores go to the lower candidate index); no near-tie allowance applies to exact ties.
    decode and prefill (300 positions) run a few waves per unit; prefill_wide (1100 positions x 2
    KV heads, over 2048 units) one wave per unit."""
    kind, dtype, d, G, f, L, k = case
    Hkv, n_q = 2, 4
    w = _w(f"tie_{kind}", B=1, Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, L=L, f=f, k=k[0], n_queries=n_q,
           theta=(1.0e6 if kind == "zero" else 0.0), seed=91)
    inp = _tie_inputs(kind, 1, Hkv, G * Hkv, d, L, dtype, 91, n_q if mode == "decode" else L)
    g = Gpu(w, inp)
    T = R.recsa_num_levels(L, f)
    kk = (k + [k[-1]] * T)[:T]
    if mode == "decode":
        res = g.decode(kk, L)
        units = [(0, j, h) for j in range(n_q) for h in range(Hkv)]
        ref = oracle.decode(inp["K"], inp["V"], inp["W"], inp["q"], L, f, kk, dtype, w.theta, units=units)
    else:
        n_p = 1100 if mode == "prefill_wide" else 300
        q_start = L - n_p
        res = g.prefill(kk, q_start, n_p)
        pos = [0, 1, 2, 15, 16, 17, 100, 255, 256, 299] + ([640, 1023, 1099] if n_p > 300 else [])
        units = [(0, p, h) for p in pos for h in range(Hkv)]
        ref = oracle.prefill(inp["K"], inp["V"], inp["W"], inp["q"][:, q_start:], q_start, f, kk, dtype, w.theta,
                             units=units)
    out, lse, sel, _ = res
    ties = 0
    for (b, j, h), r in ref.items():
        for lv in range(1, len(r.sel) + 1):
            cand, S = r.scores.get(lv, (None, None))
            s = len(r.sel[lv])
            if S is not None and 0 < s < len(S):
                Ss = np.sort(S)[::-1]
                ties += Ss[s - 1] == Ss[s]
        st, _fx = gpu_util.compare_unit(r, sel[b, j, h], out[b, j, h * G:(h + 1) * G], lse[b, j, h * G:(h + 1) * G],
                                        TOL[dtype], where=f"ties {case} {mode} unit {(b, j, h)}")
        assert st == "match"
    assert ties > 0, "no level had an exact tie at its boundary"
