"""GPU parity of the two-stage block-then-token decode (recsa_two_stage_decode) against the oracle
on seeded inputs: kept blocks and kept tokens identical (a flagged near tie, relative score gap
below 1e-5, may split either way), outputs within 1e-5 of the largest output magnitude and the
log-sum-exp within 1e-5 absolute. The token logits and the softmax are float32 on both sides of
one rounding of the oracle's float64 sums, so the outputs agree to float32 accumulation error."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Gpu, storage_bits
from long_context_hierarchical_amd import recsa as R
from oracle.two_stage import two_stage_decode, two_stage_unit
from synthetic import WORKLOADS, Workload, gen_decode_inputs, gen_kv_slice, gen_queries, gen_W

pytestmark = pytest.mark.gpu
INT32_MAX = oracle.INT32_MAX
TOL = 1e-5


def _say(msg):
    print(msg, flush=True)


def _w(name, B=1, Hq=4, Hkv=1, d=64, dtype="f32", L=4096, f=16, n_queries=4, **kw):
    std = kw.pop("std", 1.0 if dtype == "f32" else d ** -0.5)
    return Workload(name, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, L=L, f=f, k=4, n_queries=n_queries,
                    mode="decode", std=std, **kw)


def _counts(n, f, kb, kt):
    n1 = n // f
    s1 = min(kb, n1)
    C0 = f * s1 + n - f * n1
    return s1, min(kt, C0)


def _run(g, n, kb, kt, block_keys=None):
    w, sh, dev = g.w, g.shape, g.dev
    n_q = g.q.shape[1]
    s1, s0 = _counts(n, w.f, kb, kt)
    out = torch.full((w.B, n_q, w.Hq, w.d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((w.B, n_q, w.Hq), float("nan"), dtype=torch.float32, device=dev)
    selb = torch.full((w.B, n_q, w.Hkv, max(s1, 1)), -7, dtype=torch.int32, device=dev)
    selt = torch.full((w.B, n_q, w.Hkv, max(s0, 1)), -7, dtype=torch.int32, device=dev)
    nb = R.recsa_two_stage_workspace_bytes(sh, n, n_q, kb, kt, block_keys is not None)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev)
    R.recsa_two_stage_decode(sh, g.q, g.K, g.V, g.tree, n, kb, kt, out, lse, selb, selt, block_keys=block_keys,
                             workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), selb.cpu().numpy(), selt.cpu().numpy()


def _ids(row, where):
    got = [int(x) for x in row if x >= 0]
    assert all(x == -1 for x in row[len(got):]), f"{where}: bad padding"
    return got


def _compare(w, res, ref, min_match=0.9):
    out, lse, selb, selt = res
    G = w.G
    stats = {"match": 0, "excused": 0}
    for (b, j, h), r in ref.items():
        where = f"{w.name} unit {(b, j, h)}"
        if _ids(selb[b, j, h], where) != r.blocks:
            assert r.flags.get(1), f"{where}: blocks {_ids(selb[b, j, h], where)} vs oracle {r.blocks}"
            stats["excused"] += 1
            continue
        if _ids(selt[b, j, h], where) != r.tokens:
            assert r.flags.get(0), f"{where}: tokens differ from the oracle's"
            stats["excused"] += 1
            continue
        o, l = out[b, j, h * G:(h + 1) * G], lse[b, j, h * G:(h + 1) * G]
        if r.z is None:
            assert np.all(o == 0) and np.all(np.isneginf(l)), where
        else:
            scale = max(float(np.abs(r.out).max()), 1e-30)
            err = float(np.abs(o.astype(np.float64) - r.out).max())
            assert err <= TOL * scale, f"{where}: max |out - oracle| = {err:.3g} (scale {scale:.3g})"
            assert float(np.abs(l.astype(np.float64) - r.lse).max()) <= TOL, where
        stats["match"] += 1
    assert stats["match"] >= min_match * len(ref), stats
    return stats


# (workload, k_block, k_token)
CASES = [
    # 4000 blocks: four stage-1 slabs (1024, 1024, 1024, 928), merged
    (_w("ts_bf16_d128_G4_f16_slabs", Hq=8, Hkv=2, d=128, dtype="bf16", L=16 * 4000 + 5, n_queries=5, seed=81), 16, 100),
    (_w("ts_f32_d64_G2_f4", B=2, Hq=4, Hkv=2, d=64, dtype="f32", L=3001, f=4, n_queries=4, seed=82), 6, 13),
    (_w("ts_bf16_d128_G8_f32_keep_tokens", Hq=8, Hkv=1, d=128, dtype="bf16", L=32 * 300 + 31, f=32, n_queries=3,
        seed=83), 5, INT32_MAX),
    (_w("ts_bf16_d64_G1_keep_blocks", Hq=2, Hkv=2, d=64, dtype="bf16", L=16 * 20 + 7, n_queries=3, seed=84), 100, 50),
    (_w("ts_bf16_d128_G4_norope", Hq=4, Hkv=1, d=128, dtype="bf16", L=16 * 700 + 15, n_queries=4, theta=0.0,
        seed=85), 12, 64),
    (_w("ts_f32_d128_G4_f16", Hq=4, Hkv=1, d=128, dtype="f32", L=16 * 1500 + 2, n_queries=3, seed=86), 9, 70),
    (_w("ts_bf16_d128_G2_f16", B=2, Hq=4, Hkv=2, d=128, dtype="bf16", L=16 * 2500 + 11, n_queries=2, seed=87), 24, 200),
]


@pytest.mark.parametrize("w,kb,kt", CASES, ids=lambda c: c.name if hasattr(c, "name") else str(c))
def test_two_stage_matches_oracle(w, kb, kt):
    _say(f"two-stage {w.name}: gpu")
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    res = _run(g, w.L, kb, kt)
    _say(f"two-stage {w.name}: oracle")
    ref = two_stage_decode(inp["K"], inp["V"], inp["W"], inp["q"], w.L, w.f, kb, kt, w.dtype, w.theta)
    _say(f"two-stage {w.name}: {_compare(w, res, ref)}")


def test_two_stage_edge_cases():
    """Shorter prefixes of one cache: no token, fewer than f tokens (no block), k_block = 0 (only
    the trailing tokens), k_token = 0 (nothing kept), one block exactly, and everything kept."""
    w = _w("ts_edges", Hq=8, Hkv=2, d=64, dtype="bf16", L=16 * 50 + 9, n_queries=2, seed=88)
    inp = gen_decode_inputs(w)
    g = Gpu(w, inp)
    for n, kb, kt in [(0, 4, 4), (9, 4, 4), (16 * 30 + 3, 0, 10), (16 * 30 + 3, 3, 0), (16, 1, 5),
                      (16 * 50 + 9, INT32_MAX, INT32_MAX), (16 * 50 + 9, 50, 809)]:
        _say(f"two-stage edges: n={n} k_block={kb} k_token={kt}")
        res = _run(g, n, kb, kt)
        ref = two_stage_decode(inp["K"], inp["V"], inp["W"], inp["q"], n, w.f, kb, kt, w.dtype, w.theta)
        _compare(w, res, ref, min_match=1.0)


def test_two_stage_exact_ties():
    """Exact ties everywhere (no rotation; every third block's tokens share one key, the rest are
    zero): block scores and token logits take two values, so each selection keeps the lowest
    indices among equal scores -- through the selections' all-equal path and their fallback for a
    bin too full to rank -- exactly as the oracle's (score, index) order does."""
    w = _w("ts_ties", Hq=8, Hkv=2, d=64, dtype="bf16", L=16 * 3000 + 5, n_queries=3, theta=0.0, seed=89)
    inp = gen_decode_inputs(w)
    rng = np.random.default_rng(7)
    c = (rng.standard_normal(w.d) * 0.3).astype(np.float32)
    cb = (c.view(np.uint32) >> 16).astype(np.uint16)      # bf16 bits (truncation: any bf16 value will do)
    K = np.zeros_like(inp["K"])
    for g0 in range(0, 3000, 3):
        K[:, :, 16 * g0:16 * (g0 + 1)] = cb
    inp["K"] = K
    g = Gpu(w, inp)
    for kb, kt in [(100, 700), (120, 1900), (7, 50)]:
        _say(f"two-stage ties: k_block={kb} k_token={kt}")
        res = _run(g, w.L, kb, kt)
        ref = two_stage_decode(inp["K"], inp["V"], inp["W"], inp["q"], w.L, w.f, kb, kt, w.dtype, w.theta)
        _compare(w, res, ref, min_match=1.0)


def test_two_stage_rotated_block_cache():
    """A cache of rotated block keys filled in two increments gives bit for bit the outputs of the
    call that rotates them into its workspace, and holds exactly the rotated level-1 keys."""
    w = CASES[0][0]
    inp = gen_decode_inputs(w, n_q=2)
    g = Gpu(w, inp)
    sh = g.shape
    rows = w.L // w.f
    bk = torch.zeros((w.B, w.Hkv, rows, w.d), dtype=torch.bfloat16, device=g.dev)
    R.recsa_two_stage_rotate_blocks(sh, g.tree, 0, w.L // 2, bk)
    R.recsa_two_stage_rotate_blocks(sh, g.tree, w.L // 2, w.L, bk)
    a = _run(g, w.L, 16, 100)
    b = _run(g, w.L, 16, 100, block_keys=bk)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)
    NK, _ = R.tree_level_views(sh, g.tree, 1)
    c, s = oracle.rope_rows(np.arange(rows), w.d, w.theta)
    for h in range(w.Hkv):
        want = oracle.rotate(oracle.from_storage(storage_bits(NK[0, h]), w.dtype), c, s, w.dtype)
        assert np.array_equal(storage_bits(bk[0, h]), oracle.to_storage(want, w.dtype)), h


def _full_size(name, n_q, kb, kt, checked_queries):
    """One workload at full size in the configuration the benchmark times: spawned workers
    regenerate every (sequence, KV head) slice (uploaded as it arrives), build its level 1 and run
    the oracle's two-stage selection for the checked queries of that slice."""
    import oracle_pool as OP
    w = WORKLOADS[name]
    dev = "cuda:0"
    td = torch.bfloat16
    K = torch.empty(w.B, w.Hkv, w.L, w.d, dtype=td, device=dev)
    V = torch.empty_like(K)

    def up(r):
        b, h = r["slice"]
        K[b, h] = torch.from_numpy(r["K"]).view(td).to(dev)
        V[b, h] = torch.from_numpy(r["V"]).view(td).to(dev)
        _say(f"two-stage {name}: slice {(b, h)} uploaded, oracle done")
    jobs = [dict(workload=name, slice=(b, h), n_q=n_q, return_kv=True,
                 ts_units=[(j, kb, kt) for j in checked_queries]) for b in range(w.B) for h in range(w.Hkv)]
    res = OP.run_slices(jobs, on_result=up)
    qs = np.stack([gen_queries(w, b, n_q) for b in range(w.B)])
    Wn = gen_W(w)
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
    tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device=dev)
    R.recsa_build_tree(sh, K, V, torch.from_numpy(Wn).view(td).to(dev), 0, w.L, tree)

    class _G:
        pass
    g = _G()
    g.w, g.shape, g.dev, g.q, g.K, g.V, g.tree = w, sh, dev, torch.from_numpy(qs).view(td).to(dev), K, V, tree
    out = _run(g, w.L, kb, kt)
    _say(f"two-stage {name}: gpu done")
    ref = {(b, j, h): OP.Slim(r["ts_units"][(j, kb, kt)]) for (b, h), r in res.items() for j in checked_queries}
    _say(f"two-stage {name}: {_compare(w, out, ref)}")


def test_two_stage_full_size_524k():
    """The 524K workload's shape (4 sequences x 524,288 tokens, 8 KV heads, 32 query heads, d = 128,
    bf16, f = 16) with 128 blocks and 512 tokens kept, 256 queries per sequence in one call -- the
    configuration the benchmark times; the oracle checks 8 queries of every (sequence, KV head)."""
    _full_size("c2", 256, 128, 512, (0, 31, 64, 100, 127, 128, 200, 255))


def test_two_stage_full_size_2m():
    """The 2M workload's shape (2,097,152 tokens, 8 KV heads, 32 query heads, d = 128, bf16,
    f = 32): 65,536 blocks per slice, 64 slabs whose lists merge into 8192 candidates per query
    (more than 64 KB of LDS for the merge); 16 queries, the oracle checks 4 of every KV head."""
    _full_size("c4", 16, 128, 512, (0, 5, 10, 15))
