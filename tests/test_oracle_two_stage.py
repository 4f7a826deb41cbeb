"""Pins for the two-stage (block-then-token) oracle against facts that do not come from it:
an independent float64 brute force, dense attention (the no-pruning limit), the RecSA oracle
on one-level trees (same blocks, same token logits), a planted needle and the empty cases."""
import numpy as np
import pytest

from oracle import INT32_MAX, attend_unit, build_slice, dense_unit
from oracle.two_stage import two_stage_unit
from brute64 import brute_two_stage, dense_textbook
from synthetic import bf16_bits, bf16_value


def _rand(rng, shape, std=1.0, dtype="f32"):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return bf16_value(bf16_bits(x)) if dtype == "bf16" else x


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    f = int(rng.choice([2, 4, 16]))
    d = int(rng.choice([8, 16, 64]))
    G = int(rng.choice([1, 2, 4]))
    theta = float(rng.choice([0.0, 50.0, 1.0e6]))
    n = int(rng.integers(0, 700 if f < 16 else 3000))
    n1 = n // f
    k_block = int(rng.integers(0, max(n1, 1) + 2))
    k_token = int(rng.integers(0, f * k_block + f + 3))
    if rng.random() < 0.15:
        k_block = INT32_MAX
    if rng.random() < 0.15:
        k_token = INT32_MAX
    K = _rand(rng, (max(n, 1), d))
    V = _rand(rng, (max(n, 1), d))
    q = _rand(rng, (G, d))
    W = (np.eye(d) + 0.3 / np.sqrt(d) * rng.standard_normal((d, d))).astype(np.float32)
    return f, d, G, theta, n, k_block, k_token, K, V, q, W


def _oracle(K, V, W, q, n, f, kb, kt, dtype="f32", theta=1.0e6):
    tree = build_slice(K, V, W, f, dtype, n_new=n)
    NK1 = tree[0][0] if tree else np.zeros((0, K.shape[1]), np.float32)
    return two_stage_unit(q, K, V, NK1, n, f, kb, kt, dtype, theta)


@pytest.mark.parametrize("seed", range(40))
def test_two_stage_matches_float64_brute_force(seed):
    """Both stages (f32 storage) vs the brute force: equal blocks and tokens unless either side
    sees a near tie at a boundary; outputs and log-sum-exp within 1e-6."""
    f, d, G, theta, n, kb, kt, K, V, q, W = _case(seed)
    r = _oracle(K, V, W, q, n, f, kb, kt, theta=theta)
    b = brute_two_stage(q, K, V, W, n, f, kb, kt, theta)
    if r.flags.get(1) or (b["gap"][1] is not None and b["gap"][1] < 1e-5):
        pytest.skip("near tie between blocks")
    assert r.blocks == b["blocks"]
    if r.flags.get(0) or (b["gap"][0] is not None and b["gap"][0] < 1e-5):
        pytest.skip("near tie between tokens")
    assert r.tokens == b["tokens"]
    np.testing.assert_allclose(r.out, b["out"], rtol=0, atol=1e-6)
    np.testing.assert_allclose(r.lse, b["lse"], rtol=0, atol=1e-6)


def test_brute_force_cases_mostly_compared():
    """Guard against the comparison above skipping everything."""
    compared = 0
    for seed in range(40):
        f, d, G, theta, n, kb, kt, K, V, q, W = _case(seed)
        r = _oracle(K, V, W, q, n, f, kb, kt, theta=theta)
        compared += not (r.flags.get(1) or r.flags.get(0))
    assert compared >= 36


@pytest.mark.parametrize("n,f,theta", [(1000, 16, 1.0e6), (517, 4, 50.0), (5, 16, 1.0e6), (64, 2, 0.0)])
def test_no_pruning_is_dense_attention(n, f, theta):
    """Keeping every block and every token makes the candidates all tokens in order, each at its
    own position and the query at n: plain RoPE attention (float64 textbook, and the oracle's
    dense path on the same float32 logits)."""
    rng = np.random.default_rng(n)
    d, G = 64, 4
    K, V, q = _rand(rng, (n, d)), _rand(rng, (n, d)), _rand(rng, (G, d))
    W = (np.eye(d) + 0.05 * rng.standard_normal((d, d))).astype(np.float32)
    r = _oracle(K, V, W, q, n, f, INT32_MAX, INT32_MAX, theta=theta)
    assert r.tokens == list(range(n))
    out, lse = dense_textbook(q, K, V, n, n, theta)
    np.testing.assert_allclose(r.out, out, rtol=0, atol=1e-6)
    np.testing.assert_allclose(r.lse, lse, rtol=0, atol=1e-6)
    o2, l2 = dense_unit(q, K, V, n, n, "f32", theta)
    np.testing.assert_allclose(r.out, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r.lse, l2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,kb", [(16 * 15 + 7, 5), (16 * 16 - 1, 3), (16 * 9, 16), (16 * 12, 1)])
def test_one_level_tree_agrees_with_recsa(dtype, n, kb):
    """With one tree level (f <= n < f^2) the block stage is RecSA's level-1 selection, and with
    every token candidate kept the token logits are RecSA's level-0 logits: the output is RecSA's
    softmax with the summary entries removed."""
    f, d, G = 16, 64, 4
    rng = np.random.default_rng(n + kb)
    K, V, q = _rand(rng, (n, d), dtype=dtype), _rand(rng, (n, d), dtype=dtype), _rand(rng, (G, d), dtype=dtype)
    W = _rand(rng, (d, d), 0.05, dtype) + np.eye(d, dtype=np.float32)
    tree = build_slice(K, V, W, f, dtype, n_new=n)
    rec = attend_unit(q, K, V, tree, n, f, [kb], dtype)
    r = two_stage_unit(q, K, V, tree[0][0], n, f, kb, INT32_MAX, dtype)
    assert r.blocks == rec.sel[1]
    tok = [e for e, (lv, _) in enumerate(rec.entries) if lv == 0]
    assert r.tokens == [rec.entries[e][1] for e in tok]
    assert np.array_equal(r.z, rec.z[tok])
    Z = rec.z[tok].astype(np.float64)
    P = np.exp(Z - Z.max(axis=0))
    out = (P.T @ V[r.tokens].astype(np.float64)) / P.sum(axis=0)[:, None]
    np.testing.assert_allclose(r.out, out, rtol=0, atol=1e-12)


def test_planted_needle_is_found():
    """A block whose tokens point along the query is kept, and within it the needle token, whose
    value then dominates the output (no rotation, so the logit is the plain dot product)."""
    rng = np.random.default_rng(5)
    f, d, G, n = 16, 64, 4, 16 * 200 + 5
    K = _rand(rng, (n, d), 0.1)
    V = _rand(rng, (n, d), 0.1)
    u = _rand(rng, (d,))
    u /= np.linalg.norm(u)
    q = np.tile(8.0 * u, (G, 1)).astype(np.float32)
    blk, tok = 137, 137 * 16 + 9
    K[blk * 16:(blk + 1) * 16] += 0.5 * u
    K[tok] += 6.0 * u
    V[tok] = 5.0
    W = np.eye(d, dtype=np.float32)
    r = _oracle(K, V, W, q, n, f, 4, 8, theta=0.0)
    assert blk in r.blocks and tok in r.tokens
    assert np.all(r.out > 4.0)


def test_empty_and_degenerate_cases():
    """No tokens: nothing to attend (out 0, lse -inf). Fewer than f tokens: no block, every token
    a candidate. k_block = 0: only the trailing tokens. k_token = 0: no entry."""
    rng = np.random.default_rng(11)
    d, G, f = 16, 2, 4
    K, V, q = _rand(rng, (50, d)), _rand(rng, (50, d)), _rand(rng, (G, d))
    W = np.eye(d, dtype=np.float32)
    r = _oracle(K, V, W, q, 0, f, 3, 3)
    assert r.C0 == 0 and np.all(r.out == 0) and np.all(np.isneginf(r.lse))
    r = _oracle(K, V, W, q, 3, f, 3, INT32_MAX)
    assert r.blocks == [] and r.tokens == [0, 1, 2]
    r = _oracle(K, V, W, q, 43, f, 0, INT32_MAX)
    assert r.blocks == [] and r.tokens == [40, 41, 42]
    r = _oracle(K, V, W, q, 43, f, 2, 0)
    assert len(r.blocks) == 2 and r.C0 == 11 and r.tokens == [] and np.all(np.isneginf(r.lse))
