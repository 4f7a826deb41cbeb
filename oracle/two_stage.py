"""Two-stage block-then-token selection over the RecSA cache -- plain CPU oracle.

TEST INFRASTRUCTURE ONLY. Imported by tests/; never by the product path.

Sources, cited by page title and section:
  [HISA]      "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse Attention" --
              its summary in a listing of related work: a coarse pass scores blocks of the
              cache and discards the irrelevant ones, then the token-level indexer runs only
              inside the blocks kept, and attention keeps the same top-k token pattern.
  [Abstract]  "Recursive Sparse Attention: Million-Token Length Extrapolation at
              Logarithmic Cost" -- abstract: a pooled key per node, RoPE positions as
              indices among a level's candidates.

Reading (the pages give no formulas for this variant): the blocks are the level-1 nodes of
the RecSA tree, f tokens each with the pooled key W @ mean(child keys); a one-level descent
without summaries:

  1. blocks: every complete block g < n_1 = floor(n / f) is a candidate at index g, the query
     at n_1; score S_g = sum over the group's heads of fp32(scale <rot(q_h, n_1), rot(NK_1[g], g)>);
     keep s_1 = min(k_block, n_1) blocks by (S desc, g asc); the others are dropped.
  2. tokens: the tokens of the kept blocks in ascending order, then the trailing tokens
     [f n_1, n), are candidates at their index i, the query at C_0; keep s_0 = min(k_token, C_0)
     tokens by the same rule; the others are dropped.
  3. one softmax per query head over the kept tokens only, with the logits of step 2.

Precision as the RecSA oracle: the logits that decide a selection are float64 dot products of
operands rounded to the storage type, times the float32 scale, rounded once to float32; group
scores, the softmax and the weighted sum are float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .recsa import (NEAR_TIE_REL, TreeCache, _logits, default_scale, from_storage, level_counts)

_F32 = np.float32
_F64 = np.float64


@dataclass
class TwoStageResult:
    out: np.ndarray                 # [G, d] float64
    lse: np.ndarray                 # [G] float64
    blocks: list = field(default_factory=list)   # kept block ids, ascending
    tokens: list = field(default_factory=list)   # kept token ids, ascending
    flags: dict = field(default_factory=dict)    # 1: block boundary near tie, 0: token boundary
    C0: int = 0                                   # token candidates
    z: np.ndarray | None = None                   # [s_0, G] float32 logits of the kept tokens


def _keep(z: np.ndarray, s: int):
    """Indices (ascending) of the s candidates with the highest group score, ties to the lower
    index, and whether the boundary is a near tie."""
    S = z.astype(_F64).sum(axis=0)
    C = S.shape[0]
    order = np.lexsort((np.arange(C), -S))
    flag = bool(0 < s < C and 0.0 < S[order[s - 1]] - S[order[s]] < NEAR_TIE_REL * np.abs(S).max())
    return np.sort(order[:s]), flag


def two_stage_unit(q: np.ndarray, K: np.ndarray, V: np.ndarray, NK1: np.ndarray, n: int, f: int,
                   k_block: int, k_token: int, dtype: str, theta: float = 1.0e6,
                   scale=None) -> TwoStageResult:
    """One decode query (its G heads, q [G, d] float32) at position n against one KV head's n
    cached tokens K, V [>= n, d] float32; NK1 [>= floor(n/f), d] float32 level-1 node keys."""
    G, d = q.shape
    scale32 = default_scale(d) if scale is None else _F32(scale)
    n1 = n // f
    res = TwoStageResult(out=np.zeros((G, d)), lse=np.full(G, -np.inf))
    kept_blocks = np.zeros(0, dtype=np.int64)
    if n1 > 0:
        z1 = _logits(q, NK1[:n1], n1, dtype, theta, scale32)            # [G, n1], block g at index g
        kept_blocks, res.flags[1] = _keep(z1, min(int(k_block), n1))
    res.blocks = [int(g) for g in kept_blocks]
    cand = np.array([f * g + j for g in res.blocks for j in range(f)] + list(range(f * n1, n)), dtype=np.int64)
    C0 = len(cand)
    res.C0 = C0
    if C0 == 0:
        return res
    z0 = _logits(q, K[cand], C0, dtype, theta, scale32)                 # [G, C0], query at C0
    kept, res.flags[0] = _keep(z0, min(int(k_token), C0))
    res.tokens = [int(cand[i]) for i in kept]
    if len(kept) == 0:
        return res
    Z = z0[:, kept].T.astype(_F32)                                      # [s0, G]
    res.z = Z
    Zd = Z.astype(_F64)
    m = Zd.max(axis=0)
    P = np.exp(Zd - m)
    l = P.sum(axis=0)
    res.out = (P.T @ V[cand[kept]].astype(_F64)) / l[:, None]
    res.lse = m + np.log(l)
    return res


def two_stage_decode(K, V, W, q, n_tokens: int, f: int, k_block: int, k_token: int, dtype: str,
                     theta: float = 1.0e6, scale=None, units=None, cache: TreeCache | None = None) -> dict:
    """Every query of q [B][n_q][Hq][d] (storage form) at position n_tokens over the first n_tokens
    tokens of K, V [B][Hkv][cap][d]; the G heads of a KV head select together.
    Returns {(b, j, h): TwoStageResult}."""
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    cache = cache or TreeCache(K, V, W, f, dtype)
    out = {}
    all_units = [(b, j, h) for b in range(B) for j in range(n_q) for h in range(Hkv)]
    for (b, j, h) in (units if units is not None else all_units):
        Kf, Vf, tree = cache.get(b, h, n_tokens)
        NK1 = tree[0][0] if level_counts(n_tokens, f) else np.zeros((0, d), _F32)
        qg = from_storage(q[b, j, h * G:(h + 1) * G], dtype)
        out[(b, j, h)] = two_stage_unit(qg, Kf, Vf, NK1, n_tokens, f, k_block, k_token, dtype, theta, scale)
    return out
