"""Float64 brute force for RecSA tree attention on tiny inputs.

An independent formulation used to pin the oracle, sharing no code with it:
  * node summaries from their token spans: value = mean of the span's token
    values, key = W^l @ mean of the span's keys (the level-by-level pooler
    is linear, so this equals pooling the children level by level);
  * candidates as a mask over every node of a level: a node is a candidate
    when it has no complete parent or its parent was kept one level up;
    its RoPE position is its rank within the mask;
  * RoPE as complex multiplication of the pairs (x_i, x_{i+d/2});
  * selection by sorting (-score, position) with Python's sorted();
  * softmax through scipy's logsumexp.
No rounding to float32 or bf16 anywhere.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def freqs(d: int, theta: float) -> np.ndarray:
    # inverse frequencies kept in float32, as the build defines them
    return np.float32(theta) ** (-(2.0 * np.arange(d // 2)) / d)


def rot(x: np.ndarray, p: int, theta: float) -> np.ndarray:
    if theta == 0.0:
        return np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    om = np.asarray(freqs(x.shape[-1], theta), dtype=np.float32).astype(np.float64)
    zc = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * float(p) * om)
    return np.concatenate([zc.real, zc.imag], axis=-1)


def brute_unit(q, K, V, W, n, f, k_levels, theta=1.0e6, scale=None, self_in=False, fixed_sel=None):
    """Returns dict(out [G,d], lse [G], sel {level: sorted ids}, gap {level: relative boundary gap},
    entries [(level, id)]). fixed_sel {level: kept ids} replaces the selection by scores at the
    levels it lists (with every level listed: the function of q, K, V and W that gradients with
    held selections differentiate)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    W = np.asarray(W, np.float64)
    G, d = q.shape
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    T = 0
    while f ** (T + 1) <= n:
        T += 1
    kept = set()
    zs, vals, entries = [], [], []
    sel, gap = {}, {}
    for lv in range(T, 0, -1):
        span = f ** lv
        N = n // span
        n_up = n // (f * span) if lv < T else 0
        cands = [g for g in range(N) if lv == T or g >= f * n_up or (g // f) in kept]
        C = len(cands)
        Wl = np.linalg.matrix_power(W, lv)
        S, zmap = {}, {}
        for i, g in enumerate(cands):
            key = Wl @ K[g * span:(g + 1) * span].mean(axis=0)
            z = np.array([sc * np.dot(rot(q[h], C, theta), rot(key, i, theta)) for h in range(G)])
            zmap[g] = z
            S[g] = z.sum()
        if fixed_sel is not None and lv in fixed_sel:
            kept = set(fixed_sel[lv])
            rest = [i for i in range(C) if cands[i] not in kept]
        else:
            s = min(int(k_levels[lv - 1]), C)
            order = sorted(range(C), key=lambda i: (-S[cands[i]], i))
            if 0 < s < C:
                mx = max(abs(v) for v in S.values())
                gap[lv] = (S[cands[order[s - 1]]] - S[cands[order[s]]]) / mx if mx > 0 else 0.0
            kept = {cands[i] for i in order[:s]}
            rest = sorted(order[s:])
        sel[lv] = sorted(kept)
        for i in rest:
            g = cands[i]
            entries.append((lv, g))
            zs.append(zmap[g])
            vals.append(V[g * span:(g + 1) * span].mean(axis=0))
    toks = [t for t in range(n) if T == 0 or t >= f * (n // f) or (t // f) in kept]
    C0 = len(toks)
    pq = C0 - 1 if (self_in and C0 and toks[-1] == n - 1) else C0
    for i, t in enumerate(toks):
        entries.append((0, t))
        zs.append(np.array([sc * np.dot(rot(q[h], pq, theta), rot(K[t], i, theta)) for h in range(G)]))
        vals.append(V[t])
    if not zs:
        return dict(out=np.zeros((G, d)), lse=np.full(G, -np.inf), sel=sel, gap=gap, entries=entries)
    Z = np.array(zs)                       # [E, G]
    lse = logsumexp(Z, axis=0)
    Wt = np.exp(Z - lse)
    out = Wt.T @ np.array(vals)
    return dict(out=out, lse=lse, sel=sel, gap=gap, entries=entries)


def dense_textbook(q, K, V, n_keys, q_pos, theta=1.0e6, scale=None):
    """Standard RoPE softmax attention in float64: keys 0..n_keys-1 at their positions."""
    q = np.asarray(q, np.float64)
    G, d = q.shape
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    Kr = np.stack([rot(np.asarray(K[t], np.float64), t, theta) for t in range(n_keys)])
    Qr = np.stack([rot(q[h], q_pos, theta) for h in range(G)])
    Z = sc * Qr @ Kr.T                     # [G, n]
    lse = logsumexp(Z, axis=1)
    return np.exp(Z - lse[:, None]) @ np.asarray(V[:n_keys], np.float64), lse


def brute_two_stage(q, K, V, W, n, f, k_block, k_token, theta=1.0e6, scale=None):
    """Two-stage block-then-token selection in float64 from its definition: block g (tokens
    g f .. g f + f - 1) has key W @ mean(its token keys) at position g, the query at the number
    of blocks; the kept blocks' tokens and the trailing tokens are candidates at their rank, the
    query at their count; each stage keeps its best k by (-score, position); one softmax over the
    kept tokens. Returns dict(out, lse, blocks, tokens, gap {1: block gap, 0: token gap})."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    W = np.asarray(W, np.float64)
    G, d = q.shape
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    nb = n // f
    gap = {}

    def pick(S, k):
        order = sorted(range(len(S)), key=lambda i: (-S[i], i))
        s = min(k, len(S))
        if 0 < s < len(S):
            mx = max(abs(v) for v in S)
            gap_v = (S[order[s - 1]] - S[order[s]]) / mx if mx > 0 else 0.0
        else:
            gap_v = None
        return sorted(order[:s]), gap_v

    Sb = []
    for g in range(nb):
        key = W @ K[g * f:(g + 1) * f].mean(axis=0)
        Sb.append(sum(sc * np.dot(rot(q[h], nb, theta), rot(key, g, theta)) for h in range(G)))
    blocks, gap[1] = pick(Sb, k_block)
    kept = set(blocks)
    toks = [t for t in range(n) if t >= f * nb or (t // f) in kept]
    C0 = len(toks)
    Z = np.array([[sc * np.dot(rot(q[h], C0, theta), rot(K[t], i, theta)) for h in range(G)]
                  for i, t in enumerate(toks)]).reshape(C0, G)
    chosen, gap[0] = pick(list(Z.sum(axis=1)), k_token)
    tokens = [toks[i] for i in chosen]
    if not chosen:
        return dict(out=np.zeros((G, d)), lse=np.full(G, -np.inf), blocks=blocks, tokens=tokens, gap=gap)
    Zk = Z[chosen]                         # [s0, G]
    lse = logsumexp(Zk, axis=0)
    out = np.exp(Zk - lse).T @ V[tokens]
    return dict(out=out, lse=lse, blocks=blocks, tokens=tokens, gap=gap)
