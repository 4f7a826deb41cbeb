"""RecSA tree attention: plain CPU oracle.

TEST INFRASTRUCTURE ONLY. Imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; never by the product path, which has no CPU
fallback.

Sources, cited by page title and section:
  [Abstract]  "Recursive Sparse Attention: Million-Token Length Extrapolation
              at Logarithmic Cost" -- abstract (概要).
  [Core Idea] "Recursive Sparse Attention RecSA: Million-Token Context
              Extrapolation at Logarithmic Cost" -- section "Core Idea:
              Compressing the KV Cache with a Tree Structure".
  [Position]  the same page -- section "Position Encoding Ingenuity: Making
              Extrapolation Possible".

What the pages fix: a tree is kept over the KV cache, a node holding a
pooled key and the average of the values below it [Abstract, Core Idea]; the
same pooler serves every level of a layer [Abstract]; going down the tree a
query retains no more than k candidates at each level above the tokens
[Abstract, Core Idea]; the summaries it drops are not lost but are weighted in
the same softmax as the token rows it reaches [Abstract]; RoPE is applied at a
row's rank within its level's candidate list rather than at its token
position [Abstract, Position].

Readings where the pages are silent (all are listed in the design notes):
complete-node forest with orphans and an exact trailing block; pooler
key = W @ mean(child keys) applied level by level; pre-RoPE cache;
score = the scaled RoPE'd logit summed over the query heads of a KV group;
ties broken by lowest candidate index; the query sits at position C_l (at
the token level C_0 - 1 when its own token is an exact candidate); rotate-half
RoPE with fp32 inverse frequencies; scale 1/sqrt(d); no size bias.

Precision. Steps whose rounding decides a selection follow the kernel's
precision with explicit rounding points, so both sides take each decision on
the same numbers: node sums in float32 in child order, divided by f, the
pooler's product accumulated in float32 input by input with one fused
multiply-add (one rounding) per term, results rounded to the storage type; the rotation with
separate multiply and add, rounded to the storage type; the logit is the
float64 dot product of the rounded operands times the float32 scale,
rounded once to float32. The group score, the softmax and the weighted value
sum decide nothing and are computed in float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

INT32_MAX = 2 ** 31 - 1
NEAR_TIE_REL = 1e-5
_F32 = np.float32
_F64 = np.float64


# ----------------------------------------------------------------- storage

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, ties to even (returned as float32)."""
    x = np.ascontiguousarray(x, dtype=_F32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(_F32).reshape(x.shape)


def round_store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type ('f32' is the identity)."""
    x = np.asarray(x, dtype=_F32)
    return bf16_round(x) if dtype == "bf16" else x


def from_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (float32, or bf16 bit patterns as uint16) -> float32 values."""
    if dtype == "bf16":
        a = np.ascontiguousarray(a)
        return (a.astype(np.uint32) << 16).view(_F32).reshape(a.shape)
    return np.asarray(a, dtype=_F32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values exact in the storage type -> storage form."""
    x = np.ascontiguousarray(x, dtype=_F32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16).reshape(x.shape)
    return x


# ----------------------------------------------------------------- tree shape

def level_counts(n: int, f: int) -> list[int]:
    """[n_1, ..., n_T]: complete nodes per level over n tokens, n_l = floor(n / f^l).

    Reading of [Abstract]/[Core Idea] (depth grows with log L): a node exists
    once all f of its children exist; T is the highest level with a node.
    """
    out, m = [], n // f
    while m >= 1:
        out.append(m)
        m //= f
    return out


def plan_counts(n: int, f: int, k_levels, self_in: bool = False):
    """Closed-form candidate and selection counts (they do not depend on the data).

    Returns (C, s, C0): dicts level -> C_l and level -> s_l for l = 1..T, and C_0.
    C_T = n_T; C_l = f * s_{l+1} + (n_l - f * n_{l+1}); s_l = min(k_l, C_l);
    C_0 = f * s_1 + (n - f * n_1)  [Abstract: at most k kept per level].
    """
    nl = level_counts(n, f)
    T = len(nl)
    C, s = {}, {}
    s_up, n_up = 0, 0
    for lv in range(T, 0, -1):
        C[lv] = f * s_up + (nl[lv - 1] - f * n_up)
        s[lv] = min(int(k_levels[lv - 1]), C[lv])
        s_up, n_up = s[lv], nl[lv - 1]
    C0 = (f * s_up + (n - f * n_up)) if T else n
    return C, s, C0


# ----------------------------------------------------------------- tree build

def pool_nodes(cK: np.ndarray, cV: np.ndarray, W: np.ndarray, f: int, dtype: str):
    """Summaries of g complete nodes from their stored children, in child order.

    [Abstract]: a node carries a key produced by the layer's pooler and a value
    that averages what lies below it; [Core Idea]: that value is the average of
    the token values of the node's span. Reading: key = W @ m with m the mean of the
    f child keys; value = mean of the f stored child values (equal to the
    subtree mean for a complete subtree).

    Arithmetic (oracle/csrc/pool.c, plain C): child sums in float32 in child
    order, one division by f, then key_i accumulated over j = 0..d-1 as
    acc = fmaf(W[i][j], m[j], acc) (one rounding per term), rounded to the
    storage type.

    cK, cV: [g, f, d] float32; W: [d, d] float32 (key_i = sum_j W[i, j] m_j).
    """
    from . import _native
    return _native.pool(cK, cV, W, f, dtype == "bf16")


def build_slice(K: np.ndarray, V: np.ndarray, W: np.ndarray, f: int, dtype: str,
                n_new: int, n_old: int = 0, tree=None, cap: int | None = None):
    """Build every node of one (sequence, KV head) that is complete at n_new but not at n_old.

    K, V: [>= n_new, d] float32 token rows (pre-RoPE); W: [d, d] float32.
    tree: list over levels l = 1.. of (NK_l, NV_l) float32 arrays sized floor(cap / f^l);
    nodes already present are never changed. Level l >= 2 pools the stored
    level l-1 nodes with the same pooler [Abstract: one pooler for every level].
    """
    d = K.shape[1]
    cap = n_new if cap is None else cap
    caps = level_counts(cap, f)
    if tree is None:
        tree = [(np.zeros((c, d), _F32), np.zeros((c, d), _F32)) for c in caps]
    for lv in range(1, len(level_counts(n_new, f)) + 1):
        lo, hi = n_old // f ** lv, n_new // f ** lv
        if hi <= lo:
            continue
        srcK, srcV = (K, V) if lv == 1 else tree[lv - 2]
        cK = srcK[lo * f:hi * f].reshape(hi - lo, f, d)
        cV = srcV[lo * f:hi * f].reshape(hi - lo, f, d)
        NK, NV = pool_nodes(cK, cV, W, f, dtype)
        tree[lv - 1][0][lo:hi] = NK
        tree[lv - 1][1][lo:hi] = NV
    return tree


# ----------------------------------------------------------------- RoPE

def inv_freq(d: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/d), i < d/2, evaluated in float64 and kept as float32 (reading)."""
    return np.array([math.pow(theta, -2.0 * i / d) for i in range(d // 2)], dtype=_F32)


def rope_rows(pos: np.ndarray, d: int, theta: float):
    """(cos, sin) float32 [len(pos), d/2] at integer positions: cos(p * omega_i) in float64, rounded once."""
    ang = np.asarray(pos, dtype=_F64)[:, None] * inv_freq(d, theta).astype(_F64)[None, :]
    return np.cos(ang).astype(_F32), np.sin(ang).astype(_F32)


_TABLES: dict = {}


def rope_table(P: int, d: int, theta: float):
    """(cos, sin) for positions 0..P (cached)."""
    key = (d, float(theta))
    t = _TABLES.get(key)
    if t is None or t[0].shape[0] < P + 1:
        t = rope_rows(np.arange(max(P, 1023) + 1), d, theta)
        _TABLES[key] = t
    return t[0][:P + 1], t[1][:P + 1]


def rotate(x: np.ndarray, c: np.ndarray, s: np.ndarray, dtype: str) -> np.ndarray:
    """Rotate-half RoPE of rows x [..., d] by (c, s) [..., d/2], rounded to the storage type.

    [Position]: a rotation whose angle grows with the position, so that the
    logit depends only on the position difference. Pairs (i, i + d/2);
    out_i = x_i c - x_{i+d/2} s, out_{i+d/2} = x_{i+d/2} c + x_i s, each
    product and sum rounded to float32 separately.
    """
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    o1 = x1 * c - x2 * s
    o2 = x2 * c + x1 * s
    return round_store(np.concatenate([o1, o2], axis=-1), dtype)


def _logits(q: np.ndarray, rows: np.ndarray, q_pos: int, dtype: str, theta: float,
            scale32: np.float32, row_pos=None) -> np.ndarray:
    """z[h, i] = fp32(scale * <rot(q_h, q_pos), rot(row_i, pos_i)>), pos_i = i unless given."""
    C, d = rows.shape
    if theta == 0.0:
        kt, qt = rows, q
    else:
        if row_pos is None:
            c, s = rope_table(max(C - 1, q_pos), d, theta)
            kt = rotate(rows, c[:C], s[:C], dtype)
            qt = rotate(q, c[q_pos][None, :], s[q_pos][None, :], dtype)
        else:
            c, s = rope_rows(row_pos, d, theta)
            kt = rotate(rows, c, s, dtype)
            cq, sq = rope_rows(np.array([q_pos]), d, theta)
            qt = rotate(q, cq, sq, dtype)
    dot = qt.astype(_F64) @ kt.astype(_F64).T
    return (dot * _F64(scale32)).astype(_F32)


def default_scale(d: int) -> np.float32:
    return _F32(1.0 / math.sqrt(d))


# ----------------------------------------------------------------- descent + softmax

@dataclass
class UnitResult:
    out: np.ndarray                     # [G, d] float64
    lse: np.ndarray                     # [G] float64
    sel: dict = field(default_factory=dict)       # level -> ascending selected node ids
    flags: dict = field(default_factory=dict)     # level -> near tie at the selection boundary
    C: dict = field(default_factory=dict)         # level -> candidate count (level 0 included)
    entries: list = field(default_factory=list)   # (level, node or token id) per softmax entry
    epos: list = field(default_factory=list)      # each entry's rank in its level's candidate list
    z: np.ndarray | None = None                   # [E, G] float32 logits of the entries
    weights: np.ndarray | None = None             # [E, G] float64 softmax weights
    q_pos: dict = field(default_factory=dict)     # level -> query RoPE position
    scores: dict = field(default_factory=dict)    # level -> (candidate ids, float64 group scores)


def attend_unit(q: np.ndarray, K: np.ndarray, V: np.ndarray, tree, n: int, f: int, k_levels,
                dtype: str, theta: float = 1.0e6, scale=None, self_in: bool = False,
                fixed_sel: dict | None = None) -> UnitResult:
    """One query token against one KV head's cache of n tokens (RecSA descent + one softmax).

    q: [G, d] float32 (the G query heads sharing this KV head); K, V: [>= n, d]
    float32 token rows; tree: levels with every node complete at n built.
    self_in: the query's own token is token n - 1 (causal prefill).

    Steps [Abstract, Core Idea]: start from every node of the top level; at
    each level l the candidates are the children of the nodes kept at l + 1
    (in ascending node order), followed by the orphan nodes that have no
    complete parent; each candidate's key is rotated at its index among the
    candidates [Abstract, Position], the query at C_l; the s_l = min(k_l, C_l)
    candidates with the highest group score are kept, the others become
    softmax entries with their mean values; at the token level every
    candidate token is an entry. One softmax over all entries per head.

    fixed_sel {level: node ids}: the kept set of those levels is taken as given
    instead of chosen by score (forced-selection replay: where two sides split a
    near tie differently, the levels below are compared with one side's choice
    imposed on the other). A given set must hold min(k_l, C_l) distinct
    candidates of that level.
    """
    G, d = q.shape
    scale32 = default_scale(d) if scale is None else _F32(scale)
    nl = level_counts(n, f)
    T = len(nl)
    if len(k_levels) < T:
        raise ValueError(f"need k for {T} levels, got {len(k_levels)}")
    res = UnitResult(out=np.zeros((G, d)), lse=np.full(G, -np.inf))
    zs, vals = [], []
    prev: list[int] = []
    for lv in range(T, 0, -1):
        n_l = nl[lv - 1]
        n_up = nl[lv] if lv < T else 0
        kids = [f * p + j for p in prev for j in range(f)]
        cand = np.array(kids + list(range(f * n_up, n_l)), dtype=np.int64)
        C = len(cand)
        s = min(int(k_levels[lv - 1]), C)
        res.C[lv] = C
        res.q_pos[lv] = C
        if C == 0:
            res.sel[lv], res.flags[lv], prev = [], False, []
            continue
        NK, NV = tree[lv - 1]
        z = _logits(q, NK[cand], C, dtype, theta, scale32)             # [G, C]
        S = z.astype(_F64).sum(axis=0)
        res.scores[lv] = (cand, S)
        order = np.lexsort((np.arange(C), -S))                          # S desc, index asc
        res.flags[lv] = bool(0 < s < C and
                             0.0 < S[order[s - 1]] - S[order[s]] < NEAR_TIE_REL * np.abs(S).max())
        if fixed_sel is not None and lv in fixed_sel:
            pos = {int(c): i for i, c in enumerate(cand)}
            want = sorted(int(x) for x in fixed_sel[lv])
            if len(want) != s or len(set(want)) != s or any(x not in pos for x in want):
                raise ValueError(f"fixed selection at level {lv} is not {s} distinct candidates")
            keep = np.array([pos[x] for x in want], dtype=np.int64)
            order = np.concatenate([keep, np.setdiff1d(np.arange(C), keep)])
        chosen = np.sort(order[:s])
        res.sel[lv] = [int(cand[i]) for i in chosen]
        for i in np.sort(order[s:]):
            res.entries.append((lv, int(cand[i])))
            res.epos.append(int(i))
            zs.append(z[:, i])
            vals.append(NV[cand[i]])
        prev = res.sel[lv]
    base = f * nl[0] if T else 0
    kids = [f * p + j for p in prev for j in range(f)]
    cand0 = np.array(kids + list(range(base, n)), dtype=np.int64)
    C0 = len(cand0)
    res.C[0] = C0
    own = self_in and C0 > 0 and int(cand0[-1]) == n - 1
    pq = C0 - 1 if own else C0
    res.q_pos[0] = pq
    if C0:
        z0 = _logits(q, K[cand0], pq, dtype, theta, scale32)
        for i in range(C0):
            res.entries.append((0, int(cand0[i])))
            res.epos.append(i)
            zs.append(z0[:, i])
        vals.extend(V[cand0])
    if not zs:
        return res
    Z = np.array(zs, dtype=_F32)                                       # [E, G]
    Vm = np.array(vals, dtype=_F64)                                     # [E, d]
    res.z = Z
    Zd = Z.astype(_F64)
    m = Zd.max(axis=0)
    P = np.exp(Zd - m)
    l = P.sum(axis=0)
    res.out = (P.T @ Vm) / l[:, None]
    res.lse = m + np.log(l)
    res.weights = P / l
    return res


def dense_unit(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_keys: int, q_pos: int, dtype: str,
               theta: float = 1.0e6, scale=None):
    """Standard RoPE softmax attention: keys 0..n_keys-1 at their own positions, query at q_pos.

    The comparator the pages time RecSA against [Abstract]; same rotation,
    rounding and logit as the tree path, positions = original token positions.
    Returns (out [G, d] float64, lse [G] float64).
    """
    G, d = q.shape
    scale32 = default_scale(d) if scale is None else _F32(scale)
    if n_keys == 0:
        return np.zeros((G, d)), np.full(G, -np.inf)
    zs = []
    step = 1 << 16
    for lo in range(0, n_keys, step):
        hi = min(n_keys, lo + step)
        zs.append(_logits(q, K[lo:hi], q_pos, dtype, theta, scale32, row_pos=np.arange(lo, hi)))
    Z = np.concatenate(zs, axis=1).astype(_F64)                         # [G, n]
    m = Z.max(axis=1, keepdims=True)
    P = np.exp(Z - m)
    l = P.sum(axis=1)
    out = (P @ V[:n_keys].astype(_F64)) / l[:, None]
    return out, m[:, 0] + np.log(l)


# ----------------------------------------------------------------- whole-call wrappers

class TreeCache:
    """Per-(sequence, KV head) float32 views and trees, built on first use."""

    def __init__(self, K, V, W, f, dtype):
        self.K, self.V, self.f, self.dtype = K, V, f, dtype
        self.W = from_storage(W, dtype)
        self._slices: dict = {}

    def get(self, b: int, h: int, n: int):
        key = (b, h)
        ent = self._slices.get(key)
        if ent is None or ent[3] < n:
            Kf = from_storage(self.K[b, h], self.dtype)
            Vf = from_storage(self.V[b, h], self.dtype)
            tree = build_slice(Kf, Vf, self.W, self.f, self.dtype, n_new=n, cap=Kf.shape[0])
            ent = (Kf, Vf, tree, n)
            self._slices[key] = ent
        return ent[0], ent[1], ent[2]


def _all_units(B, n_q, groups):
    return [(b, j, h) for b in range(B) for j in range(n_q) for h in range(groups)]


def _groups(Hq: int, Hkv: int, select_heads):
    """(query heads per selection group, groups per sequence). By default the G = Hq / Hkv heads
    of a KV head select together [Abstract: per-query selection over the heads that share the
    KV cache]; a divisor Gs of G splits them into groups that select independently over the
    same tree and cache (Gs = 1: every head selects alone)."""
    G = Hq // Hkv
    Gs = G if not select_heads else int(select_heads)
    if G % Gs:
        raise ValueError("select_heads must divide the query heads of a KV head")
    return Gs, Hq // Gs


def decode(K, V, W, q, n_tokens: int, f: int, k_levels, dtype: str, theta: float = 1.0e6,
           scale=None, units=None, cache: TreeCache | None = None, select_heads=None) -> dict:
    """Decode: every query of q [B][n_q][Hq][d] at position n_tokens against the first
    n_tokens cached tokens of K, V [B][Hkv][cap][d] (storage form). Returns {(b, j, g): UnitResult}
    with g the selection group (the KV head by default; group g reads KV head g // (G / Gs)).
    """
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    Gs, groups = _groups(Hq, Hkv, select_heads)
    cache = cache or TreeCache(K, V, W, f, dtype)
    out = {}
    for (b, j, g) in (units if units is not None else _all_units(B, n_q, groups)):
        Kf, Vf, tree = cache.get(b, g // (G // Gs), n_tokens)
        qg = from_storage(q[b, j, g * Gs:(g + 1) * Gs], dtype)
        out[(b, j, g)] = attend_unit(qg, Kf, Vf, tree, n_tokens, f, k_levels, dtype, theta, scale)
    return out


def prefill(K, V, W, q, q_start: int, f: int, k_levels, dtype: str, theta: float = 1.0e6,
            scale=None, units=None, cache: TreeCache | None = None, select_heads=None) -> dict:
    """Causal prefill: query j of q [B][n_q][Hq][d] sits at position t = q_start + j and sees
    tokens 0..t including itself, i.e. a descent over the prefix n = t + 1 with only the
    nodes complete at n visible. Returns {(b, j, g): UnitResult} (groups as in decode).
    """
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    Gs, groups = _groups(Hq, Hkv, select_heads)
    cache = cache or TreeCache(K, V, W, f, dtype)
    out = {}
    for (b, j, g) in (units if units is not None else _all_units(B, n_q, groups)):
        t = q_start + j
        Kf, Vf, tree = cache.get(b, g // (G // Gs), q_start + n_q)
        qg = from_storage(q[b, j, g * Gs:(g + 1) * Gs], dtype)
        out[(b, j, g)] = attend_unit(qg, Kf, Vf, tree, t + 1, f, k_levels, dtype, theta, scale,
                                     self_in=True)
    return out


def generate(K, V, W, q_steps, k_steps, v_steps, n_start: int, f: int, k_levels, dtype: str,
             theta: float = 1.0e6, scale=None):
    """Autoregressive decoding over a growing cache.

    [Abstract]: the tree is kept over the KV cache and attention costs
    O(log L) per decoding step; [Core Idea]: nodes summarise complete spans of
    the cache. Reading: each generated token first joins the cache, the nodes
    its arrival completes are built (bottom level first, so a completed node
    can complete its parent), and the token's query then attends over the
    whole prefix, its own token included -- the causal semantics of prefill
    for one position.

    Step s handles position t = n_start + s: K[b, h, t] = k_steps[s, b, h] and
    V likewise, the nodes complete at t + 1 but not at t are built, and
    q_steps[s, b] (the G heads of each KV head) attends over tokens 0..t.

    K, V: [B][Hkv][cap][d] storage form, holding at least the first n_start
    tokens (not modified: each slice is copied); q_steps [S][B][Hq][d];
    k_steps, v_steps [S][B][Hkv][d]; W [d][d] storage form.
    Returns (results, slices): results[s][(b, h)] is the UnitResult of step s,
    slices[(b, h)] = (K, V, tree) as float32 after the last step.
    """
    B, Hkv, cap, d = K.shape
    S = q_steps.shape[0]
    G = q_steps.shape[2] // Hkv
    if n_start < 0 or n_start + S > cap:
        raise ValueError("positions n_start .. n_start + S - 1 must lie inside the cache")
    Wf = from_storage(W, dtype)
    results = [dict() for _ in range(S)]
    slices = {}
    for b in range(B):
        for h in range(Hkv):
            Kf = from_storage(K[b, h], dtype).copy()
            Vf = from_storage(V[b, h], dtype).copy()
            tree = build_slice(Kf, Vf, Wf, f, dtype, n_new=n_start, cap=cap)
            for s in range(S):
                t = n_start + s
                Kf[t] = from_storage(k_steps[s, b, h], dtype)
                Vf[t] = from_storage(v_steps[s, b, h], dtype)
                build_slice(Kf, Vf, Wf, f, dtype, n_new=t + 1, n_old=t, tree=tree, cap=cap)
                qg = from_storage(q_steps[s, b, h * G:(h + 1) * G], dtype)
                results[s][(b, h)] = attend_unit(qg, Kf, Vf, tree, t + 1, f, k_levels, dtype, theta, scale,
                                                 self_in=True)
            slices[(b, h)] = (Kf, Vf, tree)
    return results, slices
