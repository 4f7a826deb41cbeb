"""RecSA tree attention: gradients with the selections held fixed -- plain CPU oracle.

TEST INFRASTRUCTURE ONLY. Imported by tests/ (and the benchmark's CPU baseline); never by the
product path.

Source: "Recursive Sparse Attention: Million-Token Length Extrapolation at Logarithmic Cost",
abstract: RecSA is a trained mechanism (its pooler is distilled and the model is fine-tuned),
which needs gradients through the tree attention. The pages say nothing about how. Reading:

  * the selections of the forward pass are held fixed (which candidates a level keeps is a
    discrete choice with no gradient); what is differentiated is the softmax over the entries
    that the forward pass produced, each with the candidate index it was rotated at;
  * the forward pass's roundings to the storage type are passed straight through (each is
    differentiated as the identity), and every product is taken on the forward's own rounded
    operands: the rotated query of a level and the rotated key of an entry;
  * a node's key is W @ m with m the mean of its children's stored keys, and its value the
    mean of its children's stored values, so a node's gradients reach its children (and W)
    level by level down to the token rows.

For one unit with G query heads, entries e (logit z[h, e] = scale * <q~_h(level of e), k~_e>,
value v_e), softmax weights P[e, h], upstream gradients dout[h] and dlse[h]:
    dz[h, e]   = P[e, h] * (dout_h . v_e - dout_h . out_h) + dlse_h * P[e, h]
    dv_e       = sum_h P[e, h] * dout_h
    dk~_e      = scale * sum_h dz[h, e] * q~_h(level of e)
    dq~_h(l)   = scale * sum_{e at level l} dz[h, e] * k~_e
and each rotation is undone by its transpose: the key row of e receives rot^T(dk~_e, pos_e),
the query head receives sum_l rot^T(dq~_h(l), q_pos_l). A node's key gradient a then adds
outer(a, m) to dW and W^T a / f to each child's key gradient; its value gradient adds 1/f of
itself to each child's value gradient. Everything here is float64.
"""
from __future__ import annotations

import numpy as np

from .recsa import (attend_unit, build_slice, default_scale, from_storage, level_counts, rope_table,
                    rotate)

_F32 = np.float32
_F64 = np.float64


def unrotate(g: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Transpose of the rotate-half rotation by (c, s), applied to gradients g [..., d] (float64).

    The rotation maps (x1, x2) to (x1 c - x2 s, x2 c + x1 s); its transpose maps (g1, g2) to
    (g1 c + g2 s, g2 c - g1 s).
    """
    h = g.shape[-1] // 2
    c = np.asarray(c, _F64)
    s = np.asarray(s, _F64)
    g1, g2 = g[..., :h], g[..., h:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


def backward_unit(q: np.ndarray, K: np.ndarray, V: np.ndarray, tree, dtype: str, theta: float, scale,
                  res, dout: np.ndarray, dlse=None):
    """Gradients of one unit's outputs (forward result `res` of attend_unit on the same inputs).

    q: [G, d] float32; K, V: token rows float32; tree as built; dout: [G, d]; dlse: [G] or None.
    Returns (dq [G, d], rows) with rows a list of (level, id, dkey [d], dvalue [d]) per entry,
    level 0 = token rows, level l >= 1 = node rows of level l.
    """
    G, d = q.shape
    E = len(res.entries)
    if E == 0 or res.weights is None:
        return np.zeros((G, d)), []
    sc = float(default_scale(d) if scale is None else _F32(scale))
    P = res.weights                                                    # [E, G]
    lv_of = np.array([lv for lv, _ in res.entries])
    ids = np.array([g for _, g in res.entries])
    pos = np.array(res.epos)
    krows = np.stack([K[g] if lv == 0 else tree[lv - 1][0][g] for lv, g in res.entries]).astype(_F32)
    vrows = np.stack([V[g] if lv == 0 else tree[lv - 1][1][g] for lv, g in res.entries]).astype(_F64)
    dout = np.asarray(dout, _F64)

    dot_v = dout @ vrows.T                                             # [G, E]
    D = (P.T * dot_v).sum(axis=1)                                      # dout_h . out_h
    dz = P.T * (dot_v - D[:, None])                                    # [G, E]
    if dlse is not None:
        dz = dz + np.asarray(dlse, _F64)[:, None] * P.T
    dv = P @ dout                                                      # [E, d]

    dq = np.zeros((G, d))
    dk = np.zeros((E, d))
    for lv in sorted(set(lv_of.tolist())):
        sel = np.nonzero(lv_of == lv)[0]
        qp = res.q_pos[lv]
        if theta == 0.0:
            kt = krows[sel].astype(_F64)
            qt = np.asarray(q, _F64)
        else:
            c, s = rope_table(max(int(pos[sel].max()), qp), d, theta)
            kt = rotate(krows[sel], c[pos[sel]], s[pos[sel]], dtype).astype(_F64)
            qt = rotate(q, c[qp][None, :], s[qp][None, :], dtype).astype(_F64)
        dkt = sc * dz[:, sel].T @ qt                                   # [n_e, d]
        dqt = sc * dz[:, sel] @ kt                                     # [G, d]
        if theta == 0.0:
            dk[sel] = dkt
            dq += dqt
        else:
            dk[sel] = unrotate(dkt, c[pos[sel]], s[pos[sel]])
            dq += unrotate(dqt, c[qp][None, :], s[qp][None, :])
    rows = [(int(lv_of[e]), int(ids[e]), dk[e], dv[e]) for e in range(E)]
    return dq, rows


def backward_tree(K: np.ndarray, W: np.ndarray, tree, f: int, n: int, dNK, dNV, dK: np.ndarray, dV: np.ndarray):
    """Pushes node gradients down one (sequence, KV head) slice, top level first; returns dW.

    dNK[l - 1], dNV[l - 1]: float64 gradients of the level-l node keys and values (updated as
    parents push into them); dK, dV: float64 token-row gradients (updated). K: float32 token rows;
    W: float32 pooler. A node's m is recomputed as the forward computes it: child sums in
    float32 in child order, one division by f.
    """
    d = W.shape[0]
    dW = np.zeros((d, d))
    Wd = np.asarray(W, _F64)
    nl = level_counts(n, f)
    for lv in range(len(nl), 0, -1):
        a = dNK[lv - 1][:nl[lv - 1]]
        b = dNV[lv - 1][:nl[lv - 1]]
        g = np.nonzero(np.any(a != 0.0, axis=1) | np.any(b != 0.0, axis=1))[0]
        if len(g) == 0:
            continue
        srcK = K if lv == 1 else tree[lv - 2][0]
        gK, gV = (dK, dV) if lv == 1 else (dNK[lv - 2], dNV[lv - 2])
        acc = np.zeros((len(g), d), _F32)
        for j in range(f):
            acc = acc + srcK[f * g + j].astype(_F32)
        m = (acc / _F32(f)).astype(_F64)
        dW += a[g].T @ m
        dm = a[g] @ Wd                                                 # rows of W^T a
        for j in range(f):
            gK[f * g + j] += dm / f
            gV[f * g + j] += b[g] / f
    return dW


def backward(K, V, W, q, dout, f: int, k_levels, dtype: str, theta: float = 1.0e6, scale=None,
             n_tokens=None, q_start=None, dlse=None) -> dict:
    """Gradients of a whole call with the forward's selections held fixed.

    Decode (n_tokens given): every query of q [B][n_q][Hq][d] at position n_tokens against the
    first n_tokens tokens. Causal prefill (q_start given): query j at t = q_start + j over tokens
    0..t, its own token included. dout [B][n_q][Hq][d], dlse [B][n_q][Hq] or None.
    K, V [B][Hkv][cap][d], W [d][d] in storage form.
    Returns float64 dq [B][n_q][Hq][d], dK, dV [B][Hkv][cap][d], dW [d][d], and the forward
    results {(b, j, h): UnitResult}.
    """
    if (n_tokens is None) == (q_start is None):
        raise ValueError("give exactly one of n_tokens (decode) and q_start (causal prefill)")
    B, n_q, Hq, d = q.shape
    Hkv, cap = K.shape[1], K.shape[2]
    G = Hq // Hkv
    Wf = from_storage(W, dtype)
    n_max = n_tokens if n_tokens is not None else q_start + n_q
    dq = np.zeros((B, n_q, Hq, d))
    dK = np.zeros((B, Hkv, cap, d))
    dV = np.zeros((B, Hkv, cap, d))
    dW = np.zeros((d, d))
    results = {}
    for b in range(B):
        for h in range(Hkv):
            Kf = from_storage(K[b, h], dtype)
            Vf = from_storage(V[b, h], dtype)
            tree = build_slice(Kf, Vf, Wf, f, dtype, n_new=n_max, cap=cap)
            dNK = [np.zeros(t[0].shape) for t in tree]
            dNV = [np.zeros(t[1].shape) for t in tree]
            for j in range(n_q):
                n = n_tokens if n_tokens is not None else q_start + j + 1
                qg = from_storage(q[b, j, h * G:(h + 1) * G], dtype)
                r = attend_unit(qg, Kf, Vf, tree, n, f, k_levels, dtype, theta, scale,
                                self_in=n_tokens is None)
                results[(b, j, h)] = r
                dl = None if dlse is None else dlse[b, j, h * G:(h + 1) * G]
                dqu, rows = backward_unit(qg, Kf, Vf, tree, dtype, theta, scale, r, dout[b, j, h * G:(h + 1) * G], dl)
                dq[b, j, h * G:(h + 1) * G] = dqu
                for lv, g, dk, dv in rows:
                    if lv == 0:
                        dK[b, h, g] += dk
                        dV[b, h, g] += dv
                    else:
                        dNK[lv - 1][g] += dk
                        dNV[lv - 1][g] += dv
            dW += backward_tree(Kf, Wf, tree, f, n_max, dNK, dNV, dK[b, h], dV[b, h])
    return dict(dq=dq, dK=dK, dV=dV, dW=dW, results=results)
