"""RecSA pooler distillation: one gradient step on the pooler -- plain CPU oracle.

TEST INFRASTRUCTURE ONLY. Imported by tests/; never by the product path.

Sources: "Recursive Sparse Attention: Million-Token Length Extrapolation at Logarithmic Cost",
abstract, and "Recursive Sparse Attention RecSA: Million-Token Context Extrapolation at
Logarithmic Cost", section "Core Idea: Compressing the KV Cache with a Tree Structure": the
pooler that forms each node's key is learned by distilling from full attention. The pages give
neither the loss nor the optimiser. Reading:

  * loss: the mean over every (sequence, query, query head, dimension) of the squared
    difference between RecSA's output and a target (full attention's output on the same
    queries), with RecSA's selections held fixed while differentiating;
  * gradient: only the pooler W is learned; dL/dout = 2 (out - target) / N enters the gradient
    of the tree attention with respect to W (oracle.backward);
  * optimiser: plain gradient descent on a float64 master copy of W, W_master -= lr * dW; the
    pooler used by the next step is the master copy rounded to the storage type.
"""
from __future__ import annotations

import numpy as np

from .backward import backward
from .recsa import decode, dense_unit, from_storage, round_store, to_storage

_F32 = np.float32
_F64 = np.float64


def dense_targets(K, V, q, dtype: str, theta: float = 1.0e6, n_tokens: int | None = None) -> np.ndarray:
    """Full (dense) attention outputs of decode queries q [B][n_q][Hq][d] at position n_tokens over
    the first n_tokens cached tokens, float32 [B][n_q][Hq][d]: the distillation target."""
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, n_q, Hq, d), _F32)
    for b in range(B):
        for h in range(Hkv):
            Kf, Vf = from_storage(K[b, h], dtype), from_storage(V[b, h], dtype)
            for j in range(n_q):
                qg = from_storage(q[b, j, h * G:(h + 1) * G], dtype)
                o, _ = dense_unit(qg, Kf, Vf, n_tokens, n_tokens, dtype, theta)
                out[b, j, h * G:(h + 1) * G] = o.astype(_F32)
    return out


def distill_step(K, V, W, q, target, f: int, k_levels, dtype: str, lr: float, n_tokens: int,
                 theta: float = 1.0e6, W_master=None) -> dict:
    """One step. K, V [B][Hkv][cap][d], q [B][n_q][Hq][d], W [d][d] in storage form; target
    float32 [B][n_q][Hq][d]; W_master float64 [d][d] (default: W's values).
    Returns dict(loss (at W, before the update), dW, W_master (updated), W (storage form of the
    rounded master), out (RecSA outputs at W))."""
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    Wm = from_storage(W, dtype).astype(_F64) if W_master is None else np.asarray(W_master, _F64)
    res = decode(K, V, W, q, n_tokens, f, k_levels, dtype, theta)
    out = np.zeros((B, n_q, Hq, d))
    for (b, j, h), r in res.items():
        out[b, j, h * G:(h + 1) * G] = r.out
    diff = out - np.asarray(target, _F64)
    N = diff.size
    loss = float(np.sum(diff * diff) / N)
    dout = 2.0 * diff / N
    g = backward(K, V, W, q, dout, f, k_levels, dtype, theta, n_tokens=n_tokens)
    Wm_new = Wm - lr * g["dW"]
    W_new = to_storage(round_store(Wm_new.astype(_F32), dtype), dtype)
    return dict(loss=loss, dW=g["dW"], W_master=Wm_new, W=W_new, out=out, results=res)
