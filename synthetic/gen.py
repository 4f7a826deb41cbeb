"""Seeded synthetic workloads for RecSA tree attention.

Every array is drawn from NumPy's PCG64 through a SeedSequence keyed by
(workload seed, tensor tag, sequence, head), so any slice can be regenerated
on its own and the CPU and GPU sides see bit-identical inputs. bf16 inputs
are produced by round-to-nearest-even on the float32 draw and handed out as
uint16 bit patterns; float32 inputs are handed out as float32.

Nothing here computes any part of the attention method: it only draws
numbers, places planted "needle" keys and lays arrays out.

Recipes (the shapes and value distributions follow the five workloads the
method is measured on: Qwen3-4B-like GQA heads, lengths 4K-2M, i.i.d. or
clustered keys, needle keys planted along a query direction):
  * i.i.d.: K, V, q ~ N(0, std^2) per element.
  * mixture: per (sequence, KV head) draw `centres` centre vectors
    mu ~ N(0, std^2 I); each contiguous run of `run` tokens picks one centre
    uniformly; key = mu + mix_sigma * N(0, std^2 I). Queries of a mixture
    workload pick one centre per (query, KV head) and add mix_sigma noise per
    query head. V stays i.i.d.
  * needles: `needles` keys per (sequence, KV head) at evenly spaced
    positions floor((j + 1/2) * L / m); needle j is needle_gain * rho * u,
    rho = std * sqrt(d) (the background key norm) and u the unit direction of
    one target query head of that KV group.
  * pooler: W = I + (w_gain / sqrt(d)) * N(0, 1), rounded to the storage type.
  * generated tokens (decoding past the end of a workload's cache): new keys
    and values ~ N(0, std^2) per element, drawn per (sequence, KV head).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

_TAG_W, _TAG_K, _TAG_V, _TAG_Q, _TAG_CENTRE, _TAG_RUN, _TAG_QNOISE, _TAG_QCENTRE, _TAG_NEWK, _TAG_NEWV = range(1, 11)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str              # 'f32' or 'bf16' storage for K, V, q, W and tree nodes
    L: int                  # tokens in the cache (decode) or positions prefilled (prefill)
    f: int                  # tree fanout
    k: int                  # candidates kept per level (same at every level)
    n_queries: int          # decode queries per sequence; prefill: every position
    mode: str               # 'decode' or 'prefill'
    chunk: int = 0          # prefill chunk length
    std: float = 1.0
    needles: int = 0        # planted needle keys per (sequence, KV head)
    needle_gain: float = 3.0
    centres: int = 0        # 0 = i.i.d. keys
    run: int = 0
    mix_sigma: float = 0.3
    w_gain: float = 0.05
    theta: float = 1.0e6    # RoPE base; 0 disables the rotation
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    # tiny CPU-checkable case
    "c0": Workload("c0", B=1, Hq=4, Hkv=1, d=64, dtype="f32", L=4096, f=16, k=4,
                   n_queries=8, mode="decode", std=1.0, needles=2, seed=100),
    # single-sequence decode, Qwen3-4B-like GQA
    "c1": Workload("c1", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", L=131072, f=16, k=8,
                   n_queries=256, mode="decode", std=128 ** -0.5, needles=16, seed=101),
    # four sequences at 512K tokens, clustered keys
    "c2": Workload("c2", B=4, Hq=32, Hkv=8, d=128, dtype="bf16", L=524288, f=16, k=8,
                   n_queries=256, mode="decode", std=128 ** -0.5, needles=32,
                   centres=64, run=4096, seed=102),
    # chunked causal prefill over 64K positions
    "c3": Workload("c3", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", L=65536, f=16, k=8,
                   n_queries=65536, mode="prefill", chunk=4096, std=128 ** -0.5, seed=103),
    # 2M-token decode, fanout 32
    "c4": Workload("c4", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", L=2097152, f=32, k=16,
                   n_queries=256, mode="decode", std=128 ** -0.5, needles=64,
                   centres=256, run=32768, seed=104),
}


def with_overrides(w: Workload, **kw) -> Workload:
    """Same recipe with some fields replaced (smaller L, fewer queries, other seed...)."""
    return dataclasses.replace(w, **kw)


# ---------------------------------------------------------------- storage helpers

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return bf16_bits(x) if dtype == "bf16" else x


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (float32 or bf16 bits) -> float32 values."""
    return bf16_value(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


def _rng(w: Workload, tag: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.seed, tag, b, h]))


# ---------------------------------------------------------------- tensors

def gen_W(w: Workload) -> np.ndarray:
    """Pooler matrix [d][d] (storage form), key = W @ mean."""
    g = _rng(w, _TAG_W).standard_normal((w.d, w.d), dtype=np.float32)
    W = np.eye(w.d, dtype=np.float32) + np.float32(w.w_gain / np.sqrt(w.d)) * g
    return _store(W, w.dtype)


def _centres(w: Workload, b: int, h: int) -> np.ndarray:
    return _rng(w, _TAG_CENTRE, b, h).standard_normal((w.centres, w.d), dtype=np.float32) * np.float32(w.std)


def gen_queries(w: Workload, b: int, n_q: int | None = None) -> np.ndarray:
    """Queries of sequence b, [n_q][Hq][d] storage form."""
    n_q = w.n_queries if n_q is None else n_q
    if w.centres == 0:
        q = _rng(w, _TAG_Q, b).standard_normal((n_q, w.Hq, w.d), dtype=np.float32) * np.float32(w.std)
        return _store(q, w.dtype)
    q = np.empty((n_q, w.Hq, w.d), dtype=np.float32)
    for h in range(w.Hkv):
        mu = _centres(w, b, h)
        pick = _rng(w, _TAG_QCENTRE, b, h).integers(0, w.centres, n_q)
        noise = _rng(w, _TAG_QNOISE, b, h).standard_normal((n_q, w.G, w.d), dtype=np.float32)
        q[:, h * w.G:(h + 1) * w.G, :] = mu[pick][:, None, :] + np.float32(w.mix_sigma * w.std) * noise
    return _store(q, w.dtype)


def needle_plan(w: Workload, n_q: int | None = None):
    """[(position, target query index, target query head offset within the group)] per KV head."""
    n_q = w.n_queries if n_q is None else n_q
    m = w.needles
    plan = []
    for j in range(m):
        pos = int((2 * j + 1) * w.L // (2 * m))
        tq = (j * max(n_q // max(m, 1), 1)) % n_q
        plan.append((pos, tq, j % w.G))
    return plan


def gen_kv_slice(w: Workload, b: int, h: int, q: np.ndarray | None = None):
    """(K, V) of sequence b, KV head h: each [L][d] storage form, pre-RoPE.

    `q` (storage form, [n_q][Hq][d]) is needed only when needles are planted;
    it is regenerated when omitted.
    """
    L, d = w.L, w.d
    if w.centres == 0:
        K = _rng(w, _TAG_K, b, h).standard_normal((L, d), dtype=np.float32)
        K *= np.float32(w.std)
    else:
        mu = _centres(w, b, h)
        n_runs = -(-L // w.run)
        assign = _rng(w, _TAG_RUN, b, h).integers(0, w.centres, n_runs)
        K = _rng(w, _TAG_K, b, h).standard_normal((L, d), dtype=np.float32)
        K *= np.float32(w.mix_sigma * w.std)
        K += np.repeat(mu[assign], w.run, axis=0)[:L]
    if w.needles:
        if q is None:
            q = gen_queries(w, b)
        qf = storage_to_f32(q, w.dtype)
        rho = w.std * np.sqrt(d)
        for pos, tq, hg in needle_plan(w, qf.shape[0]):
            u = qf[tq, h * w.G + hg].astype(np.float64)
            u /= max(np.linalg.norm(u), 1e-30)
            K[pos] = (w.needle_gain * rho * u).astype(np.float32)
    V = _rng(w, _TAG_V, b, h).standard_normal((L, d), dtype=np.float32)
    V *= np.float32(w.std)
    return _store(K, w.dtype), _store(V, w.dtype)


def gen_decode_inputs(w: Workload, n_q: int | None = None, heads=None, seqs=None):
    """Whole-workload host arrays: K, V [B][Hkv][L][d], q [B][n_q][Hq][d], W [d][d] (storage form).

    `heads`/`seqs` restrict which (sequence, KV head) slices are filled (others stay zero);
    meant for small workloads and for tests that look at a few slices only.
    """
    n_q = w.n_queries if n_q is None else n_q
    st = np.uint16 if w.dtype == "bf16" else np.float32
    K = np.zeros((w.B, w.Hkv, w.L, w.d), dtype=st)
    V = np.zeros_like(K)
    q = np.zeros((w.B, n_q, w.Hq, w.d), dtype=st)
    for b in range(w.B) if seqs is None else seqs:
        q[b] = gen_queries(w, b, n_q)
        for h in range(w.Hkv) if heads is None else heads:
            K[b, h], V[b, h] = gen_kv_slice(w, b, h, q[b])
    return {"K": K, "V": V, "q": q, "W": gen_W(w)}


def gen_new_tokens(w: Workload, n_new: int):
    """Keys and values of n_new tokens generated after the workload's L cached ones:
    (k_new, v_new), each [n_new][B][Hkv][d] storage form, i.i.d. N(0, std^2)."""
    k = np.empty((n_new, w.B, w.Hkv, w.d), dtype=np.float32)
    v = np.empty_like(k)
    for b in range(w.B):
        for h in range(w.Hkv):
            k[:, b, h] = _rng(w, _TAG_NEWK, b, h).standard_normal((n_new, w.d), dtype=np.float32) * np.float32(w.std)
            v[:, b, h] = _rng(w, _TAG_NEWV, b, h).standard_normal((n_new, w.d), dtype=np.float32) * np.float32(w.std)
    return _store(k, w.dtype), _store(v, w.dtype)
