"""Oracle work for the full-size GPU tests, spread over worker processes.

Workers are started with the 'spawn' method, so they never inherit the test
process's GPU state (a worker that cannot start breaks the pool with an error
instead of being restarted); they import only numpy, the synthetic input generators and
the oracle. A job names a workload and one (sequence, KV head) slice; the worker
regenerates that slice from its seeds, builds the oracle's tree over it, and
runs the requested (query, KV head) units. It returns the slice in storage form
(for upload), a digest of every tree level (to compare with the library's tree
bit for bit without shipping it), and per-unit results.
"""
from __future__ import annotations

import hashlib
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor, as_completed

import numpy as np

_POOL = None


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool():
    """The shared worker pool (created once per test session)."""
    global _POOL
    if _POOL is None:
        _POOL = ProcessPoolExecutor(workers(), mp_context=mp.get_context("spawn"))
    return _POOL


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True, cancel_futures=True)
        _POOL = None


def level_digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _slim(r):
    """The parts of a UnitResult the comparisons use (picklable, small)."""
    return {"sel": r.sel, "flags": r.flags, "out": r.out, "lse": r.lse, "has_entries": r.z is not None,
            "n_entries": len(r.entries), "zmax": float(np.abs(r.z).max()) if r.z is not None else 0.0,
            "scores": {lv: (np.asarray(c), np.asarray(s)) for lv, (c, s) in r.scores.items()}}


class Slim:
    """Attribute view of a slimmed unit result (RecSA: as compare_unit expects; two-stage: blocks,
    tokens, flags, out, lse and z, as the two-stage comparison expects)."""

    def __init__(self, d):
        self.flags, self.out, self.lse = d["flags"], d["out"], d["lse"]
        self.z = True if d["has_entries"] else None
        if "blocks" in d:
            self.blocks, self.tokens = d["blocks"], d["tokens"]
        else:
            self.sel, self.n_entries, self.zmax, self.scores = d["sel"], d["n_entries"], d["zmax"], d["scores"]


def _slice_job(job):
    from threadpoolctl import threadpool_limits

    import oracle
    from synthetic import WORKLOADS, gen_kv_slice, gen_queries, gen_W, with_overrides
    w = with_overrides(WORKLOADS[job["workload"]], **job.get("overrides", {}))
    b, h = job["slice"]
    with threadpool_limits(limits=1):
        q = gen_queries(w, b, job["n_q"])
        K, V = gen_kv_slice(w, b, h, q)
        out = {"slice": (b, h)}
        if job.get("return_kv"):
            out["K"], out["V"] = K, V
        if not job.get("units") and not job.get("digest") and not job.get("ts_units"):
            return out
        Kf, Vf = oracle.from_storage(K, w.dtype), oracle.from_storage(V, w.dtype)
        Wf = oracle.from_storage(gen_W(w), w.dtype)
        tree = oracle.build_slice(Kf, Vf, Wf, w.f, w.dtype, n_new=w.L)
        if job.get("digest"):
            out["digest"] = [(level_digest(oracle.to_storage(NK, w.dtype)), level_digest(oracle.to_storage(NV, w.dtype)))
                             for NK, NV in tree]
        G = w.G
        k = job.get("k")
        res = {}
        for (j, n, self_in, fixed) in job.get("units", []):
            qg = oracle.from_storage(q[j, h * G:(h + 1) * G], w.dtype)
            r = oracle.attend_unit(qg, Kf, Vf, tree, n, w.f, k, w.dtype, w.theta, self_in=self_in,
                                   fixed_sel=fixed)
            res[(j, n, self_in, tuple(sorted((lv, tuple(v)) for lv, v in (fixed or {}).items())))] = _slim(r)
        out["units"] = res
        if job.get("ts_units"):
            from oracle.two_stage import two_stage_unit
            ts = {}
            for (j, kb, kt) in job["ts_units"]:
                qg = oracle.from_storage(q[j, h * G:(h + 1) * G], w.dtype)
                r = two_stage_unit(qg, Kf, Vf, tree[0][0], w.L, w.f, kb, kt, w.dtype, w.theta)
                ts[(j, kb, kt)] = {"blocks": r.blocks, "tokens": r.tokens, "flags": r.flags, "out": r.out,
                                   "lse": r.lse, "has_entries": r.z is not None}
            out["ts_units"] = ts
        return out


def run_slices(jobs, on_result=None):
    """Runs slice jobs on the pool; calls on_result(result) as each arrives (any order) and
    returns {slice: result} without the K/V arrays."""
    done = {}
    futs = [pool().submit(_slice_job, j) for j in jobs]
    for fu in as_completed(futs):
        r = fu.result()
        if on_result is not None:
            on_result(r)
        r.pop("K", None)
        r.pop("V", None)
        done[r["slice"]] = r
    return done


def unit_key(j, n, self_in, fixed=None):
    return (j, n, self_in, tuple(sorted((lv, tuple(v)) for lv, v in (fixed or {}).items())))
