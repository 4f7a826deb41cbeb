"""Benchmark: RecSA tree attention on one MI355X.

Workload (default): four independent sequences of 524,288 cached tokens, 32 query heads over
8 KV heads, head_dim 128, bf16, fanout 16, k = 8 per level, keys from a 64-centre Gaussian
mixture with planted needles; 256 decode queries per sequence.

One step = the whole hot path on that batch: build the tree over all 4 x 524,288 tokens
(node keys and mean values for every level), then decode all 4 x 256 queries (descent,
level-index RoPE, per-level top-k, one softmax) in one call. Inputs are resident in HBM
before timing starts. `value` is decode queries per second of whole-step time.

Prints one JSON line. --gpus above 1 is refused: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
METRIC = "decode queries/s & prefill tok/s per layer at 524K; % of HBM/MFMA roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-units", type=int, default=24, help="oracle decode units timed for the baseline")
    ap.add_argument("--calib-copy", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-step-mode", action="store_true", help="skip timing one-query-per-sequence decode calls")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip measuring the achievable HBM read/copy bandwidth with the probe program")
    ap.add_argument("--no-library-legs", action="store_true",
                    help="skip the library flash-attention comparison (torch scaled_dot_product_attention)")
    ap.add_argument("--no-legs", action="store_true", help="skip the dense and prefill comparison legs")
    ap.add_argument("--no-dense", action="store_true",
                    help="in the comparison legs, skip the dense comparator (RecSA prefill legs only)")
    ap.add_argument("--no-prefill64k", action="store_true", help="skip the 64K chunked-prefill workload")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the gradients")
    ap.add_argument("--no-two-stage", action="store_true", help="skip the two-stage block-then-token variant")
    ap.add_argument("--ts-blocks", type=int, default=128, help="two-stage variant: blocks kept")
    ap.add_argument("--ts-tokens", type=int, default=512, help="two-stage variant: tokens kept")
    ap.add_argument("--prefill-chunk", type=int, default=4096)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step benchmark, sweep the context length (decode 4K-2M, chunked "
                         "prefill 4K-64K) at the 131K workload's shape and print one JSON line of it")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def hbm_probe():
    """Achievable HBM read and copy bandwidth on this GPU from the probe program built with the
    library (streaming kernels over 8 GiB), or the reason it could not run."""
    import subprocess
    exe = os.path.join(ROOT, "long_context_hierarchical_amd", "probe", "hbm_probe")
    if not os.path.exists(exe):
        return {"error": "probe program not built"}
    try:
        r = subprocess.run([exe, "8"], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        return {"error": "probe timed out"}
    if r.returncode != 0:
        return {"error": (r.stderr or r.stdout).strip()[-200:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def kernel_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_hierarchical_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, src_hash: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters for this exact kernel source on this
    workload (the record names it, e.g. 'recsa-c2: ...'), if recorded."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != src_hash or not str(rec.get("workload", "")).startswith(f"recsa-{workload}:"):
        return None
    return rec.get("hbm_bytes_per_launch")


def decode_bytes_per_query(w, k):
    """Rows one query must read (all KV heads): node keys of every scored level, node values of
    every unkept candidate, and the key and value of every token-level candidate."""
    from long_context_hierarchical_amd.recsa import recsa_num_levels  # noqa: F401  (library sizing check)
    T = 0
    m = w.L // w.f
    nl = []
    while m >= 1:
        nl.append(m)
        m //= w.f
        T += 1
    s_up, n_up, key_rows, val_rows = 0, 0, 0, 0
    for lv in range(T, 0, -1):
        C = w.f * s_up + (nl[lv - 1] - w.f * n_up)
        s = min(k[lv - 1], C)
        if s < C:
            key_rows += C
            val_rows += C - s
        s_up, n_up = s, nl[lv - 1]
    C0 = w.f * s_up + (w.L - w.f * n_up) if T else w.L
    rows = key_rows + val_rows + 2 * C0
    return rows * w.d * w.elem_bytes * w.Hkv, dict(key_rows=key_rows, val_rows=val_rows, tok_rows=C0)


def decode_unique_bytes(w, k, sel):
    """Bytes of the distinct rows one decode call reads (the union over its queries, per
    sequence and KV head), from the kernel's selections sel [B][n_q][H_kv][T][width] (kept ids
    ascending, -1 padded): the key of every candidate of a level that is scored, the value of
    every candidate that some query did not keep, and the key and value of every token-level
    candidate. A level whose candidates are all kept reads nothing."""
    import numpy as np
    sel = np.asarray(sel)
    B, nq, H, T = sel.shape[:4]
    f, L = w.f, w.L
    nl, m = [], L // f
    while m >= 1:
        nl.append(m)
        m //= f
    if len(nl) != T:
        raise ValueError(f"sel holds {T} levels, the context has {len(nl)}")
    slab = np.arange(B * H, dtype=np.int64).reshape(B, H, 1)

    def per_slice(ids, n):
        # ids [B][n_q][H][c] -> flat indices into a [B * H * n] count array
        flat = ids.transpose(0, 2, 1, 3).reshape(B, H, -1).astype(np.int64)
        return (slab * n + flat).ravel()

    rows, s_up, n_up, parents = 0, 0, 0, None
    for lv in range(T, 0, -1):
        n_l = nl[lv - 1]
        C = f * s_up + (n_l - f * n_up)
        s = min(int(k[lv - 1]), C)
        kept = sel[:, :, :, lv - 1, :s]
        if s < C:
            cand = np.zeros(B * H * n_l, np.int64)
            if s_up:
                kids = parents[..., None].astype(np.int64) * f + np.arange(f)
                cand += np.bincount(per_slice(kids.reshape(B, nq, H, -1), n_l), minlength=B * H * n_l)
            cand = cand.reshape(B, H, n_l)
            cand[:, :, f * n_up:] += nq
            ksel = np.bincount(per_slice(kept, n_l), minlength=B * H * n_l).reshape(B, H, n_l)
            rows += int((cand > 0).sum()) + int((cand > ksel).sum())
        parents, s_up, n_up = kept, s, n_l
    tok = np.zeros(B * H * L, bool)
    if s_up:
        kids = parents[..., None].astype(np.int64) * f + np.arange(f)
        tok[per_slice(kids.reshape(B, nq, H, -1), L)] = True
    tok = tok.reshape(B, H, L)
    tok[:, :, f * n_up:] = True
    rows += 2 * int(tok.sum())
    return rows * w.d * w.elem_bytes


def build_bytes(w):
    """Read every token row of K and V once, write every node key and value once (all levels)."""
    nodes, m = 0, w.L // w.f
    while m >= 1:
        nodes += m
        m //= w.f
    return w.B * w.Hkv * w.d * w.elem_bytes * (2 * w.L + 2 * nodes), nodes


def pool_launches(w):
    """Pool-kernel launches of one full build: the library builds two levels per launch when
    the fanout divides the nodes of one tile (32 at d = 128, 64 at d = 64), else one level."""
    T, m = 0, w.L // w.f
    while m >= 1:
        T += 1
        m //= w.f
    fused = {128: 32, 64: 64}[w.d] % w.f == 0
    return (T + 1) // 2 if fused else T


def sweep():
    """Context-length sweep at the 131K workload's shape (one sequence, 32 query heads, 8 KV
    heads, d = 128, bf16, f = 16, k = 8): for L = 4K..2M (powers of 2) the full tree build, a
    256-query batched decode, a 1-query decode step and the dense 1-query decode step; for
    L = 4K..64K the causal prefill of all L positions in chunks of 4096 (the tree extended
    chunk by chunk) against dense causal prefill. Seeded random inputs, timing only."""
    import torch

    from long_context_hierarchical_amd import recsa as R
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, f, kk, nq = 1, 32, 8, 128, 16, 8, 256
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def inputs(L, n_q):
        s = d ** -0.5
        K = (torch.randn(B, Hkv, L, d, device=dev, generator=gen) * s).to(torch.bfloat16)
        V = (torch.randn(B, Hkv, L, d, device=dev, generator=gen) * s).to(torch.bfloat16)
        q = (torch.randn(B, n_q, Hq, d, device=dev, generator=gen) * s).to(torch.bfloat16)
        W = (torch.eye(d, device=dev) + 0.05 * s * torch.randn(d, d, device=dev, generator=gen)).to(torch.bfloat16)
        return K, V, q, W

    decode_rows = []
    for lg in range(12, 22):
        L = 1 << lg
        log(f"sweep decode L={L}")
        sh = R.Shape(B, Hkv, Hq, d, f, "bf16", L, 0.0, 1.0e6)
        K, V, q, W = inputs(L, nq)
        tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device=dev)
        T = R.recsa_num_levels(L, f)
        k = [kk] * T
        ws = torch.zeros(max(R.recsa_workspace_bytes(sh, L, k), 16), dtype=torch.uint8, device=dev)
        out = torch.empty(B, nq, Hq, d, dtype=torch.float32, device=dev)
        t_build = timed(lambda: R.recsa_build_tree(sh, K, V, W, 0, L, tree), 5)
        t_dec = timed(lambda: R.recsa_decode(sh, q, K, V, tree, L, k, out, None, None, 0, ws), 10)
        q1 = q[:, :1].contiguous()
        o1 = torch.empty(B, 1, Hq, d, dtype=torch.float32, device=dev)
        t_step = timed(lambda: R.recsa_decode(sh, q1, K, V, tree, L, k, o1, None, None, 0, ws), 20)
        Kr = torch.empty_like(K)
        R.recsa_rotate_keys(sh, K, L, Kr)
        mode = R.RECSA_DENSE_KEYS_ROTATED
        dws = torch.empty(max(R.recsa_dense_workspace_bytes(sh, L, 1, mode), 16), dtype=torch.uint8, device=dev)
        t_dense = timed(lambda: R.recsa_dense_ref_attn(sh, q1, 0, Kr, V, L, mode, o1, None, dws), 10)
        nodes, m = 0, L // f
        while m >= 1:
            nodes += m
            m //= f
        build_bytes = B * Hkv * d * 2 * (2 * L + 2 * nodes)
        decode_rows.append({"L": L, "levels": T, "build_ms": round(t_build, 4),
                            "build_GBps": round(build_bytes / (t_build * 1e-3) / 1e9, 1),
                            "decode_batched_ms": round(t_dec, 4),
                            "decode_queries_per_s": round(B * nq / (t_dec * 1e-3), 1),
                            "decode_step_ms": round(t_step, 4), "dense_step_ms": round(t_dense, 4),
                            "step_speedup_vs_dense": round(t_dense / t_step, 2)})
        del K, V, q, tree, Kr, dws, ws
        torch.cuda.empty_cache()

    prefill_rows = []
    chunk = 4096
    for lg in range(12, 17):
        L = 1 << lg
        log(f"sweep prefill L={L}")
        sh = R.Shape(B, Hkv, Hq, d, f, "bf16", L, 0.0, 1.0e6)
        K, V, q, W = inputs(L, L)
        tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device=dev)
        k = [kk] * max(R.recsa_num_levels(L, f), 1)
        ws = torch.zeros(max(R.recsa_workspace_bytes(sh, L, k), 16), dtype=torch.uint8, device=dev)
        out = torch.empty(B, L, Hq, d, dtype=torch.float32, device=dev)

        def recsa_prefill_all():
            for c0 in range(0, L, chunk):
                R.recsa_build_tree(sh, K, V, W, c0, c0 + chunk, tree)
                R.recsa_prefill(sh, q[:, c0:c0 + chunk], c0, K, V, tree, k, out[:, c0:c0 + chunk], None, None, 0,
                                ws)
        t_r = timed(recsa_prefill_all, 2)
        mode = R.RECSA_DENSE_CAUSAL
        dws = torch.empty(max(R.recsa_dense_workspace_bytes(sh, L, L, mode), 16), dtype=torch.uint8, device=dev)
        t_d = timed(lambda: R.recsa_dense_ref_attn(sh, q, 0, K, V, L, mode, out, None, dws), 1)
        prefill_rows.append({"L": L, "recsa_ms": round(t_r, 3), "recsa_tokens_per_s": round(L / (t_r * 1e-3), 1),
                             "dense_ms": round(t_d, 3), "dense_tokens_per_s": round(L / (t_d * 1e-3), 1),
                             "speedup": round(t_d / t_r, 2)})
        del K, V, q, tree, out, dws, ws
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "context length, 131K workload shape (B=1, Hq=32, Hkv=8, d=128, bf16, f=16, k=8)",
                      "data": "synthetic (seeded random, timing only)",
                      "decode": decode_rows, "prefill_chunked_4096": prefill_rows}), flush=True)


# Vector-ALU issue peak of the MI355X: 256 CUs x 4 SIMDs x 2.4 GHz, a wave64 instruction every 4
# clocks per SIMD: 39.3 T lane-instructions/s. A v_dot2_f32_bf16 lane-instruction is 2
# multiply-adds (the 157.3 TFLOP/s vector peak), a v_fma_f32 one (78.6 TFLOP/s).
VALU_LANE_OPS = 256 * 4 * 2.4e9 * 64 / 4


def shared_level(n, f, k):
    """(level, node count) of the first level a query over n tokens scores: every level above it
    keeps all its nodes, so its candidates are all its nodes (closed form); (0, 0) if none."""
    nl, m = [], n // f
    while m >= 1:
        nl.append(m)
        m //= f
    for lv in range(len(nl), 0, -1):
        if k[lv - 1] < nl[lv - 1]:
            return lv, nl[lv - 1]
    return 0, 0


def values_on_mfma(w):
    """bf16 storage with at least two query heads per KV head: the weighted value sums run on the
    matrix cores."""
    return w.dtype == "bf16" and w.Hq // w.Hkv >= 2


def valu_roofline(w, rows, n_queries, ms, mf_rows=0):
    """The attention kernel against the vector-ALU roofline (it is issue-bound; its row reads
    mostly hit the cache). Algorithmic work per query: one multiply-add per (query head, element)
    for every logit computed on the vector units (the scored rows, less the first scored level's
    mf_rows, whose logits come from the matrix cores) and, when the value sums run on the vector
    units (float32 storage, one query head per KV head), for every weighted value row; key
    rotation, selection and exponentials are not counted. Logits run on v_dot2_f32_bf16 (2
    multiply-adds per lane-instruction; v_fma_f32 for float32 storage), values on v_fma_f32 (1):
    the time at peak issue is logit_macs / (2 or 1) + value_macs lane-instructions over
    VALU_LANE_OPS, and `peak` is the flop rate that time implies for this mix."""
    logit_macs = w.d * w.Hq * (rows["key_rows"] + rows["tok_rows"] - mf_rows)
    value_macs = 0 if values_on_mfma(w) else w.d * w.Hq * (rows["val_rows"] + rows["tok_rows"])
    per_dot = 2 if w.dtype == "bf16" else 1
    t_peak = (logit_macs / per_dot + value_macs) / VALU_LANE_OPS * n_queries
    flops = 2 * (logit_macs + value_macs) * n_queries
    ach = flops / (ms * 1e-3) / 1e12
    peak = flops / t_peak / 1e12
    return {"bound": "alu", "achieved": round(ach, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
            "frac": round(t_peak / (ms * 1e-3), 4), "flops_per_query": 2 * (logit_macs + value_macs),
            "peak_derivation": "256 CU x 4 SIMD x 2.4 GHz / 4 clk x 64 lanes; dot2 = 2 MAC, fma = 1 MAC"}


def mfma_share(w, n_queries, ms, c_shared, rows):
    """Useful matrix-core flops: the first scored level's logits, 2 * d * H_q * C per query (rows
    past the workgroup's queries not counted), and, when they run there (values_on_mfma), the
    weighted value sums, 2 * d * H_q per weighted row (each weight's two bf16 terms counted once);
    as a rate over the whole call and as a fraction of the 2.5 PFLOP/s bf16 peak."""
    tile = 2.0 * w.d * w.Hq * c_shared * n_queries
    vals = 2.0 * w.d * w.Hq * (rows["val_rows"] + rows["tok_rows"]) * n_queries if values_on_mfma(w) else 0.0
    ach = (tile + vals) / (ms * 1e-3) / 1e12
    return {"flops_per_call": tile + vals, "tile_flops": tile, "value_flops": vals, "candidates": c_shared,
            "achieved_over_call": round(ach, 2), "unit": "TFLOP/s", "frac_of_peak_over_call": round(ach / 2500.0, 5)}


def needle_recall(w, sel, cpu):
    """Fraction of planted needles that end as exact token entries of their target query (the
    needle's level-1 block kept, or the needle in the trailing partial block): over every needle
    from the GPU call's selections sel [B][n_q][H_kv][T][width], and on the oracle's sample (the
    CPU baseline decodes each sampled slice's needle targets) from both sides."""
    from synthetic import needle_plan
    if not w.needles:
        return None
    f, n1 = w.f, w.L // w.f

    def gpu_hit(b, h, pos, tq):
        return pos >= f * n1 or pos // f in set(int(x) for x in sel[b, tq, h, 0] if x >= 0)
    tot = hit = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            for pos, tq, _hg in needle_plan(w, w.n_queries):
                tot += 1
                hit += gpu_hit(b, h, pos, tq)
    out = {"gpu_all": round(hit / tot, 4), "needles": tot}
    hits = (cpu or {}).get("_needle_hits") or []
    if hits:
        out["oracle_sample"] = round(sum(x[4] for x in hits) / len(hits), 4)
        out["gpu_same_sample"] = round(sum(gpu_hit(b, h, pos, tq) for (b, h, pos, tq, _o) in hits) / len(hits), 4)
        out["sample_needles"] = len(hits)
        out["sample_agree"] = all(gpu_hit(b, h, pos, tq) == o for (b, h, pos, tq, o) in hits)
    return out


def prefill_counts(L, f, k):
    """Closed-form (scored rows, softmax entries) summed over every causal position t < L: the
    query at t descends over the prefix n = t + 1, its own token included; a level is scored
    unless it keeps all its candidates."""
    scored = entries = 0
    for n in range(1, L + 1):
        nl, m = [], n // f
        while m >= 1:
            nl.append(m)
            m //= f
        s_up, n_up = 0, 0
        for lv in range(len(nl), 0, -1):
            C = f * s_up + (nl[lv - 1] - f * n_up)
            s = min(k[lv - 1], C)
            if s < C:
                scored += C
                entries += C - s
            s_up, n_up = s, nl[lv - 1]
        C0 = f * s_up + (n - f * n_up) if nl else n
        scored += C0
        entries += C0
    return scored, entries


def prefill_64k_leg(R, dev, timed, dense=True):
    """The 64K chunked-prefill workload: one sequence, 8 KV heads, bf16, f = 16, k = 8, queries at
    every position in chunks of 4096; per chunk the tree is extended over the chunk's complete
    blocks, then the chunk's queries attend. Timed over all 16 chunks (builds included), next to
    the dense comparator's causal prefill of the same 65,536 positions."""
    import numpy as np
    import torch
    from synthetic import WORKLOADS, gen_kv_slice, gen_queries, gen_W
    w = WORKLOADS["c3"]
    td = torch.bfloat16
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
    q_h = gen_queries(w, 0, w.L)
    K = torch.empty(1, w.Hkv, w.L, w.d, dtype=td, device=dev)
    V = torch.empty_like(K)
    for h in range(w.Hkv):
        Kb, Vb = gen_kv_slice(w, 0, h, q_h)
        K[0, h] = torch.from_numpy(Kb).view(td).to(dev)
        V[0, h] = torch.from_numpy(Vb).view(td).to(dev)
    q = torch.from_numpy(q_h[None]).view(td).to(dev)
    W = torch.from_numpy(gen_W(w)).view(td).to(dev)
    T = R.recsa_num_levels(w.L, w.f)
    k = [w.k] * T
    tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device=dev)
    ws = torch.zeros(R.recsa_workspace_bytes(sh, w.L, k), dtype=torch.uint8, device=dev)
    out = torch.empty(1, w.L, w.Hq, w.d, dtype=torch.float32, device=dev)

    def run():
        for c0 in range(0, w.L, w.chunk):
            R.recsa_build_tree(sh, K, V, W, c0, c0 + w.chunk, tree)
            R.recsa_prefill(sh, q[:, c0:c0 + w.chunk], c0, K, V, tree, k, out[:, c0:c0 + w.chunk], None, None, 0, ws)
    ms = timed(run, 5)
    scored, entries = prefill_counts(w.L, w.f, k)
    mf_rows = sum(shared_level(n, w.f, k)[1] for n in range(1, w.L + 1))
    rows = {"key_rows": scored, "tok_rows": 0, "val_rows": entries}
    leg = {"workload": f"recsa-c3: chunked causal prefill, L={w.L}, chunk={w.chunk}, Hq={w.Hq}, Hkv={w.Hkv}, "
                       f"d={w.d}, fanout={w.f}, k={w.k}",
           "ms": round(ms, 4), "tokens_per_s": round(w.L / (ms * 1e-3), 1),
           "scored_rows": scored, "entries": entries,
           "roofline_alu": valu_roofline(w, rows, 1, ms, mf_rows=mf_rows),
           "mfma": mfma_share(w, 1, ms, mf_rows, rows)}
    if dense:
        mode = R.RECSA_DENSE_CAUSAL
        dws = torch.empty(max(R.recsa_dense_workspace_bytes(sh, w.L, w.L, mode), 16), dtype=torch.uint8, device=dev)
        dms = timed(lambda: R.recsa_dense_ref_attn(sh, q, 0, K, V, w.L, mode, out, None, dws), 1)
        leg["dense_ms"] = round(dms, 3)
        leg["dense_tokens_per_s"] = round(w.L / (dms * 1e-3), 1)
        leg["speedup_vs_dense"] = round(dms / ms, 2)
        del dws
    del K, V, q, tree, ws, out
    torch.cuda.empty_cache()
    return leg


def tile_sharing(sel):
    """How many (query, KV head) units of one call share each candidate tile: at level l the
    children of the level-(l+1) node kept at rank r form one tile of keys rotated at the same
    positions, shared by every unit that kept that node at that rank. sel: [B][n_q][H_kv][T][w]."""
    import numpy as np
    B, nq, H, T, width = sel.shape
    out = {}
    for lv in range(T, 0, -1):                        # parents kept at level lv -> tiles at lv - 1
        s = sel[:, :, :, lv - 1, :]
        bb, _, hh, rr = np.nonzero(s >= 0)
        if bb.size == 0:
            continue
        node = s[s >= 0].astype(np.int64)
        key = ((bb.astype(np.int64) * H + hh) * (int(node.max()) + 1) + node) * width + rr
        tiles = np.unique(key).size
        out[f"level_{lv - 1}"] = {"unit_tiles": int(bb.size), "distinct_tiles": int(tiles),
                                  "units_per_tile": round(bb.size / tiles, 2)}
    return out


def library_legs(w, Kr, V, q, qp, c, timed):
    """The same dense attention through torch.nn.functional.scaled_dot_product_attention (the
    platform's flash-attention library), timing only: the KV heads are expanded to the query
    heads first and the queries are used as stored (no rotation), so outputs are not compared.
    Records the backend used, or the error if no fused backend accepts the shapes."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    G = w.Hq // w.Hkv
    out = {}
    try:
        Ke = Kr.repeat_interleave(G, dim=1)        # [B][Hq][L][d]
        Ve = V.repeat_interleave(G, dim=1)
    except RuntimeError as e:                      # out of memory
        return {"error": str(e)[:200]}
    qd = q.transpose(1, 2).contiguous()            # [B][Hq][n_q][d]
    qs = q[:, :1].transpose(1, 2).contiguous()
    qpre = qp.transpose(1, 2).contiguous()         # [B][Hq][c][d]
    for backend in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel(backend):
                ms_b = timed(lambda: F.scaled_dot_product_attention(qd, Ke, Ve), 3)
                ms_s = timed(lambda: F.scaled_dot_product_attention(qs, Ke, Ve), 10)
            out = {"backend": backend.name,
                   "decode_batched_ms": round(ms_b, 4),
                   "decode_batched_queries_per_s": round(w.B * w.n_queries / (ms_b * 1e-3), 1),
                   "decode_batched_TFLOPs": round(4.0 * w.B * w.n_queries * w.Hq * w.d * w.L / (ms_b * 1e-3) / 1e12, 1),
                   "decode_step_ms": round(ms_s, 4),
                   "decode_step_GBps": round(2 * w.B * w.Hkv * w.L * w.d * w.elem_bytes / (ms_s * 1e-3) / 1e9, 1)}
            break
        except RuntimeError as e:
            out = {"error": f"{backend.name}: {str(e)[:200]}"}
    if "backend" in out:
        try:
            from torch.nn.attention.bias import causal_lower_right
            mask = causal_lower_right(c, w.L)
            with sdpa_kernel(getattr(SDPBackend, out["backend"])):
                ms_p = timed(lambda: F.scaled_dot_product_attention(qpre, Ke, Ve, attn_mask=mask), 2)
            flops = 4.0 * w.B * w.Hq * w.d * sum(range(w.L - c + 1, w.L + 1))
            out["prefill_last_chunk_ms"] = round(ms_p, 4)
            out["prefill_last_chunk_TFLOPs"] = round(flops / (ms_p * 1e-3) / 1e12, 1)
        except (RuntimeError, ImportError, TypeError) as e:
            out["prefill_error"] = str(e)[:200]
    del Ke, Ve
    torch.cuda.empty_cache()
    return out


def _cpu_worker(job):
    """One worker of the CPU baseline (a separate process, one thread): generate one
    (sequence, KV head) slice, build its tree with the oracle, decode `n_units` units -- the
    slice's needle target queries first -- and note for each needle target whether its needle
    ended as an exact token entry (its level-1 block kept, or the token in the trailing block)."""
    name, slice_idx, n_units, k = job
    from threadpoolctl import threadpool_limits

    import oracle
    from synthetic import WORKLOADS, gen_kv_slice, gen_queries, gen_W, needle_plan
    w = WORKLOADS[name]
    b, h = divmod(slice_idx, w.Hkv)
    plan = needle_plan(w) if w.needles else []
    targets = {}
    for pos, tq, _hg in plan:
        targets.setdefault(tq, []).append(pos)
    order = list(targets) + [j for j in range(w.n_queries) if j not in targets]
    hits = []
    with threadpool_limits(limits=1):
        q = gen_queries(w, b)
        K, V = gen_kv_slice(w, b, h, q)
        Kf, Vf, Wf = (oracle.from_storage(x, w.dtype) for x in (K, V, gen_W(w)))
        t0 = time.perf_counter()
        tree = oracle.build_slice(Kf, Vf, Wf, w.f, w.dtype, n_new=w.L)
        t_build = time.perf_counter() - t0
        t0 = time.perf_counter()
        for j in order[:n_units]:
            qg = oracle.from_storage(q[j, h * w.G:(h + 1) * w.G], w.dtype)
            r = oracle.attend_unit(qg, Kf, Vf, tree, w.L, w.f, k, w.dtype, w.theta)
            for pos in targets.get(j, []):
                hits.append((b, h, pos, j, bool(pos >= w.f * (w.L // w.f) or pos // w.f in r.sel.get(1, []))))
        t_unit = (time.perf_counter() - t0) / n_units
    return t_build, t_unit, hits


def _cpu_prefill_worker(job):
    """One worker of the CPU prefill baseline: generate one KV head's slice of the 64K chunked
    prefill workload, build its tree with the oracle, and prefill `n_units` positions drawn
    uniformly (each a descent over its prefix, its own token included)."""
    name, h, n_units, k, seed = job
    from threadpoolctl import threadpool_limits

    import numpy as np

    import oracle
    from synthetic import WORKLOADS, gen_kv_slice, gen_queries, gen_W
    w = WORKLOADS[name]
    pos = np.random.default_rng(seed).integers(0, w.L, n_units)
    with threadpool_limits(limits=1):
        q = gen_queries(w, 0, w.L)
        K, V = gen_kv_slice(w, 0, h, q)
        Kf, Vf, Wf = (oracle.from_storage(x, w.dtype) for x in (K, V, gen_W(w)))
        t0 = time.perf_counter()
        tree = oracle.build_slice(Kf, Vf, Wf, w.f, w.dtype, n_new=w.L)
        t_build = time.perf_counter() - t0
        t0 = time.perf_counter()
        for p in pos:
            qg = oracle.from_storage(q[p, h * w.G:(h + 1) * w.G], w.dtype)
            oracle.attend_unit(qg, Kf, Vf, tree, int(p) + 1, w.f, k, w.dtype, w.theta, self_in=True)
        t_unit = (time.perf_counter() - t0) / n_units
    return t_build, t_unit


def cpu_baseline(w, k, n_units):
    """The oracle as it stands on the host's cores: P single-threaded worker processes (P = the
    CPUs this process may use, at most 16), each building one (sequence, KV head) slice of the
    tree and decoding `n_units` (query, KV head) units; the per-worker times under that load
    are extrapolated to one step spread over the P cores. Runs before this process touches
    the GPU (the workers are forked)."""
    import multiprocessing as mp
    import statistics
    from synthetic import WORKLOADS
    P = max(1, min(16, len(os.sched_getaffinity(0)), w.B * w.Hkv))
    jobs = [(w.name, i, n_units, list(k)) for i in range(P)]
    wp = WORKLOADS["c3"]
    Tp, m = 0, wp.L // wp.f
    while m >= 1:
        Tp, m = Tp + 1, m // wp.f
    Pp = max(1, min(P, wp.Hkv))
    pjobs = [("c3", h, n_units, [wp.k] * Tp, 500 + h) for h in range(Pp)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(P) as pool:
        res = pool.map(_cpu_worker, jobs)
        wall = time.perf_counter() - t0
        pres = pool.map(_cpu_prefill_worker, pjobs)
    t_build = statistics.median(r[0] for r in res)
    t_unit = statistics.median(r[1] for r in res)
    step_s = (w.B * w.Hkv * t_build + w.B * w.n_queries * w.Hkv * t_unit) / P
    pb = statistics.median(r[0] for r in pres)
    pu = statistics.median(r[1] for r in pres)
    prefill_s = (wp.Hkv * pb + wp.L * wp.Hkv * pu) / Pp
    return {
        "value": w.B * w.n_queries / step_s,
        "unit": "queries/s",
        "cores": P,
        "kind": "oracle",
        "sample": (f"{P} worker processes, one thread each: each built 1 of the {w.B * w.Hkv} (sequence, KV "
                   f"head) slices (median {t_build:.2f} s) and decoded {n_units} of the "
                   f"{w.B * w.n_queries * w.Hkv} units (median {t_unit * 1e3:.2f} ms each); one step "
                   f"extrapolated over {P} cores: {step_s:.2f} s (sample wall {wall:.1f} s incl. input generation)"),
        "build_GBps": build_bytes(w)[0] / (w.B * w.Hkv) / t_build * P / 1e9,
        "prefill_64k": {"tokens_per_s": wp.L / prefill_s, "cores": Pp,
                        "sample": (f"{Pp} worker processes, one thread each: each built one KV head's slice of the "
                                   f"64K chunked-prefill workload (median {pb:.2f} s) and prefilled {n_units} "
                                   f"positions drawn uniformly (median {pu * 1e3:.2f} ms each); all "
                                   f"{wp.L} positions x {wp.Hkv} KV heads extrapolated over {Pp} cores: "
                                   f"{prefill_s:.1f} s")},
        "host": host_cpu(),
        "_needle_hits": [hh for r in res for hh in r[2]],
    }


def host_cpu():
    """The host CPU's model name and its physical core count (from /proc/cpuinfo)."""
    model, cores = None, set()
    try:
        phys = core = None
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
    except OSError:
        pass
    return {"model": model, "physical_cores": len(cores) or None, "usable_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by (sequence, KV head) with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep()
        return

    # run first, as child processes, before this process touches the GPU
    probe = None if args.no_hbm_probe else hbm_probe()
    cpu = None
    if not args.no_cpu:
        from synthetic import WORKLOADS as _W
        _w = _W[args.workload]
        _T, _m = 0, _w.L // _w.f
        while _m >= 1:
            _T += 1
            _m //= _w.f
        log("timing the CPU oracle on a sample (host cores)")
        cpu = cpu_baseline(_w, [_w.k] * _T, args.cpu_units)

    import numpy as np
    import torch

    from long_context_hierarchical_amd import recsa as R
    from synthetic import WORKLOADS, gen_kv_slice, gen_queries, gen_W

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
    T = R.recsa_num_levels(w.L, w.f)
    k = [w.k] * T

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if w.dtype == "bf16" else t).to(dev, non_blocking=False)

    log(f"generating {w.name}: B={w.B} L={w.L} Hkv={w.Hkv} d={w.d} {w.dtype}")
    t0 = time.time()
    K = torch.empty(w.B, w.Hkv, w.L, w.d, dtype=td, device=dev)
    V = torch.empty_like(K)
    q = torch.empty(w.B, w.n_queries, w.Hq, w.d, dtype=td, device=dev)
    for b in range(w.B):
        qb = gen_queries(w, b)
        q[b] = up(qb)
        for h in range(w.Hkv):
            Kb, Vb = gen_kv_slice(w, b, h, qb)
            K[b, h] = up(Kb)
            V[b, h] = up(Vb)
    W = up(gen_W(w))
    log(f"inputs resident ({time.time() - t0:.1f} s)")

    tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device=dev)
    ws = torch.zeros(R.recsa_workspace_bytes(sh, w.L, k), dtype=torch.uint8, device=dev)
    width = R.recsa_sel_width(sh, w.L, w.L, k)
    out = torch.empty(w.B, w.n_queries, w.Hq, w.d, dtype=torch.float32, device=dev)
    lse = torch.empty(w.B, w.n_queries, w.Hq, dtype=torch.float32, device=dev)
    sel = torch.empty(w.B, w.n_queries, w.Hkv, T, width, dtype=torch.int32, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        R.recsa_build_tree(sh, K, V, W, 0, w.L, tree)
        if ev:
            ev[1].record()
        R.recsa_decode(sh, q, K, V, tree, w.L, k, out, lse, sel, width, ws)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    build_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    decode_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_per_step = wall * 1e3 / args.steps
    n_queries = w.B * w.n_queries

    bb, n_nodes = build_bytes(w)
    qb_bytes, rows = decode_bytes_per_query(w, k)
    mf_c = shared_level(w.L, w.f, k)[1] if w.dtype == "bf16" else 0
    db = qb_bytes * n_queries
    build_launches = pool_launches(w)
    kinfo = {
        "pool_kernel": dict(bytes=bb / build_launches, ms=build_ms / build_launches,
                            src=kernel_hash("build_tree.hip", "common.hpp", "sizing.hpp")),
        "attend_kernel": dict(bytes=db, ms=decode_ms, src=kernel_hash("attend.hip", "common.hpp", "lanes.hpp", "sizing.hpp"),
                              unique=decode_unique_bytes(w, k, sel.cpu().numpy())),
    }
    dom = "pool_kernel" if build_ms >= decode_ms else "attend_kernel"

    def roof(name):
        ki = kinfo[name]
        ach = ki["bytes"] / (ki["ms"] * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(name, ki["src"], w.name),
             "kernel": name}
        if probe and "read_GBps" in probe:
            r["measured_read_peak"] = probe["read_GBps"]
            r["frac_of_measured_read"] = round(ach / probe["read_GBps"], 4)
        if "unique" in ki:
            # HBM counts the distinct rows of the call (the union over its queries, from its own
            # selections): what it must at least bring from HBM. The per-query row bytes (what
            # the queries would read with no sharing, mostly cache hits) are an effective
            # bandwidth, reported apart.
            ua = ki["unique"] / (ki["ms"] * 1e-3) / 1e9
            r["effective_GBps"] = r["achieved"]
            r["effective_frac"] = r["frac"]
            r["per_query_row_bytes"] = ki["bytes"]
            r["achieved"] = round(ua, 1)
            r["frac"] = round(ua / HBM_PEAK_GBS, 4)
            r["algorithmic_bytes"] = ki["unique"]
            if probe and "read_GBps" in probe:
                r["frac_of_measured_read"] = round(ua / probe["read_GBps"], 4)
        if name == "pool_kernel" and probe and "read16_write1_GBps" in probe:
            # the build reads every child row once and writes one node row per f rows read
            r["measured_mix_peak"] = probe["read16_write1_GBps"]
            r["frac_of_measured_mix"] = round(ach / probe["read16_write1_GBps"], 4)
        return r

    res = {
        "metric": METRIC,
        "value": round(n_queries / (ms_per_step * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"recsa-{w.name}: tree build + batched decode, B={w.B}, L={w.L}, "
                               f"Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}, fanout={w.f}, k={w.k}, "
                               f"{w.n_queries} queries/sequence",
                   "global_batch": n_queries, "seq_len": w.L, "parallelism": "none (1 GPU)"},
        "roofline": roof(dom),
        "breakdown": {
            "build_ms": round(build_ms, 4), "decode_ms": round(decode_ms, 4),
            "build_GBps": round(bb / (build_ms * 1e-3) / 1e9, 1),
            "decode_queries_per_s": round(n_queries / (decode_ms * 1e-3), 1),
            "decode_bytes_per_query": qb_bytes, "decode_rows_per_unit": rows,
            "build_bytes": bb, "tree_nodes_per_slice": n_nodes,
            "roofline_other": roof("attend_kernel" if dom == "pool_kernel" else "pool_kernel"),
            "decode_alu": valu_roofline(w, rows, n_queries, decode_ms, mf_rows=mf_c),
            "decode_mfma": mfma_share(w, n_queries, decode_ms, mf_c, rows),
            "needle_recall": needle_recall(w, sel.cpu().numpy(), cpu),
            "hbm_probe": probe,
        },
    }

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    if not args.no_legs:
        log("comparison legs: dense decode, prefill")
        legs = {}
        # dense attention at the same context; keys rotated once beforehand, as a dense cache holds them
        Kr = torch.empty_like(K)
        R.recsa_rotate_keys(sh, K, w.L, Kr)
        mode = R.RECSA_DENSE_KEYS_ROTATED
        if not args.no_dense:
            dws = torch.empty(max(R.recsa_dense_workspace_bytes(sh, w.L, w.n_queries, mode), 16), dtype=torch.uint8,
                              device=dev)
            dout = torch.empty_like(out)
            ms = timed(lambda: R.recsa_dense_ref_attn(sh, q, 0, Kr, V, w.L, mode, dout, None, dws), 3)
            legs["dense_decode_batched"] = {"ms_per_call": round(ms, 4), "queries_per_call": n_queries,
                                            "queries_per_s": round(n_queries / (ms * 1e-3), 1)}
            q1 = q[:, :1].contiguous()
            o1 = torch.empty(w.B, 1, w.Hq, w.d, dtype=torch.float32, device=dev)
            dws1 = torch.empty(max(R.recsa_dense_workspace_bytes(sh, w.L, 1, mode), 16), dtype=torch.uint8,
                               device=dev)
            ms = timed(lambda: R.recsa_dense_ref_attn(sh, q1, 0, Kr, V, w.L, mode, o1, None, dws1), 10)
            legs["dense_decode_step"] = {"ms_per_call": round(ms, 4), "queries_per_call": w.B,
                                         "queries_per_s": round(w.B / (ms * 1e-3), 1),
                                         "GBps": round(2 * w.B * w.Hkv * w.L * w.d * w.elem_bytes / (ms * 1e-3) / 1e9,
                                                       1)}
        # causal prefill of the last chunk of positions [L - c, L): RecSA over the built tree, dense over all keys
        from synthetic import with_overrides
        c = args.prefill_chunk
        wq = with_overrides(w, seed=w.seed + 1000)
        qp = torch.empty(w.B, c, w.Hq, w.d, dtype=td, device=dev)
        for b in range(w.B):
            qp[b] = up(gen_queries(wq, b, c))
        pout = torch.empty(w.B, c, w.Hq, w.d, dtype=torch.float32, device=dev)
        pws = torch.empty(R.recsa_workspace_bytes(sh, w.L, k), dtype=torch.uint8, device=dev)
        ms = timed(lambda: R.recsa_prefill(sh, qp, w.L - c, K, V, tree, k, pout, None, None, 0, pws), 3)
        legs["recsa_prefill_last_chunk"] = {"ms_per_call": round(ms, 4), "tokens_per_call": w.B * c,
                                            "tokens_per_s": round(w.B * c / (ms * 1e-3), 1),
                                            "positions": [w.L - c, w.L],
                                            # a position within c of L scores and reads what a
                                            # query at L does
                                            "roofline_alu": valu_roofline(w, rows, w.B * c, ms, mf_rows=mf_c),
                                            "mfma": mfma_share(w, w.B * c, ms, mf_c, rows)}
        psw = R.recsa_sel_width(sh, w.L - c + 1, w.L, k)
        psel = torch.empty(w.B, c, w.Hkv, len(k), psw, dtype=torch.int32, device=dev)
        R.recsa_prefill(sh, qp, w.L - c, K, V, tree, k, pout, None, psel, psw, pws)
        legs["recsa_prefill_last_chunk"]["tile_sharing"] = tile_sharing(psel.cpu().numpy())
        del psel
        if args.no_dense:
            del Kr
            res["breakdown"]["legs"] = legs
    if not args.no_legs and not args.no_dense:
        pmode = R.RECSA_DENSE_KEYS_ROTATED | R.RECSA_DENSE_CAUSAL
        dpws = torch.empty(max(R.recsa_dense_workspace_bytes(sh, w.L, c, pmode), 16), dtype=torch.uint8, device=dev)
        ms = timed(lambda: R.recsa_dense_ref_attn(sh, qp, w.L - c, Kr, V, w.L, pmode, pout, None, dpws), 2)
        flops = 4.0 * w.B * w.Hq * w.d * sum(range(w.L - c + 1, w.L + 1))
        legs["dense_prefill_last_chunk"] = {"ms_per_call": round(ms, 4), "tokens_per_call": w.B * c,
                                            "tokens_per_s": round(w.B * c / (ms * 1e-3), 1),
                                            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1)}
        legs["speedup_decode_batched"] = round(legs["dense_decode_batched"]["ms_per_call"] / decode_ms, 2)
        legs["speedup_prefill_last_chunk"] = round(legs["dense_prefill_last_chunk"]["ms_per_call"] /
                                                   legs["recsa_prefill_last_chunk"]["ms_per_call"], 2)
        if not args.no_library_legs:
            log("library flash-attention legs (timing only)")
            legs["library_sdpa"] = library_legs(w, Kr, V, q, qp, c, timed)
        del Kr
        res["breakdown"]["legs"] = legs

    if not args.no_step_mode:
        one_q = q[:, :1].contiguous()
        o1 = torch.empty(w.B, 1, w.Hq, w.d, dtype=torch.float32, device=dev)
        for _ in range(3):
            R.recsa_decode(sh, one_q, K, V, tree, w.L, k, o1, None, None, 0, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_calls = 64
        q_steps = [q[:, i:i + 1].contiguous() for i in range(n_calls)]
        torch.cuda.synchronize()
        e0.record()
        for i in range(n_calls):
            R.recsa_decode(sh, q_steps[i], K, V, tree, w.L, k, o1, None, None, 0, ws)
        e1.record()
        torch.cuda.synchronize()
        per = e0.elapsed_time(e1) / n_calls
        res["breakdown"]["step_mode"] = {"ms_per_call": round(per, 4), "queries_per_call": w.B,
                                         "queries_per_s": round(w.B / (per * 1e-3), 1)}

        # autoregressive decoding: the cache's last S positions generated again, one
        # recsa_decode_step per token (append, build what completes, attend with the own token).
        # Re-appending a cached token rebuilds its completed nodes bit for bit, so the work per
        # step is exactly that of generating at that position.
        S = min(256, w.n_queries)
        n0 = w.L - S
        kn = K[:, :, n0:].permute(2, 0, 1, 3).contiguous()
        vn = V[:, :, n0:].permute(2, 0, 1, 3).contiguous()
        qs = q[:, :S].transpose(0, 1).contiguous()
        gout = torch.empty(S, w.B, w.Hq, w.d, dtype=torch.float32, device=dev)

        def generate():
            for s in range(S):
                R.recsa_decode_step(sh, qs[s], kn[s], vn[s], K, V, W, tree, n0 + s, k, gout[s], None, None, 0, ws)

        def generate_unfused():
            for s in range(S):
                t = n0 + s
                K[:, :, t].copy_(kn[s])
                V[:, :, t].copy_(vn[s])
                R.recsa_build_tree(sh, K, V, W, t, t + 1, tree)
                R.recsa_prefill(sh, qs[s].unsqueeze(1), t, K, V, tree, k, gout[s].unsqueeze(1), None, None, 0, ws)

        gen = {"positions": [n0, w.L], "tokens_per_step": w.B}
        for name, fn in (("fused", generate), ("unfused", generate_unfused)):
            fn()
            torch.cuda.synchronize()
            h0 = time.perf_counter()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            host = (time.perf_counter() - h0) * 1e3 / S
            per = e0.elapsed_time(e1) / S
            gen[name] = {"ms_per_step": round(per, 4), "tokens_per_s": round(w.B / (per * 1e-3), 1),
                         "host_ms_per_step": round(host, 4)}
        res["breakdown"]["generation"] = gen
        del kn, vn, qs, gout

    if not args.no_two_stage:
        # two-stage block-then-token selection over the same cache and tree: every block (level-1
        # node) scored, the best ts_blocks kept, their tokens scored, the best ts_tokens attended
        log("two-stage variant: batched and one-query decode")
        kb_, kt_ = args.ts_blocks, args.ts_tokens
        n1 = w.L // w.f
        s1 = min(kb_, n1)
        C0 = w.f * s1 + w.L - w.f * n1
        s0 = min(kt_, C0)
        bk = torch.empty(w.B, w.Hkv, n1, w.d, dtype=td, device=dev)
        R.recsa_two_stage_rotate_blocks(sh, tree, 0, w.L, bk)
        tout = torch.empty_like(out)
        tws = torch.empty(R.recsa_two_stage_workspace_bytes(sh, w.L, w.n_queries, kb_, kt_), dtype=torch.uint8,
                          device=dev)
        ms_rot = timed(lambda: R.recsa_two_stage_decode(sh, q, K, V, tree, w.L, kb_, kt_, tout, workspace=tws), 5)
        ms_cached = timed(lambda: R.recsa_two_stage_decode(sh, q, K, V, tree, w.L, kb_, kt_, tout, block_keys=bk,
                                                           workspace=tws), 5)
        one_q = q[:, :1].contiguous()
        o1 = torch.empty(w.B, 1, w.Hq, w.d, dtype=torch.float32, device=dev)
        tws1 = torch.empty(R.recsa_two_stage_workspace_bytes(sh, w.L, 1, kb_, kt_, True), dtype=torch.uint8, device=dev)
        ms_step = timed(lambda: R.recsa_two_stage_decode(sh, one_q, K, V, tree, w.L, kb_, kt_, o1, block_keys=bk,
                                                         workspace=tws1), 32)
        esz = w.elem_bytes
        block_bytes = w.B * w.Hkv * n1 * w.d * esz               # every block key, once per call
        tok_bytes_q = w.Hkv * (C0 + s0) * w.d * esz              # per query: candidate key rows + kept value rows
        flops_q = 2.0 * w.d * w.Hq * n1                          # per query: block logits
        res["breakdown"]["two_stage"] = {
            "k_block": kb_, "k_token": kt_, "blocks": n1, "token_candidates": C0, "tokens_kept": s0,
            "batched": {"ms_per_call": round(ms_rot, 4), "queries_per_call": n_queries,
                        "queries_per_s": round(n_queries / (ms_rot * 1e-3), 1),
                        "note": "block keys rotated inside the call"},
            "batched_rotated_block_cache": {
                "ms_per_call": round(ms_cached, 4), "queries_per_s": round(n_queries / (ms_cached * 1e-3), 1),
                "block_TFLOPs": round(flops_q * n_queries / (ms_cached * 1e-3) / 1e12, 1),
                "token_GBps": round(tok_bytes_q * n_queries / (ms_cached * 1e-3) / 1e9, 1)},
            "step_rotated_block_cache": {
                "ms_per_call": round(ms_step, 4), "queries_per_call": w.B,
                "queries_per_s": round(w.B / (ms_step * 1e-3), 1),
                "GBps": round((block_bytes + tok_bytes_q * w.B) / (ms_step * 1e-3) / 1e9, 1)},
            "per_query": {"block_flops": flops_q, "token_bytes": tok_bytes_q}, "block_key_bytes": block_bytes,
            "speedup_vs_dense_step": (round(res["breakdown"]["legs"]["dense_decode_step"]["ms_per_call"] / ms_step, 2)
                                      if "legs" in res["breakdown"] else None),
        }
        del bk, tout, tws, tws1, o1

    if not args.no_backward:
        # gradients with the forward's selections held fixed: the batched decode's 1024 queries,
        # and causal prefill of the last 4096 positions of each sequence
        log("gradients: batched decode, prefill chunk")
        bwd = {}
        bws = torch.zeros(R.recsa_backward_workspace_bytes(sh, w.L, k), dtype=torch.uint8, device=dev)
        dK = torch.zeros(w.B, w.Hkv, w.L, w.d, dtype=torch.float32, device=dev)
        dV = torch.zeros_like(dK)
        dW = torch.zeros(w.d, w.d, dtype=torch.float32, device=dev)
        R.recsa_decode(sh, q, K, V, tree, w.L, k, out, lse, sel, width, ws)
        dout = torch.randn(out.shape, device=dev, generator=torch.Generator(device=dev).manual_seed(5))
        dq = torch.empty_like(out)
        ms = timed(lambda: R.recsa_backward(sh, False, q, 0, w.L, K, V, W, tree, k, out, lse, sel, width, dout, dq, dK,
                                            dV, dW, workspace=bws), 3)
        bwd["decode_batched"] = {"ms_per_call": round(ms, 4), "queries_per_call": n_queries,
                                 "queries_per_s": round(n_queries / (ms * 1e-3), 1),
                                 "forward_ms": round(decode_ms, 4)}
        c = args.prefill_chunk
        from synthetic import with_overrides as _wo
        wq = _wo(w, seed=w.seed + 1000)
        qc = torch.empty(w.B, c, w.Hq, w.d, dtype=td, device=dev)
        for b in range(w.B):
            qc[b] = up(gen_queries(wq, b, c))
        csw = R.recsa_sel_width(sh, w.L - c + 1, w.L, k)
        cout = torch.empty(w.B, c, w.Hq, w.d, dtype=torch.float32, device=dev)
        clse = torch.empty(w.B, c, w.Hq, dtype=torch.float32, device=dev)
        csel = torch.empty(w.B, c, w.Hkv, len(k), csw, dtype=torch.int32, device=dev)
        fwd_ms = timed(lambda: R.recsa_prefill(sh, qc, w.L - c, K, V, tree, k, cout, clse, csel, csw, ws), 3)
        cdout = torch.randn(cout.shape, device=dev, generator=torch.Generator(device=dev).manual_seed(6))
        cdq = torch.empty_like(cout)
        ms = timed(lambda: R.recsa_backward(sh, True, qc, w.L - c, 0, K, V, W, tree, k, cout, clse, csel, csw, cdout, cdq,
                                            dK, dV, dW, workspace=bws), 2)
        bwd["prefill_last_chunk"] = {"ms_per_call": round(ms, 4), "tokens_per_call": w.B * c,
                                     "tokens_per_s": round(w.B * c / (ms * 1e-3), 1), "forward_ms": round(fwd_ms, 4)}
        del bws, dK, dV, dW, dout, dq, qc, cout, clse, csel, cdout, cdq
        # pooler distillation: one step = tree rebuild with the current pooler, decode of the 1024
        # queries, squared-error loss against full attention's outputs (computed once, outside
        # the timed steps), gradient for W only, update
        mode = R.RECSA_DENSE_KEYS_ROTATED
        Kr = torch.empty_like(K)
        R.recsa_rotate_keys(sh, K, w.L, Kr)
        tgt = torch.empty_like(out)
        dws = torch.empty(max(R.recsa_dense_workspace_bytes(sh, w.L, w.n_queries, mode), 16), dtype=torch.uint8,
                          device=dev)
        R.recsa_dense_ref_attn(sh, q, 0, Kr, V, w.L, mode, tgt, None, dws)
        del Kr, dws
        Wm = W.float().clone()
        Wd = W.clone()
        dtree = torch.zeros_like(tree)
        dloss = torch.zeros(4, dtype=torch.float32, device=dev)
        dws = torch.zeros(R.recsa_distill_workspace_bytes(sh, w.L, w.n_queries, k), dtype=torch.uint8, device=dev)
        losses = []

        def dstep():
            R.recsa_distill_step(sh, q, K, V, w.L, k, tgt, 1.0, Wm, Wd, dtree, dloss, dws)

        dstep()
        losses.append(float(dloss[0].cpu()))
        ms = timed(dstep, 3)
        losses.append(float(dloss[0].cpu()))
        bwd["distill_step"] = {"ms_per_step": round(ms, 4), "queries_per_step": n_queries,
                               "loss_first_last": [round(losses[0], 8), round(losses[-1], 8)]}
        res["breakdown"]["backward"] = bwd
        del Wm, Wd, dtree, dloss, dws, tgt

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        res["breakdown"]["calib_copy_bytes"] = 1 << 30

    if not args.no_prefill64k:
        log("64K chunked prefill workload")
        res["breakdown"]["prefill_64k"] = prefill_64k_leg(R, dev, timed, dense=not args.no_dense)
        if cpu is not None:
            res["breakdown"]["prefill_64k"]["cpu_oracle_tokens_per_s"] = round(cpu["prefill_64k"]["tokens_per_s"], 2)

    if cpu is not None:
        cpu.pop("_needle_hits", None)
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
