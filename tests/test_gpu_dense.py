"""GPU parity of the dense comparator (standard RoPE attention at original positions) and of
the key-rotation pre-pass, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, dev_tensor, storage_bits
from long_context_hierarchical_amd import recsa as R
from synthetic import Workload, gen_decode_inputs

pytestmark = pytest.mark.gpu


def _w(name, B=1, Hq=4, Hkv=1, d=64, dtype="f32", L=1000, n_queries=3, **kw):
    std = 1.0 if dtype == "f32" else d ** -0.5
    return Workload(name, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, L=L, f=16, k=8, n_queries=n_queries,
                    mode="decode", std=std, **kw)


def _setup(w, n_q=None):
    inp = gen_decode_inputs(w, n_q=n_q)
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
    return inp, sh, dev_tensor(inp["K"], w.dtype), dev_tensor(inp["V"], w.dtype), dev_tensor(inp["q"], w.dtype)


def test_rotate_keys_bitwise():
    for w in (_w("rk_bf16", Hq=8, Hkv=2, d=128, dtype="bf16", L=3000, seed=41),
              _w("rk_f32", d=64, dtype="f32", L=2000, seed=42)):
        inp, sh, K, V, q = _setup(w, n_q=1)
        Kr = torch.zeros_like(K)
        R.recsa_rotate_keys(sh, K, w.L, Kr)
        torch.cuda.synchronize()
        for b in range(w.B):
            for h in range(w.Hkv):
                Kf = oracle.from_storage(inp["K"][b, h], w.dtype)
                c, s = oracle.rope_rows(np.arange(w.L), w.d, w.theta)
                want = oracle.to_storage(oracle.rotate(Kf, c, s, w.dtype), w.dtype)
                got = storage_bits(Kr[b, h])
                assert np.array_equal(got, want.view(got.dtype)), (w.name, b, h, int(np.sum(got != want.view(got.dtype))))


DENSE_CASES = [
    (_w("dn_f32_G4", d=64, dtype="f32", L=1000, seed=51), 0.0),
    (_w("dn_bf16_G4_d128", Hq=8, Hkv=2, d=128, dtype="bf16", L=1500, seed=52), 0.0),
    (_w("dn_bf16_G2_d64", B=2, Hq=4, Hkv=2, d=64, dtype="bf16", L=777, seed=53), 0.0),
    (_w("dn_bf16_G8", Hq=16, Hkv=2, d=128, dtype="bf16", L=1200, seed=54), 0.0),
    (_w("dn_bf16_G1", Hq=2, Hkv=2, d=128, dtype="bf16", L=600, seed=55), 0.0),
    (_w("dn_bf16_split", Hq=4, Hkv=1, d=128, dtype="bf16", L=20000, n_queries=1, seed=56), 0.0),
    (_w("dn_bf16_norope", Hq=8, Hkv=2, d=128, dtype="bf16", L=900, theta=0.0, seed=57), 0.0),
]


def _compare(w, inp, out, lse, rows, mode):
    G = w.G
    for (b, j, h, n_keys, q_pos) in rows:
        qg = oracle.from_storage(inp["q"][b, j, h * G:(h + 1) * G], w.dtype)
        Kf = oracle.from_storage(inp["K"][b, h], w.dtype)
        Vf = oracle.from_storage(inp["V"][b, h], w.dtype)
        ro, rl = oracle.dense_unit(qg, Kf, Vf, n_keys, q_pos, w.dtype, w.theta)
        err = np.abs(out[b, j, h * G:(h + 1) * G] - ro).max()
        assert err <= TOL[w.dtype], (w.name, mode, b, j, h, err)
        # lse: 10 times the output tolerance (the worst-case float32 bound for a sum of up to
        # 2M terms, n * 2^-23, would be vacuous here)
        lerr = np.abs(lse[b, j, h * G:(h + 1) * G] - rl).max()
        assert lerr <= 10 * TOL[w.dtype], (w.name, mode, b, j, h, lerr)


@pytest.mark.parametrize("w,_", DENSE_CASES, ids=lambda x: getattr(x, "name", ""))
@pytest.mark.parametrize("rotated", [False, True])
def test_dense_decode(w, _, rotated):
    inp, sh, K, V, q = _setup(w)
    Kin = K
    mode = 0
    if rotated:
        Kin = torch.zeros_like(K)
        R.recsa_rotate_keys(sh, K, w.L, Kin)
        mode |= R.RECSA_DENSE_KEYS_ROTATED
    ws = torch.zeros(max(R.recsa_dense_workspace_bytes(sh, w.L, w.n_queries, mode), 16), dtype=torch.uint8, device="cuda")
    out = torch.full((w.B, w.n_queries, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((w.B, w.n_queries, w.Hq), float("nan"), device="cuda")
    R.recsa_dense_ref_attn(sh, q, 0, Kin, V, w.L, mode, out, lse, ws)
    torch.cuda.synchronize()
    rows = [(b, j, h, w.L, w.L) for b in range(w.B) for j in range(w.n_queries) for h in range(w.Hkv)]
    _compare(w, inp, out.cpu().numpy(), lse.cpu().numpy(), rows, mode)


@pytest.mark.parametrize("w,_", DENSE_CASES[:5], ids=lambda x: getattr(x, "name", ""))
def test_dense_causal_prefill(w, _):
    n_q = min(w.L, 300)
    inp, sh, K, V, q = _setup(w, n_q=w.L)
    q_start = w.L - n_q
    qs = q[:, q_start:].contiguous()
    mode = R.RECSA_DENSE_CAUSAL
    ws = torch.zeros(max(R.recsa_dense_workspace_bytes(sh, w.L, n_q, mode), 16), dtype=torch.uint8, device="cuda")
    out = torch.full((w.B, n_q, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((w.B, n_q, w.Hq), float("nan"), device="cuda")
    R.recsa_dense_ref_attn(sh, qs, q_start, K, V, w.L, mode, out, lse, ws)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    inp_slice = dict(inp)
    inp_slice["q"] = inp["q"][:, q_start:]
    picks = sorted(set([0, 1, 2, 15, 16, 17, n_q - 1] + list(range(100, 140))))
    rows = [(b, j, h, q_start + j + 1, q_start + j) for b in range(w.B) for j in picks if j < n_q
            for h in range(w.Hkv)]
    _compare(w, inp_slice, out, lse, rows, mode)


def test_dense_matches_no_pruning_tree_path():
    """With every level keeping everything, the tree path is dense attention: both GPU paths agree."""
    w = _w("dn_vs_tree", Hq=8, Hkv=2, d=128, dtype="bf16", L=2500, n_queries=2, seed=58)
    inp, sh, K, V, q = _setup(w)
    ws = torch.zeros(max(R.recsa_dense_workspace_bytes(sh, w.L, w.n_queries, 0), 16), dtype=torch.uint8, device="cuda")
    out_d = torch.empty(w.B, w.n_queries, w.Hq, w.d, device="cuda")
    R.recsa_dense_ref_attn(sh, q, 0, K, V, w.L, 0, out_d, None, ws)
    W = dev_tensor(inp["W"], w.dtype)
    tree = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device="cuda")
    R.recsa_build_tree(sh, K, V, W, 0, w.L, tree)
    k = [R.INT32_MAX] * R.recsa_num_levels(w.L, w.f)
    ws2 = torch.zeros(R.recsa_workspace_bytes(sh, w.L, k), dtype=torch.uint8, device="cuda")
    out_t = torch.empty_like(out_d)
    R.recsa_decode(sh, q, K, V, tree, w.L, k, out_t, None, None, 0, ws2)
    torch.cuda.synchronize()
    assert (out_d - out_t).abs().max().item() <= TOL["bf16"]


@pytest.mark.parametrize("rotated", [False, True])
def test_dense_at_524k_sampled(rotated):
    """The comparator at the 524K benchmark length (bf16, d = 128, G = 4), where RoPE angles reach
    5e5 rad: decode and the causal last positions, sampled (query, KV head) units against the
    oracle; keys pre-RoPE (rotated into the workspace) or rotated beforehand."""
    L = 524288 + 37
    w = _w("dn_524k", Hq=8, Hkv=2, d=128, dtype="bf16", L=L, n_queries=64, seed=59)
    inp, sh, K, V, q = _setup(w)
    Kin, mode = K, 0
    if rotated:
        Kin = torch.empty_like(K)
        R.recsa_rotate_keys(sh, K, L, Kin)
        mode |= R.RECSA_DENSE_KEYS_ROTATED
    n_dec = 2
    qd = q[:, :n_dec].contiguous()
    nbytes = max(R.recsa_dense_workspace_bytes(sh, L, 64, mode | R.RECSA_DENSE_CAUSAL),
                 R.recsa_dense_workspace_bytes(sh, L, n_dec, mode), 16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((1, n_dec, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((1, n_dec, w.Hq), float("nan"), device="cuda")
    R.recsa_dense_ref_attn(sh, qd, 0, Kin, V, L, mode, out, lse, ws)
    q_start = L - 64
    pout = torch.full((1, 64, w.Hq, w.d), float("nan"), device="cuda")
    plse = torch.full((1, 64, w.Hq), float("nan"), device="cuda")
    R.recsa_dense_ref_attn(sh, q, q_start, Kin, V, L, mode | R.RECSA_DENSE_CAUSAL, pout, plse, ws)
    torch.cuda.synchronize()
    rows = [(0, j, h, L, L) for j in range(n_dec) for h in range(w.Hkv)]
    _compare(w, inp, out.cpu().numpy(), lse.cpu().numpy(), rows, f"decode rotated={rotated}")
    rows = [(0, j, h, q_start + j + 1, q_start + j) for j in (0, 31, 63) for h in range(w.Hkv)]
    _compare(w, inp, pout.cpu().numpy(), plse.cpu().numpy(), rows, f"causal rotated={rotated}")
