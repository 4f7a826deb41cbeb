"""GPU parity of autoregressive decoding (recsa_decode_step) against the oracle's step-by-step
generation: every step's selections and outputs, then the caches and the tree bit for bit.

The cache rows the steps will write start out as NaN on the device, so a token written to the
wrong row, or a node built from a row that was not written, shows up in the outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, check_unit, dev_tensor, storage_bits
from long_context_hierarchical_amd import recsa as R
from synthetic import Workload, gen_decode_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _w(name, B, Hq, Hkv, d, dtype, L, f, k, seed, theta=1.0e6):
    std = 1.0 if dtype == "f32" else d ** -0.5
    return Workload(name, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, L=L, f=f, k=k, n_queries=1, mode="decode",
                    std=std, theta=theta, seed=seed)


# (workload, first generated position); the workload's L is the position after the last step.
# Each case crosses a completion cascade: t + 1 = 192 and 256 (f = 4: three and four levels),
# 4096 (f = 16: three levels), 2048 (f = 32: two levels), 9 and 27 (f = 3, division path).
STEP_CASES = [
    (_w("s_bf16_d128_f4_G4", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", L=270, f=4, k=2, seed=41), 190),
    (_w("s_f32_d64_f3_G1_empty", B=1, Hq=2, Hkv=2, d=64, dtype="f32", L=30, f=3, k=2, seed=42), 0),
    (_w("s_bf16_d128_f16_G8", B=1, Hq=16, Hkv=2, d=128, dtype="bf16", L=16 ** 3 + 40, f=16, k=4, seed=43), 4088),
    (_w("s_bf16_d64_f32_G2", B=1, Hq=4, Hkv=2, d=64, dtype="bf16", L=2 * 32 ** 2 + 12, f=32, k=16, seed=44), 2043),
    (_w("s_f32_d128_f4_norope", B=1, Hq=4, Hkv=1, d=128, dtype="f32", L=80, f=4, k=3, seed=45, theta=0.0), 60),
]


def _nan_rows(a: np.ndarray, start: int, dtype: str) -> np.ndarray:
    a = a.copy()
    if dtype == "bf16":
        a[:, :, start:] = 0x7FC0
    else:
        a[:, :, start:] = np.float32("nan")
    return a


@pytest.mark.parametrize("w,n_start", STEP_CASES, ids=lambda c: c.name if hasattr(c, "name") else str(c))
def test_decode_steps_match_oracle_generation(w, n_start):
    S = w.L - n_start
    _say(f"decode step {w.name}: {S} steps from position {n_start}")
    inp = gen_decode_inputs(w, n_q=S)
    K, V, W = inp["K"], inp["V"], inp["W"]
    q_steps = np.ascontiguousarray(inp["q"].transpose(1, 0, 2, 3))          # [S][B][Hq][d]
    k_steps = np.ascontiguousarray(K[:, :, n_start:].transpose(2, 0, 1, 3))  # [S][B][Hkv][d]
    v_steps = np.ascontiguousarray(V[:, :, n_start:].transpose(2, 0, 1, 3))
    T = R.recsa_num_levels(w.L, w.f)
    k = [w.k] * max(T, 1)

    dev = "cuda:0"
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
    Kd = dev_tensor(_nan_rows(K, n_start, w.dtype), w.dtype)
    Vd = dev_tensor(_nan_rows(V, n_start, w.dtype), w.dtype)
    Wd = dev_tensor(W, w.dtype)
    qd = dev_tensor(q_steps, w.dtype)
    knd, vnd = dev_tensor(k_steps, w.dtype), dev_tensor(v_steps, w.dtype)
    tree = torch.zeros(max(R.recsa_tree_bytes(sh), 16), dtype=torch.uint8, device=dev)
    R.recsa_build_tree(sh, Kd, Vd, Wd, 0, n_start, tree)
    width = max(R.recsa_sel_width(sh, n_start + 1, w.L, k), 1)
    ws = torch.zeros(max(R.recsa_workspace_bytes(sh, w.L, k), 16), dtype=torch.uint8, device=dev)
    out = torch.full((S, w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((S, w.B, w.Hq), float("nan"), dtype=torch.float32, device=dev)
    sel = torch.full((S, w.B, w.Hkv, len(k), width), -7, dtype=torch.int32, device=dev)
    for s in range(S):
        R.recsa_decode_step(sh, qd[s], knd[s], vnd[s], Kd, Vd, Wd, tree, n_start + s, k, out[s], lse[s], sel[s],
                            width, ws)
    torch.cuda.synchronize()
    _say(f"decode step {w.name}: gpu done")

    # the header's contract: the same outputs, bit for bit, as prefill over the final cache
    qp = qd.transpose(0, 1).contiguous()
    outp = torch.empty(w.B, S, w.Hq, w.d, dtype=torch.float32, device=dev)
    lsep = torch.empty(w.B, S, w.Hq, dtype=torch.float32, device=dev)
    selp = torch.full((w.B, S, w.Hkv, len(k), width), -7, dtype=torch.int32, device=dev)
    R.recsa_prefill(sh, qp, n_start, Kd, Vd, tree, k, outp, lsep, selp, width, ws)
    torch.cuda.synchronize()
    assert torch.equal(outp.transpose(0, 1).cpu().view(torch.int32), out.cpu().view(torch.int32))
    assert torch.equal(lsep.transpose(0, 1).cpu().view(torch.int32), lse.cpu().view(torch.int32))
    assert torch.equal(selp.transpose(0, 1).cpu(), sel.cpu())

    res, slices = oracle.generate(K, V, W, q_steps, k_steps, v_steps, n_start, w.f, k, w.dtype, w.theta)
    out, lse, sel = out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()
    G = w.G
    stats = {"match": 0, "replayed": 0}
    for s in range(S):
        for (b, h), r in res[s].items():
            Kf, Vf, tr = slices[(b, h)]
            qg = oracle.from_storage(q_steps[s, b, h * G:(h + 1) * G], w.dtype)
            t = n_start + s

            def rep(fixed, qg=qg, Kf=Kf, Vf=Vf, tr=tr, t=t):
                # the final cache and tree hold everything step s saw; the unit reads only the
                # rows and nodes complete at t + 1
                return oracle.attend_unit(qg, Kf, Vf, tr, t + 1, w.f, k, w.dtype, w.theta, self_in=True,
                                          fixed_sel=fixed)
            st = check_unit(r, sel[s, b, h], out[s, b, h * G:(h + 1) * G], lse[s, b, h * G:(h + 1) * G],
                            TOL[w.dtype], where=f"{w.name} step {s} slice {(b, h)}", replay=rep)
            stats[st] += 1
    _say(f"decode step {w.name}: {stats}")

    Kg, Vg = storage_bits(Kd), storage_bits(Vd)
    for (b, h), (Kf, Vf, tr) in slices.items():
        for got, ref in ((Kg[b, h], Kf), (Vg[b, h], Vf)):
            assert np.array_equal(got, oracle.to_storage(ref, w.dtype).view(got.dtype)), (b, h)
        for lv in range(1, T + 1):
            NK, NV = R.tree_level_views(sh, tree, lv)
            for arr, ref in ((NK, tr[lv - 1][0]), (NV, tr[lv - 1][1])):
                got = storage_bits(arr[b, h])
                assert np.array_equal(got, oracle.to_storage(ref, w.dtype).view(got.dtype)), (b, h, lv)
