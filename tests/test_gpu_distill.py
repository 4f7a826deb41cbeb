"""GPU parity of one pooler-distillation step (recsa_distill_step) against the oracle's step, and a
short run whose loss goes down. The distillation target (full attention's outputs on the same
queries) is computed by the oracle and handed to both sides."""
import numpy as np
import pytest
import torch

from oracle import level_counts
from oracle.distill import dense_targets, distill_step
from gpu_util import dev_tensor, storage_bits
from long_context_hierarchical_amd import recsa as R
from synthetic import Workload, gen_decode_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _w(name, Hq, Hkv, d, dtype, L, f, k, n_queries, seed, w_gain):
    std = 1.0   # unit-scale logits: RecSA's outputs differ visibly from the target
    return Workload(name, B=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, L=L, f=f, k=k, n_queries=n_queries, mode="decode",
                    std=std, w_gain=w_gain, seed=seed)


CASES = [
    _w("dist_bf16_d128_G4_f16", 8, 2, 128, "bf16", 16 ** 3 + 300, 16, 4, 4, 61, 0.5),
    _w("dist_f32_d64_G2_f4", 4, 2, 64, "f32", 900, 4, 2, 6, 62, 0.5),
]


def _setup(w):
    inp = gen_decode_inputs(w)
    T = len(level_counts(w.L, w.f))
    k = [w.k] * T
    target = dense_targets(inp["K"], inp["V"], inp["q"], w.dtype, w.theta, n_tokens=w.L)
    sh = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, w.L, 0.0, w.theta)
    dev = "cuda:0"
    g = dict(K=dev_tensor(inp["K"], w.dtype), V=dev_tensor(inp["V"], w.dtype), q=dev_tensor(inp["q"], w.dtype),
             W=dev_tensor(inp["W"], w.dtype), target=torch.from_numpy(target).to(dev))
    Wf = inp["W"].astype(np.float32) if w.dtype == "f32" else (inp["W"].astype(np.uint32) << 16).view(np.float32)
    g["W_master"] = torch.from_numpy(Wf.copy()).to(dev)
    g["tree"] = torch.zeros(R.recsa_tree_bytes(sh), dtype=torch.uint8, device=dev)
    g["loss"] = torch.zeros(4, dtype=torch.float32, device=dev)
    g["ws"] = torch.zeros(R.recsa_distill_workspace_bytes(sh, w.L, inp["q"].shape[1], k), dtype=torch.uint8, device=dev)
    return inp, k, target, sh, g


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_distill_step_matches_oracle(w):
    inp, k, target, sh, g = _setup(w)
    lr = 0.5 if w.dtype == "f32" else 50.0   # bf16 gradients are small: a step well above float32's resolution
    W0 = g["W_master"].clone()
    R.recsa_distill_step(sh, g["q"], g["K"], g["V"], w.L, k, g["target"], lr, g["W_master"], g["W"], g["tree"],
                         g["loss"], g["ws"])
    torch.cuda.synchronize()
    loss = float(g["loss"][0].cpu())
    step = (g["W_master"] - W0).cpu().numpy().astype(np.float64)
    _say(f"distill {w.name}: gpu loss {loss:.6g}")
    ref = distill_step(inp["K"], inp["V"], inp["W"], inp["q"], target, w.f, k, w.dtype, lr, w.L, w.theta)
    for r in ref["results"].values():
        assert not any(r.flags.values()), "near tie in the oracle's selections"
    ref_step = ref["W_master"] - W0.cpu().numpy().astype(np.float64)
    _say(f"distill {w.name}: oracle loss {ref['loss']:.6g}; max |step| {np.abs(ref_step).max():.3g}, "
         f"max |gpu - oracle| {np.abs(step - ref_step).max():.3g}")
    assert loss == pytest.approx(ref["loss"], rel=1e-4)
    # the float32 master copy rounds each updated entry (half an ulp of |W| each side)
    ulp = 2.0 ** -23 * float(np.abs(W0.cpu().numpy()).max())
    assert np.abs(step - ref_step).max() <= 1e-4 * np.abs(ref_step).max() + 2 * ulp
    # the pooler the next step uses is the master copy rounded to the storage type
    Wm = g["W_master"].cpu()
    Wr = Wm.to(torch.bfloat16) if w.dtype == "bf16" else Wm
    assert np.array_equal(storage_bits(g["W"]), storage_bits(Wr))


def test_distill_run_lowers_the_loss():
    w = CASES[1]
    inp, k, target, sh, g = _setup(w)
    losses = []
    for _ in range(20):
        R.recsa_distill_step(sh, g["q"], g["K"], g["V"], w.L, k, g["target"], 0.5, g["W_master"], g["W"], g["tree"],
                             g["loss"], g["ws"])
        losses.append(float(g["loss"][0].cpu()))
    _say(f"distill run: loss {losses[0]:.5g} -> {losses[-1]:.5g}")
    assert all(np.isfinite(losses)) and losses[-1] < 0.9 * losses[0]
