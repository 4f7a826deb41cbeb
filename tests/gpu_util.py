"""Helpers for the GPU parity tests: upload synthetic inputs, call the library through its
binding, and compare one (sequence, query, KV head) unit with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from long_context_hierarchical_amd import recsa as R

TOL = {"f32": 1e-5, "bf16": 2e-3}


def dev_tensor(a: np.ndarray, dtype: str, dev="cuda:0") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(dev)


def storage_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


class Gpu:
    """Device copies of one workload plus its tree, built through the library."""

    def __init__(self, w, inp, cap=None, build=True, dev="cuda:0"):
        self.w, self.dev = w, dev
        cap = w.L if cap is None else cap
        self.shape = R.Shape(w.B, w.Hkv, w.Hq, w.d, w.f, w.dtype, cap, 0.0, w.theta)
        self.K = dev_tensor(inp["K"], w.dtype, dev)
        self.V = dev_tensor(inp["V"], w.dtype, dev)
        self.W = dev_tensor(inp["W"], w.dtype, dev)
        self.q = dev_tensor(inp["q"], w.dtype, dev)
        self.tree = torch.zeros(max(R.recsa_tree_bytes(self.shape), 16), dtype=torch.uint8, device=dev)
        if build:
            R.recsa_build_tree(self.shape, self.K, self.V, self.W, 0, cap, self.tree)

    def _alloc(self, n_q, n_levels, width):
        w = self.w
        out = torch.full((w.B, n_q, w.Hq, w.d), float("nan"), dtype=torch.float32, device=self.dev)
        lse = torch.full((w.B, n_q, w.Hq), float("nan"), dtype=torch.float32, device=self.dev)
        sel = torch.full((w.B, n_q, w.Hkv, n_levels, max(width, 1)), -7, dtype=torch.int32, device=self.dev)
        return out, lse, sel

    def decode(self, k, n_tokens, q=None):
        q = self.q if q is None else q
        width = R.recsa_sel_width(self.shape, n_tokens, n_tokens, k)
        ws = torch.zeros(max(R.recsa_workspace_bytes(self.shape, n_tokens, k), 16), dtype=torch.uint8, device=self.dev)
        out, lse, sel = self._alloc(q.shape[1], len(k), width)
        R.recsa_decode(self.shape, q, self.K, self.V, self.tree, n_tokens, k, out, lse, sel, max(width, 1), ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy(), ws

    def prefill(self, k, q_start, n_q, q=None):
        q = self.q[:, q_start:q_start + n_q].contiguous() if q is None else q
        width = R.recsa_sel_width(self.shape, q_start + 1, q_start + n_q, k)
        ws = torch.zeros(max(R.recsa_workspace_bytes(self.shape, q_start + n_q, k), 16), dtype=torch.uint8,
                         device=self.dev)
        out, lse, sel = self._alloc(n_q, len(k), width)
        R.recsa_prefill(self.shape, q, q_start, self.K, self.V, self.tree, k, out, lse, sel, max(width, 1), ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy(), ws


def compare_unit(r, sel_rows: np.ndarray, out: np.ndarray, lse: np.ndarray, tol: float, where=""):
    """Selections level by level, then outputs. Returns 'match', or 'excused' when the two
    sides split a flagged near tie differently (levels below it are then not comparable)."""
    T = len(r.sel)
    for lv in range(T, 0, -1):
        got = [int(x) for x in sel_rows[lv - 1] if x >= 0]
        assert all(x == -1 for x in sel_rows[lv - 1][len(got):]), f"{where} level {lv}: bad padding"
        if got != r.sel[lv]:
            assert r.flags.get(lv), f"{where} level {lv}: kept {got} vs oracle {r.sel[lv]}"
            return "excused"
    for lv in range(T + 1, sel_rows.shape[0] + 1):
        assert np.all(sel_rows[lv - 1] == -1), f"{where} level {lv} above the tree is not empty"
    err = np.abs(out.astype(np.float64) - r.out).max() if r.z is not None else np.abs(out).max()
    assert err <= tol, f"{where} max |out - oracle| = {err:.3g} > {tol}"
    if r.z is not None:
        lerr = np.abs(lse.astype(np.float64) - r.lse).max()
        assert lerr <= 10 * tol, f"{where} lse error {lerr:.3g}"
    else:
        assert np.all(np.isneginf(lse)), where
    return "match"
