"""Python binding of librecsa.so (RecSA tree attention on MI355X).

Argument marshalling only: every function forwards torch tensors' device
pointers and the current HIP stream to the C entry point of the same name
and raises RecsaError on a negative status. There is no fallback: importing
works without the library, but any call fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librecsa.so")

RECSA_F32, RECSA_BF16 = 0, 1
INT32_MAX = 2 ** 31 - 1
EXPORTS = (
    "recsa_abi_version", "recsa_last_error", "recsa_num_levels", "recsa_tree_bytes", "recsa_level_offset",
    "recsa_sel_width", "recsa_workspace_bytes", "recsa_build_tree", "recsa_decode", "recsa_prefill",
    "recsa_decode_step", "recsa_backward_workspace_bytes", "recsa_backward", "recsa_distill_workspace_bytes",
    "recsa_distill_step",
    "recsa_dense_workspace_bytes", "recsa_dense_ref_attn", "recsa_rotate_keys",
    "recsa_two_stage_workspace_bytes", "recsa_two_stage_decode", "recsa_two_stage_rotate_blocks",
    "recsa_decode_noalloc",
)
RECSA_DENSE_CAUSAL, RECSA_DENSE_KEYS_ROTATED = 1, 2


class RecsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"recsa status {code}: {msg}")
        self.code = code


class _Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("fanout", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("capacity", ctypes.c_int64), ("softmax_scale", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("select_heads", ctypes.c_int32),
    ]


@dataclass(frozen=True)
class Shape:
    batch: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    fanout: int
    dtype: str            # 'f32' or 'bf16'
    capacity: int
    softmax_scale: float = 0.0
    rope_theta: float = 1.0e6
    select_heads: int = 0     # query heads per selection (0 = the KV head's group)

    def c(self) -> _Shape:
        # the C struct, built once per (immutable) shape: a decoding loop passes it every step
        st = self.__dict__.get("_c")
        if st is None:
            st = _Shape(self.batch, self.n_kv_heads, self.n_q_heads, self.head_dim, self.fanout,
                        RECSA_BF16 if self.dtype == "bf16" else RECSA_F32, self.capacity,
                        self.softmax_scale, self.rope_theta, self.select_heads)
            object.__setattr__(self, "_c", st)
        return st

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        SP = ctypes.POINTER(_Shape)
        K = ctypes.POINTER(ctypes.c_int32)
        sig = {
            "recsa_abi_version": (I32, []),
            "recsa_last_error": (ctypes.c_char_p, []),
            "recsa_num_levels": (I32, [I64, I32]),
            "recsa_tree_bytes": (I64, [SP]),
            "recsa_level_offset": (I64, [SP, I32, I32]),
            "recsa_sel_width": (I32, [SP, I64, I64, K, I32]),
            "recsa_workspace_bytes": (I64, [SP, I64, K, I32]),
            "recsa_build_tree": (I32, [SP, P, P, P, I64, I64, P, P]),
            "recsa_decode": (I32, [SP, P, I64, P, P, P, I64, K, I32, P, P, P, I32, P, I64, P]),
            "recsa_prefill": (I32, [SP, P, I64, I64, P, P, P, K, I32, P, P, P, I32, P, I64, P]),
            "recsa_decode_noalloc": (I32, [SP, P, I64, P, P, P, I64, K, I32, P, P, P, I32, P]),
            "recsa_decode_step": (I32, [SP, P, P, P, P, P, P, P, I64, K, I32, P, P, P, I32, P, I64, P]),
            "recsa_backward_workspace_bytes": (I64, [SP, I64, K, I32]),
            "recsa_distill_workspace_bytes": (I64, [SP, I64, I64, K, I32]),
            "recsa_distill_step": (I32, [SP, P, I64, P, P, I64, K, I32, P, ctypes.c_float, P, P, P, P, P, I64, P]),
            "recsa_backward": (I32, [SP, I32, P, I64, I64, I64, P, P, P, P, K, I32, P, P, P, I32, P, P, P, P, P, P,
                                     P, I64, P]),
            "recsa_dense_workspace_bytes": (I64, [SP, I64, I64, I32]),
            "recsa_dense_ref_attn": (I32, [SP, P, I64, I64, P, P, I64, I32, P, P, P, I64, P]),
            "recsa_rotate_keys": (I32, [SP, P, I64, P, P]),
            "recsa_two_stage_workspace_bytes": (I64, [SP, I64, I64, I32, I32, I32]),
            "recsa_two_stage_decode": (I32, [SP, P, I64, P, P, P, P, I64, I32, I32, P, P, P, I32, P, I32, P, I64,
                                             P]),
            "recsa_two_stage_rotate_blocks": (I32, [SP, P, I64, I64, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(t):
    # the argument types are c_void_p: an int (or None = NULL) converts directly
    return None if t is None else t.data_ptr()


_K_ARRAYS: dict = {}


def _k(k_levels):
    # the k_l array, built once per distinct tuple (the library reads it during the call only)
    key = tuple(int(x) for x in k_levels)
    hit = _K_ARRAYS.get(key)
    if hit is None:
        hit = ((ctypes.c_int32 * max(len(key), 1))(*key), len(key))
        if len(_K_ARRAYS) < 1024:
            _K_ARRAYS[key] = hit
    return hit


_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    # the HIP stream handle: the given stream's, else torch's current stream on the current device
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is not None:
        return _RAW_STREAM(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int):
    if rc != 0:
        raise RecsaError(rc, lib().recsa_last_error().decode())


def _nbytes(rc: int) -> int:
    if rc < 0:
        raise RecsaError(-1, lib().recsa_last_error().decode())
    return int(rc)


# ----------------------------------------------------------------- sizing

def recsa_abi_version() -> int:
    return int(lib().recsa_abi_version())


def recsa_num_levels(n_tokens: int, fanout: int) -> int:
    return int(lib().recsa_num_levels(n_tokens, fanout))


def recsa_tree_bytes(shape: Shape) -> int:
    return _nbytes(lib().recsa_tree_bytes(ctypes.byref(shape.c())))


def recsa_level_offset(shape: Shape, level: int, which: int) -> int:
    return _nbytes(lib().recsa_level_offset(ctypes.byref(shape.c()), level, which))


def recsa_sel_width(shape: Shape, n_min: int, n_max: int, k_levels) -> int:
    k, nl = _k(k_levels)
    return _nbytes(lib().recsa_sel_width(ctypes.byref(shape.c()), n_min, n_max, k, nl))


def recsa_workspace_bytes(shape: Shape, n_max: int, k_levels) -> int:
    k, nl = _k(k_levels)
    return _nbytes(lib().recsa_workspace_bytes(ctypes.byref(shape.c()), n_max, k, nl))


def recsa_backward_workspace_bytes(shape: Shape, n_max: int, k_levels) -> int:
    k, nl = _k(k_levels)
    return _nbytes(lib().recsa_backward_workspace_bytes(ctypes.byref(shape.c()), n_max, k, nl))


def recsa_dense_workspace_bytes(shape: Shape, n_tokens: int, n_q: int, mode: int) -> int:
    return _nbytes(lib().recsa_dense_workspace_bytes(ctypes.byref(shape.c()), n_tokens, n_q, mode))


# ----------------------------------------------------------------- entry points

def recsa_build_tree(shape: Shape, K, V, W, n_old: int, n_new: int, tree, stream=None):
    _check(lib().recsa_build_tree(ctypes.byref(shape.c()), _p(K), _p(V), _p(W), n_old, n_new, _p(tree),
                                  _stream(stream)))


def recsa_decode(shape: Shape, q, K, V, tree, n_tokens: int, k_levels, out, lse=None, sel=None,
                 sel_width: int = 0, workspace=None, stream=None):
    k, nl = _k(k_levels)
    n_q = q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().recsa_decode(ctypes.byref(shape.c()), _p(q), n_q, _p(K), _p(V), _p(tree), n_tokens, k, nl,
                              _p(out), _p(lse), _p(sel), sel_width, _p(workspace), ws_bytes, _stream(stream)))


def recsa_decode_noalloc(shape: Shape, q, K, V, tree, n_tokens: int, k_levels, out, lse=None, sel=None,
                         sel_width: int = 0, stream=None):
    k, nl = _k(k_levels)
    _check(lib().recsa_decode_noalloc(ctypes.byref(shape.c()), _p(q), q.shape[1], _p(K), _p(V), _p(tree), n_tokens,
                                      k, nl, _p(out), _p(lse), _p(sel), sel_width, _stream(stream)))


def recsa_prefill(shape: Shape, q, q_start: int, K, V, tree, k_levels, out, lse=None, sel=None,
                  sel_width: int = 0, workspace=None, stream=None):
    k, nl = _k(k_levels)
    n_q = q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().recsa_prefill(ctypes.byref(shape.c()), _p(q), q_start, n_q, _p(K), _p(V), _p(tree), k, nl,
                               _p(out), _p(lse), _p(sel), sel_width, _p(workspace), ws_bytes, _stream(stream)))


def recsa_decode_step(shape: Shape, q, k_new, v_new, K, V, W, tree, n_tokens: int, k_levels, out, lse=None,
                      sel=None, sel_width: int = 0, workspace=None, stream=None):
    k, nl = _k(k_levels)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().recsa_decode_step(ctypes.byref(shape.c()), _p(q), _p(k_new), _p(v_new), _p(K), _p(V), _p(W),
                                   _p(tree), n_tokens, k, nl, _p(out), _p(lse), _p(sel), sel_width,
                                   _p(workspace), ws_bytes, _stream(stream)))


def recsa_backward(shape: Shape, causal: bool, q, q_start: int, n_tokens: int, K, V, W, tree, k_levels, out, lse,
                   sel, sel_width: int, dout, dq, dK, dV, dW, dlse=None, workspace=None, stream=None):
    k, nl = _k(k_levels)
    n_q = q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().recsa_backward(ctypes.byref(shape.c()), 1 if causal else 0, _p(q), q_start, n_q, n_tokens, _p(K),
                                _p(V), _p(W), _p(tree), k, nl, _p(out), _p(lse), _p(sel), sel_width, _p(dout),
                                _p(dlse), _p(dq), _p(dK), _p(dV), _p(dW), _p(workspace), ws_bytes,
                                _stream(stream)))


def recsa_distill_workspace_bytes(shape: Shape, n_tokens: int, n_q: int, k_levels) -> int:
    k, nl = _k(k_levels)
    return _nbytes(lib().recsa_distill_workspace_bytes(ctypes.byref(shape.c()), n_tokens, n_q, k, nl))


def recsa_distill_step(shape: Shape, q, K, V, n_tokens: int, k_levels, target, lr: float, W_master, W, tree, loss,
                       workspace, stream=None):
    k, nl = _k(k_levels)
    n_q = q.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().recsa_distill_step(ctypes.byref(shape.c()), _p(q), n_q, _p(K), _p(V), n_tokens, k, nl, _p(target),
                                    float(lr), _p(W_master), _p(W), _p(tree), _p(loss), _p(workspace), ws_bytes,
                                    _stream(stream)))


def recsa_dense_ref_attn(shape: Shape, q, q_start: int, K, V, n_tokens: int, mode: int, out, lse=None,
                         workspace=None, stream=None):
    n_q = q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().recsa_dense_ref_attn(ctypes.byref(shape.c()), _p(q), q_start, n_q, _p(K), _p(V), n_tokens,
                                      mode, _p(out), _p(lse), _p(workspace), ws_bytes, _stream(stream)))


def recsa_rotate_keys(shape: Shape, K, n_tokens: int, K_rot, stream=None):
    _check(lib().recsa_rotate_keys(ctypes.byref(shape.c()), _p(K), n_tokens, _p(K_rot), _stream(stream)))


def recsa_two_stage_workspace_bytes(shape: Shape, n_tokens: int, n_q: int, k_block: int, k_token: int,
                                    blocks_rotated: bool = False) -> int:
    return _nbytes(lib().recsa_two_stage_workspace_bytes(ctypes.byref(shape.c()), n_tokens, n_q, int(k_block),
                                                         int(k_token), 1 if blocks_rotated else 0))


def recsa_two_stage_decode(shape: Shape, q, K, V, tree, n_tokens: int, k_block: int, k_token: int, out, lse=None,
                           sel_blocks=None, sel_tokens=None, block_keys=None, workspace=None, stream=None):
    n_q = q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    bw = 0 if sel_blocks is None else sel_blocks.shape[-1]
    tw = 0 if sel_tokens is None else sel_tokens.shape[-1]
    _check(lib().recsa_two_stage_decode(ctypes.byref(shape.c()), _p(q), n_q, _p(K), _p(V), _p(tree), _p(block_keys),
                                        n_tokens, int(k_block), int(k_token), _p(out), _p(lse), _p(sel_blocks), bw,
                                        _p(sel_tokens), tw, _p(workspace), ws_bytes, _stream(stream)))


def recsa_two_stage_rotate_blocks(shape: Shape, tree, n_old: int, n_new: int, block_keys, stream=None):
    _check(lib().recsa_two_stage_rotate_blocks(ctypes.byref(shape.c()), _p(tree), n_old, n_new, _p(block_keys),
                                               _stream(stream)))


# ----------------------------------------------------------------- views

def tree_level_views(shape: Shape, tree: torch.Tensor, level: int):
    """(NK_l, NV_l) views [B][H_kv][rows][d] into a flat uint8 tree buffer."""
    rows = shape.capacity // shape.fanout ** level
    esz = 2 if shape.dtype == "bf16" else 4
    n = shape.batch * shape.n_kv_heads * rows * shape.head_dim
    out = []
    for which in (0, 1):
        off = recsa_level_offset(shape, level, which)
        v = tree[off:off + n * esz].view(shape.torch_dtype)
        out.append(v.view(shape.batch, shape.n_kv_heads, rows, shape.head_dim))
    return out[0], out[1]
