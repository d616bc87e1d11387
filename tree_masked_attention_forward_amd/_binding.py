"""ctypes binding of libtreeattn.so (include/tree_attn.h), same call names.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device addresses and torch's current HIP stream are passed
through, and a non-OK status raises.  Every step of the computation runs in
the library's kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libtreeattn.so")

TA_OK = 0
TA_ERR_INVALID_ARG = 1
TA_ERR_INVALID_TREE = 2
TA_ERR_UNSUPPORTED = 3
TA_ERR_WORKSPACE = 4
TA_ERR_HIP = 5
TA_F32 = 0
TA_BF16 = 1
TA_MAX_NODES = 4096
TA_MERGE_PLACEMENT = 1
TA_MERGE_TIMEOUT = 2
TA_MERGE_STALE = 4
TA_NOALLOC_MAX_WORKSPACE = 64 << 20

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class TreeAttnError(RuntimeError):
    def __init__(self, call: str, status: int, msg: str):
        super().__init__(f"{call}: {msg} (status {status})")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libtreeattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with "
                          "`python tree_masked_attention_forward_amd/build.py`")
    lib = ctypes.CDLL(p)
    lib.tree_attn_status_string.restype = ctypes.c_char_p
    lib.tree_attn_status_string.argtypes = [ctypes.c_int]
    lib.tree_attn_build_mask.restype = ctypes.c_int
    lib.tree_attn_build_mask.argtypes = [_c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p,
                                         _c_void_p, _c_void_p, _c_void_p]
    lib.tree_attn_forward_workspace_size.restype = ctypes.c_size_t
    lib.tree_attn_forward_workspace_size.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32,
                                                     _i32, _i64, _i64]
    lib.tree_attn_forward.restype = ctypes.c_int
    lib.tree_attn_forward.argtypes = [ctypes.c_int] + [_c_void_p] * 9 + [
        _i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32, ctypes.c_float, _c_void_p, _c_void_p,
        _c_void_p, ctypes.c_size_t, _c_void_p]
    lib.tree_attn_forward_noalloc.restype = ctypes.c_int
    lib.tree_attn_forward_noalloc.argtypes = [ctypes.c_int] + [_c_void_p] * 9 + [
        _i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32, ctypes.c_float, _c_void_p, _c_void_p,
        _c_void_p, _c_void_p]
    lib.tree_attn_mask_and_forward.restype = ctypes.c_int
    lib.tree_attn_mask_and_forward.argtypes = [ctypes.c_int] + [_c_void_p] * 9 + [
        _i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32, ctypes.c_float] + [_c_void_p] * 6 + [
        ctypes.c_size_t, _c_void_p]
    lib.tree_verify_greedy_workspace_size.restype = ctypes.c_size_t
    lib.tree_verify_greedy_workspace_size.argtypes = [_i32, _i32, _i32]
    lib.tree_verify_greedy.restype = ctypes.c_int
    lib.tree_verify_greedy.argtypes = [ctypes.c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _i32, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p]
    lib.tree_verify_greedy_next.restype = ctypes.c_int
    lib.tree_verify_greedy_next.argtypes = [ctypes.c_int] + [_c_void_p] * 5 + [_i32] * 4 + [
        _c_void_p] * 6 + [ctypes.c_size_t, _c_void_p]
    lib.tree_verify_sample_workspace_size.restype = ctypes.c_size_t
    lib.tree_verify_sample_workspace_size.argtypes = [_i32, _i32, _i32]
    lib.tree_verify_sample.restype = ctypes.c_int
    lib.tree_verify_sample.argtypes = [ctypes.c_int] + [_c_void_p] * 7 + [_i32] * 4 + [
        ctypes.c_float] + [_c_void_p] * 7 + [ctypes.c_size_t, _c_void_p]
    lib.tree_kv_commit.restype = ctypes.c_int
    lib.tree_kv_commit.argtypes = [ctypes.c_int] + [_c_void_p] * 5 + [_i32] * 5 + [
        _c_void_p] * 4 + [_i64, _c_void_p, _c_void_p]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().tree_attn_status_string(int(status)).decode()


def _check(call: str, status: int) -> None:
    if status != TA_OK:
        raise TreeAttnError(call, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else (t.data_ptr() or None)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, device: torch.device, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _device_of(t: torch.Tensor) -> torch.device:
    if t.device.type != "cuda":
        raise ValueError("tensors must live on a ROCm GPU device (torch 'cuda')")
    return t.device


def mask_words(max_nodes: int) -> int:
    return max(1, (max_nodes + 63) // 64)


def build_mask(parents: torch.Tensor, node_offsets: torch.Tensor, max_nodes: int, *,
               mask: Optional[torch.Tensor] = None, depth: Optional[torch.Tensor] = None,
               status: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """tree_attn_build_mask: (mask uint64 [sum_N][W], depth int32, status int32 [B])."""
    dev = _device_of(parents)
    _need(parents, "parents", torch.int32, dev, 1)
    _need(node_offsets, "node_offsets", torch.int32, dev, 1)
    B = node_offsets.numel() - 1
    total = parents.numel()
    W = mask_words(max_nodes)
    if mask is None:
        mask = torch.empty((total, W), dtype=torch.uint64, device=dev)
    if depth is None:
        depth = torch.empty(total, dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(mask, "mask", torch.uint64, dev, 2)
    if tuple(mask.shape) != (total, W):
        raise ValueError(f"mask must be [{total}, {W}]")
    _check("tree_attn_build_mask", load_library().tree_attn_build_mask(
        _ptr(parents), _ptr(node_offsets), B, total, int(max_nodes), _ptr(mask), _ptr(depth),
        _ptr(status), _stream(dev)))
    return mask, depth, status


def forward_workspace_size(dtype: torch.dtype, B: int, total_nodes: int, max_nodes: int,
                           Hq: int, Hkv: int, D: int, total_prefix: int, max_prefix: int) -> int:
    code = TA_BF16 if dtype == torch.bfloat16 else TA_F32
    return int(load_library().tree_attn_forward_workspace_size(
        code, B, total_nodes, max_nodes, Hq, Hkv, D, total_prefix, max_prefix))


def merge_status(workspace: torch.Tensor, clear: bool = False) -> int:
    """The merge status word of a forward workspace (the uint32 at byte 0; bits
    TA_MERGE_*), read after synchronising the current stream; with clear=True
    it is zeroed afterwards."""
    word = workspace.view(torch.uint8)[:4]
    torch.cuda.current_stream(workspace.device).synchronize()
    value = int.from_bytes(bytes(word.cpu().tolist()), "little")
    if clear:
        word.zero_()
    return value


def _forward_args(q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets, node_offsets,
                  max_nodes, max_prefix, out, lse, return_lse, workspace, prefix_lens):
    """Checks shared by forward() and mask_and_forward(); allocates outputs and
    the (zero-filled) workspace when they are not given."""
    dev = _device_of(q)
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    _need(q, "q", dtype, dev, 3)
    total, Hq, D = q.shape
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree), ("k_prefix", k_prefix),
                    ("v_prefix", v_prefix)):
        _need(t, name, dtype, dev, 3)
        if t.shape[2] != D:
            raise ValueError(f"{name} head size {t.shape[2]} != {D}")
    Hkv = k_tree.shape[1]
    if k_tree.shape[0] != total or v_tree.shape != k_tree.shape:
        raise ValueError("k_tree/v_tree must be [sum_N, Hkv, D]")
    if v_prefix.shape != k_prefix.shape or k_prefix.shape[1] != Hkv:
        raise ValueError("k_prefix/v_prefix must be [sum_L, Hkv, D]")
    _need(prefix_offsets, "prefix_offsets", torch.int64, dev, 1)
    _need(node_offsets, "node_offsets", torch.int32, dev, 1)
    B = node_offsets.numel() - 1
    if prefix_offsets.numel() != B + 1:
        raise ValueError("prefix_offsets and node_offsets must both hold B+1 entries")
    if prefix_lens is not None:
        _need(prefix_lens, "prefix_lens", torch.int64, dev, 1)
        if prefix_lens.numel() != B:
            raise ValueError("prefix_lens must hold B entries")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype, dev, 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if return_lse and lse is None:
        lse = torch.empty((total, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    total_prefix = k_prefix.shape[0]
    ws_bytes = forward_workspace_size(dtype, B, total, max_nodes, Hq, Hkv, D, total_prefix,
                                      max_prefix)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        # zero-filled once: the library keeps its counters at zero between calls
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = TA_BF16 if dtype == torch.bfloat16 else TA_F32
    return dict(dev=dev, code=code, B=B, total=total, Hq=Hq, Hkv=Hkv, D=D,
                total_prefix=total_prefix, out=out, lse=lse, workspace=workspace, ws_len=ws_len)


def forward(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor,
            k_prefix: torch.Tensor, v_prefix: torch.Tensor, prefix_offsets: torch.Tensor,
            node_offsets: torch.Tensor, mask: torch.Tensor, max_nodes: int, max_prefix: int,
            scale: float, *, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
            prefix_lens: Optional[torch.Tensor] = None):
    """tree_attn_forward.  Returns out (and lse when asked or given).  A
    workspace passed in must have been zero-filled before its first use.
    prefix_lens (int64 [B]) reads only the first prefix_lens[b] rows of each
    prefix range (a cache slot)."""
    a = _forward_args(q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets, node_offsets,
                      max_nodes, max_prefix, out, lse, return_lse, workspace, prefix_lens)
    _need(mask, "mask", torch.uint64, a["dev"], 2)
    if mask.shape != (a["total"], mask_words(max_nodes)):
        raise ValueError("mask must be [sum_N, ceil(max_nodes/64)]")
    _check("tree_attn_forward", load_library().tree_attn_forward(
        a["code"], _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_prefix), _ptr(v_prefix),
        _ptr(prefix_offsets), _ptr(prefix_lens), _ptr(node_offsets), _ptr(mask), a["B"],
        a["total"], int(max_nodes),
        a["total_prefix"], int(max_prefix), a["Hq"], a["Hkv"], a["D"], float(scale),
        _ptr(a["out"]), _ptr(a["lse"]), _ptr(a["workspace"]), a["ws_len"], _stream(a["dev"])))
    return (a["out"], a["lse"]) if (return_lse or lse is not None) else a["out"]


def forward_noalloc(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor,
                    k_prefix: torch.Tensor, v_prefix: torch.Tensor, prefix_offsets: torch.Tensor,
                    node_offsets: torch.Tensor, mask: torch.Tensor, max_nodes: int,
                    max_prefix: int, scale: float, *, out: torch.Tensor, lse: torch.Tensor = None,
                    merge_status: Optional[torch.Tensor] = None,
                    prefix_lens: Optional[torch.Tensor] = None):
    """tree_attn_forward_noalloc: tree_attn_forward on the library's static
    scratch (no workspace; the library allocates nothing).  `out` (and `lse`)
    must be given, so that this call allocates nothing either.  merge_status
    (uint32 [1], optional) receives the in-kernel merge's failure bits."""
    dev = _device_of(q)
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    _need(q, "q", dtype, dev, 3)
    total, Hq, D = q.shape
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree), ("k_prefix", k_prefix),
                    ("v_prefix", v_prefix), ("out", out)):
        _need(t, name, dtype, dev, 3)
    Hkv = k_tree.shape[1]
    if out.shape != q.shape or k_tree.shape != (total, Hkv, D) or v_tree.shape != k_tree.shape:
        raise ValueError("q/out [sum_N, Hq, D], k_tree/v_tree [sum_N, Hkv, D]")
    if v_prefix.shape != k_prefix.shape or tuple(k_prefix.shape[1:]) != (Hkv, D):
        raise ValueError("k_prefix/v_prefix must be [sum_L, Hkv, D]")
    _need(prefix_offsets, "prefix_offsets", torch.int64, dev, 1)
    _need(node_offsets, "node_offsets", torch.int32, dev, 1)
    _need(mask, "mask", torch.uint64, dev, 2)
    B = node_offsets.numel() - 1
    if prefix_offsets.numel() != B + 1 or mask.shape != (total, mask_words(max_nodes)):
        raise ValueError("offsets hold B+1 entries; mask is [sum_N, ceil(max_nodes/64)]")
    if prefix_lens is not None:
        _need(prefix_lens, "prefix_lens", torch.int64, dev, 1)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    if merge_status is not None:
        _need(merge_status, "merge_status", torch.int32, dev, 1)
    code = TA_BF16 if dtype == torch.bfloat16 else TA_F32
    _check("tree_attn_forward_noalloc", load_library().tree_attn_forward_noalloc(
        code, _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_prefix), _ptr(v_prefix),
        _ptr(prefix_offsets), _ptr(prefix_lens), _ptr(node_offsets), _ptr(mask), B, total,
        int(max_nodes), k_prefix.shape[0], int(max_prefix), Hq, Hkv, D, float(scale), _ptr(out),
        _ptr(lse), _ptr(merge_status), _stream(dev)))
    return out


def mask_and_forward(parents: torch.Tensor, q: torch.Tensor, k_tree: torch.Tensor,
                     v_tree: torch.Tensor, k_prefix: torch.Tensor, v_prefix: torch.Tensor,
                     prefix_offsets: torch.Tensor, node_offsets: torch.Tensor, max_nodes: int,
                     max_prefix: int, scale: float, *, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, return_lse: bool = False,
                     mask: Optional[torch.Tensor] = None, depth: Optional[torch.Tensor] = None,
                     status: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     prefix_lens: Optional[torch.Tensor] = None):
    """tree_attn_mask_and_forward: the ancestor mask and the attention in one
    call.  Returns (out, [lse,] mask, depth, status)."""
    a = _forward_args(q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets, node_offsets,
                      max_nodes, max_prefix, out, lse, return_lse, workspace, prefix_lens)
    dev, total, B = a["dev"], a["total"], a["B"]
    _need(parents, "parents", torch.int32, dev, 1)
    if parents.numel() != total:
        raise ValueError("parents must hold one entry per tree node")
    W = mask_words(max_nodes)
    if mask is None:
        mask = torch.empty((total, W), dtype=torch.uint64, device=dev)
    if depth is None:
        depth = torch.empty(total, dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(mask, "mask", torch.uint64, dev, 2)
    if tuple(mask.shape) != (total, W):
        raise ValueError(f"mask must be [{total}, {W}]")
    _check("tree_attn_mask_and_forward", load_library().tree_attn_mask_and_forward(
        a["code"], _ptr(parents), _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_prefix),
        _ptr(v_prefix), _ptr(prefix_offsets), _ptr(prefix_lens), _ptr(node_offsets), B, total,
        int(max_nodes),
        a["total_prefix"], int(max_prefix), a["Hq"], a["Hkv"], a["D"], float(scale), _ptr(mask),
        _ptr(depth), _ptr(status), _ptr(a["out"]), _ptr(a["lse"]), _ptr(a["workspace"]),
        a["ws_len"], _stream(dev)))
    head = (a["out"], a["lse"]) if (return_lse or lse is not None) else (a["out"],)
    return head + (mask, depth, status)


def verify_workspace_size(total_nodes: int, max_nodes: int, V: int) -> int:
    return int(load_library().tree_verify_greedy_workspace_size(total_nodes, max_nodes, V))


def verify_greedy(logits: torch.Tensor, draft_tokens: torch.Tensor, mask: torch.Tensor,
                  node_offsets: torch.Tensor, max_nodes: int, *,
                  workspace: Optional[torch.Tensor] = None, target_argmax: Optional[torch.Tensor] = None,
                  accept_len: Optional[torch.Tensor] = None,
                  accept_nodes: Optional[torch.Tensor] = None,
                  accept_tokens: Optional[torch.Tensor] = None):
    """tree_verify_greedy: (target_argmax, accept_len, accept_nodes, accept_tokens)."""
    dev = _device_of(logits)
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be bfloat16 or float32")
    _need(logits, "logits", logits.dtype, dev, 2)
    total, V = logits.shape
    _need(draft_tokens, "draft_tokens", torch.int32, dev, 1)
    _need(mask, "mask", torch.uint64, dev, 2)
    _need(node_offsets, "node_offsets", torch.int32, dev, 1)
    if draft_tokens.numel() != total or mask.shape != (total, mask_words(max_nodes)):
        raise ValueError("draft_tokens/mask do not match the logits rows")
    B = node_offsets.numel() - 1
    if target_argmax is None:
        target_argmax = torch.empty(total, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if accept_nodes is None:
        accept_nodes = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    if accept_tokens is None:
        accept_tokens = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    ws_bytes = verify_workspace_size(total, max_nodes, V)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = TA_BF16 if logits.dtype == torch.bfloat16 else TA_F32
    _check("tree_verify_greedy", load_library().tree_verify_greedy(
        code, _ptr(logits), _ptr(draft_tokens), _ptr(mask), _ptr(node_offsets), B, total,
        int(max_nodes), V, _ptr(target_argmax), _ptr(accept_len), _ptr(accept_nodes),
        _ptr(accept_tokens), _ptr(workspace), ws_len, _stream(dev)))
    return target_argmax, accept_len, accept_nodes, accept_tokens


def verify_greedy_next(logits: torch.Tensor, root_logits: torch.Tensor,
                       draft_tokens: torch.Tensor, mask: torch.Tensor,
                       node_offsets: torch.Tensor, max_nodes: int, *,
                       workspace: Optional[torch.Tensor] = None,
                       target_argmax: Optional[torch.Tensor] = None,
                       accept_len: Optional[torch.Tensor] = None,
                       accept_nodes: Optional[torch.Tensor] = None,
                       accept_tokens: Optional[torch.Tensor] = None,
                       bonus_token: Optional[torch.Tensor] = None):
    """tree_verify_greedy_next (row i: the token after node i; root_logits row
    b: the token after sequence b's prefix).  Returns (target_argmax,
    accept_len, accept_nodes, accept_tokens, bonus_token)."""
    dev = _device_of(logits)
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be bfloat16 or float32")
    _need(logits, "logits", logits.dtype, dev, 2)
    _need(root_logits, "root_logits", logits.dtype, dev, 2)
    total, V = logits.shape
    _need(draft_tokens, "draft_tokens", torch.int32, dev, 1)
    _need(mask, "mask", torch.uint64, dev, 2)
    _need(node_offsets, "node_offsets", torch.int32, dev, 1)
    B = node_offsets.numel() - 1
    if tuple(root_logits.shape) != (B, V):
        raise ValueError("root_logits must be [B, V]")
    if draft_tokens.numel() != total or mask.shape != (total, mask_words(max_nodes)):
        raise ValueError("draft_tokens/mask do not match the logits rows")
    if target_argmax is None:
        target_argmax = torch.empty(total, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if accept_nodes is None:
        accept_nodes = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    if accept_tokens is None:
        accept_tokens = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    if bonus_token is None:
        bonus_token = torch.empty(B, dtype=torch.int32, device=dev)
    ws_bytes = verify_workspace_size(total + B, max_nodes, V)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    code = TA_BF16 if logits.dtype == torch.bfloat16 else TA_F32
    _check("tree_verify_greedy_next", load_library().tree_verify_greedy_next(
        code, _ptr(logits), _ptr(root_logits), _ptr(draft_tokens), _ptr(mask), _ptr(node_offsets),
        B, total, int(max_nodes), V, _ptr(target_argmax), _ptr(accept_len), _ptr(accept_nodes),
        _ptr(accept_tokens), _ptr(bonus_token), _ptr(workspace), ws_len, _stream(dev)))
    return target_argmax, accept_len, accept_nodes, accept_tokens, bonus_token


def verify_sample_workspace_size(B: int, total_nodes: int, V: int) -> int:
    return int(load_library().tree_verify_sample_workspace_size(B, total_nodes, V))


def verify_sample(logits: torch.Tensor, root_logits: torch.Tensor, draft_probs: torch.Tensor,
                  root_draft_probs: torch.Tensor, draft_tokens: torch.Tensor,
                  parents: torch.Tensor, node_offsets: torch.Tensor, max_nodes: int,
                  temperature: float, u_accept: torch.Tensor, u_final: torch.Tensor, *,
                  workspace: Optional[torch.Tensor] = None,
                  accept_len: Optional[torch.Tensor] = None,
                  accept_nodes: Optional[torch.Tensor] = None,
                  accept_tokens: Optional[torch.Tensor] = None,
                  bonus_token: Optional[torch.Tensor] = None):
    """tree_verify_sample (rejection sampling down the tree; the random numbers
    are inputs).  Returns (accept_len, accept_nodes, accept_tokens,
    bonus_token)."""
    dev = _device_of(logits)
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be bfloat16 or float32")
    _need(logits, "logits", logits.dtype, dev, 2)
    _need(root_logits, "root_logits", logits.dtype, dev, 2)
    total, V = logits.shape
    _need(draft_probs, "draft_probs", torch.float32, dev, 2)
    _need(root_draft_probs, "root_draft_probs", torch.float32, dev, 2)
    _need(draft_tokens, "draft_tokens", torch.int32, dev, 1)
    _need(parents, "parents", torch.int32, dev, 1)
    _need(node_offsets, "node_offsets", torch.int32, dev, 1)
    _need(u_accept, "u_accept", torch.float32, dev, 1)
    _need(u_final, "u_final", torch.float32, dev, 1)
    B = node_offsets.numel() - 1
    if tuple(root_logits.shape) != (B, V) or tuple(root_draft_probs.shape) != (B, V):
        raise ValueError("root_logits and root_draft_probs must be [B, V]")
    if tuple(draft_probs.shape) != (total, V):
        raise ValueError("draft_probs must match the logits rows")
    if draft_tokens.numel() != total or parents.numel() != total or u_accept.numel() != total:
        raise ValueError("draft_tokens/parents/u_accept must have one entry per node")
    if u_final.numel() != B:
        raise ValueError("u_final must have one entry per sequence")
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if accept_nodes is None:
        accept_nodes = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    if accept_tokens is None:
        accept_tokens = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    if bonus_token is None:
        bonus_token = torch.empty(B, dtype=torch.int32, device=dev)
    ws_bytes = verify_sample_workspace_size(B, total, V)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    code = TA_BF16 if logits.dtype == torch.bfloat16 else TA_F32
    _check("tree_verify_sample", load_library().tree_verify_sample(
        code, _ptr(logits), _ptr(root_logits), _ptr(draft_probs), _ptr(root_draft_probs),
        _ptr(draft_tokens), _ptr(parents), _ptr(node_offsets), B, total, int(max_nodes), V,
        float(temperature), _ptr(u_accept), _ptr(u_final), _ptr(accept_len), _ptr(accept_nodes),
        _ptr(accept_tokens), _ptr(bonus_token), _ptr(workspace), ws_len, _stream(dev)))
    return accept_len, accept_nodes, accept_tokens, bonus_token


def kv_commit(k_tree: torch.Tensor, v_tree: torch.Tensor, node_offsets: torch.Tensor,
              accept_len: torch.Tensor, accept_nodes: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, cache_offsets: torch.Tensor, cache_lens: torch.Tensor, *,
              status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """tree_kv_commit: append each sequence's accepted path to its cache slot
    (k_cache/v_cache and cache_lens are updated in place).  Returns the
    per-sequence status."""
    dev = _device_of(k_tree)
    dtype = k_tree.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("k_tree must be bfloat16 or float32")
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _need(t, name, dtype, dev, 3)
    total, Hkv, D = k_tree.shape
    if v_tree.shape != k_tree.shape:
        raise ValueError("v_tree must have k_tree's shape")
    if v_cache.shape != k_cache.shape or tuple(k_cache.shape[1:]) != (Hkv, D):
        raise ValueError("k_cache/v_cache must be [total_cache, Hkv, D]")
    _need(node_offsets, "node_offsets", torch.int32, dev, 1)
    _need(accept_len, "accept_len", torch.int32, dev, 1)
    _need(accept_nodes, "accept_nodes", torch.int32, dev, 2)
    _need(cache_offsets, "cache_offsets", torch.int64, dev, 1)
    _need(cache_lens, "cache_lens", torch.int64, dev, 1)
    B = node_offsets.numel() - 1
    max_nodes = accept_nodes.shape[1]
    if accept_len.numel() != B or accept_nodes.shape[0] != B or cache_lens.numel() != B:
        raise ValueError("accept_len, accept_nodes and cache_lens must have B rows")
    if cache_offsets.numel() != B + 1:
        raise ValueError("cache_offsets must hold B+1 entries")
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(status, "status", torch.int32, dev, 1)
    code = TA_BF16 if dtype == torch.bfloat16 else TA_F32
    _check("tree_kv_commit", load_library().tree_kv_commit(
        code, _ptr(k_tree), _ptr(v_tree), _ptr(node_offsets), _ptr(accept_len),
        _ptr(accept_nodes), B, total, int(max_nodes), Hkv, D, _ptr(k_cache), _ptr(v_cache),
        _ptr(cache_offsets), _ptr(cache_lens), k_cache.shape[0], _ptr(status), _stream(dev)))
    return status
