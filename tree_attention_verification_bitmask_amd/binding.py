"""Thin ctypes binding of libtreeverify (include/treeverify.h).

Each function has the C entry point's name and only marshals arguments:
torch tensors -> device pointers, the current HIP stream -> hipStream_t, and
a non-zero tv_status -> TreeVerifyError.  Output tensors are allocated with
torch when not passed in.  Every step of the pass runs in the HIP library;
there is no fallback: if libtreeverify.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtreeverify.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "treeverify.h")

TV_F32, TV_BF16 = 0, 1
TV_MAX_NODES, TV_MAX_DEPTH, TV_MAX_LEDGER, TV_MAX_VOCAB = 1024, 64, 8192, 16777216
DEVERR_BAD_PARENT, DEVERR_TOO_DEEP, DEVERR_BAD_REQUEST, DEVERR_BAD_PATH, DEVERR_BAD_LEDGER = 1, 2, 3, 4, 5
DEVERR_LIMIT = 6
DEVERR_BAD_SLOT = 7
DEVERR_BAD_TOKEN = 8
TV_GDN_HEAD_DIM, TV_GDN_MAX_NODES, TV_GDN_MAX_TABLE = 128, 256, 4096


class TreeVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """Load libtreeverify.so (once) and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m tree_attention_verification_bitmask_amd.build`")
    L = C.CDLL(LIB_PATH)
    i32, i64, f32, sz, vp = C.c_int32, C.c_int64, C.c_float, C.c_size_t, C.c_void_p
    L.tv_status_string.argtypes = [C.c_int]
    L.tv_status_string.restype = C.c_char_p
    L.tv_abi_version.argtypes = []
    L.tv_abi_version.restype = C.c_int
    L.tree_mask_build.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.tree_mask_build.restype = C.c_int
    L.tree_attn_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, C.c_int]
    L.tree_attn_verify_workspace_size.restype = sz
    L.tree_attn_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, i32, i32,
                                   f32, C.c_int, vp, vp, sz, vp, vp]
    L.tree_attn_verify.restype = C.c_int
    L.tree_attn_verify_workspace_size_ex.argtypes = [i32, i32, i32, i32, i32, i32, i32, C.c_int, vp, vp]
    L.tree_attn_verify_workspace_size_ex.restype = sz
    L.tree_attn_verify_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, i32, i32,
                                      f32, C.c_int, vp, vp, vp, sz, vp, vp, vp]
    L.tree_attn_verify_ex.restype = C.c_int
    L.tree_attn_verify_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, C.c_int, vp, vp]
    L.tree_attn_verify_plan.restype = C.c_int
    L.tree_attn_verify_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, i32, i32,
                                           f32, C.c_int, vp, vp, vp]
    L.tree_attn_verify_noalloc.restype = C.c_int
    L.tree_accept_greedy.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.tree_accept_greedy.restype = C.c_int
    L.kv_compact_path.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, C.c_int,
                                  vp, vp, vp]
    L.kv_compact_path.restype = C.c_int
    L.tree_accept_commit.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, C.c_int,
                                     vp, vp, vp, vp, vp, vp, vp, vp]
    L.tree_accept_commit.restype = C.c_int
    L.tree_select_topb.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp]
    L.tree_select_topb.restype = C.c_int
    L.tree_target_argmax.argtypes = [vp, i32, i32, C.c_int, vp, vp]
    L.tree_target_argmax.restype = C.c_int
    L.tree_target_sample_workspace_size.argtypes = [i32, i32]
    L.tree_target_sample_workspace_size.restype = sz
    L.tree_target_sample.argtypes = [vp, i32, i32, C.c_int, f32, vp, vp, vp, sz, vp]
    L.tree_target_sample.restype = C.c_int
    L.tree_accept_stochastic_workspace_size.argtypes = [i32, i32, i32]
    L.tree_accept_stochastic_workspace_size.restype = sz
    L.tree_accept_stochastic.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, C.c_int, f32, vp, vp, i32, vp, vp,
                                         vp, vp, vp, vp, sz, vp, vp]
    L.tree_accept_stochastic.restype = C.c_int
    L.tree_rope_apply.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, C.c_int, vp, vp]
    L.tree_rope_apply.restype = C.c_int
    L.kv_rollback_token_table.argtypes = [vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.kv_rollback_token_table.restype = C.c_int
    L.tree_gdn_conv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    L.tree_gdn_conv.restype = C.c_int
    L.tree_gdn_verify.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                  vp, vp, vp]
    L.tree_gdn_verify.restype = C.c_int
    L.tree_gdn_commit.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                  i32, i32, vp, vp]
    L.tree_gdn_commit.restype = C.c_int
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/treeverify.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)


def _check(fn: str, status: int):
    if status != 0:
        raise TreeVerifyError(fn, status, lib().tv_status_string(status).decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return TV_F32
    if t.dtype == torch.bfloat16:
        return TV_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need(t, name, dtype=None, numel=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def tree_mask_build(parent, cu_nodes, prefix_len, max_nodes: int, max_depth: int,
                    anc=None, level=None, pos=None, err=None, stream=None):
    """-> (anc uint64-as-int64 [T, W], level int32 [T], pos int32 [T], err int32 [1])."""
    import torch
    B = cu_nodes.numel() - 1
    T = parent.numel()
    W = (max_nodes + 63) // 64
    dev = parent.device
    for t, n in ((parent, "parent"), (cu_nodes, "cu_nodes"), (prefix_len, "prefix_len")):
        _need(t, n, torch.int32)
    anc = torch.empty((T, W), dtype=torch.int64, device=dev) if anc is None else anc
    level = torch.empty(T, dtype=torch.int32, device=dev) if level is None else level
    pos = torch.empty(T, dtype=torch.int32, device=dev) if pos is None else pos
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    _need(anc, "anc", torch.int64, T * W)
    _need(level, "level", torch.int32, T)
    _need(pos, "pos", torch.int32, T)
    _check("tree_mask_build", lib().tree_mask_build(
        _ptr(parent), _ptr(cu_nodes), _ptr(prefix_len), B, T, max_nodes, max_depth,
        _ptr(anc), _ptr(level), _ptr(pos), _ptr(err), _stream(stream)))
    return anc, level, pos, err


TV_ORDER_AUTO, TV_ORDER_STATIC, TV_ORDER_PLANNED, TV_ORDER_BALANCED = 0, 1, 2, 3


class PlanOverride(C.Structure):
    """tv_attn_plan_override: key-axis slices (0 = the library's choice) and
    the batch task order (TV_ORDER_*)."""
    _fields_ = [("splits", C.c_int32), ("order", C.c_int32), ("waves", C.c_int32), ("reserved", C.c_int32 * 5)]


def _override(splits: int = 0, order: int = TV_ORDER_AUTO, waves: int = 0):
    if not splits and order == TV_ORDER_AUTO and not waves:
        return None
    return PlanOverride(int(splits), int(order), int(waves))


class AttnInputs(C.Structure):
    """tv_attn_inputs: RoPE inside the call (rope_base > 0, positions pos_ids)
    and K/V rows through a token table (req_to_token [B, table_stride])."""
    _fields_ = [("pos_ids", C.c_void_p), ("req_to_token", C.c_void_p), ("table_stride", C.c_int64),
                ("rope_base", C.c_float), ("reserved", C.c_int32 * 5)]


def _inputs(pos_ids=None, rope_base: float = 0.0, req_to_token=None):
    if not rope_base and req_to_token is None:
        return None
    stride = 0 if req_to_token is None else int(req_to_token.shape[-1])
    addr = lambda t: None if t is None else int(t.data_ptr())
    return AttnInputs(addr(pos_ids) if rope_base else None, addr(req_to_token), stride, float(rope_base))


def tree_attn_verify_workspace_size(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim,
                                    dtype_code, splits: int = 0, order: int = TV_ORDER_AUTO,
                                    waves: int = 0, inputs=None) -> int:
    ov = _override(splits, order, waves)
    if ov is None and inputs is None:
        return int(lib().tree_attn_verify_workspace_size(batch, total_nodes, max_nodes, max_prefix, hq,
                                                         hkv, head_dim, dtype_code))
    return int(lib().tree_attn_verify_workspace_size_ex(
        batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype_code,
        C.byref(inputs) if inputs is not None else None, C.byref(ov) if ov is not None else None))


PLAN_FIELDS = ("mfma", "rows_per_tile", "row_tiles", "splits", "keys_per_split", "planned", "lookahead",
               "workspace_bytes")


def tree_attn_verify_plan(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype_code,
                          splits: int = 0, order: int = TV_ORDER_AUTO, waves: int = 0) -> dict:
    """The plan tree_attn_verify would run for these host sizes (no GPU needed)."""
    ov = _override(splits, order, waves)
    info = (C.c_int32 * 8)()
    _check("tree_attn_verify_plan", lib().tree_attn_verify_plan(
        batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype_code,
        C.byref(ov) if ov is not None else None, info))
    return dict(zip(PLAN_FIELDS, (int(x) for x in info)))


def tree_attn_verify(q, k_cache, v_cache, cu_nodes, kv_start, prefix_len, anc, max_nodes: int,
                     max_prefix: int, scale: float | None = None, out=None, workspace=None,
                     err=None, stream=None, splits: int = 0, order: int = TV_ORDER_AUTO, waves: int = 0,
                     pos_ids=None, rope_base: float = 0.0, req_to_token=None):
    """q [T, hq, d]; k_cache / v_cache [rows, hkv, d] -> out [T, hq, d] (same dtype).
    splits / order / waves: a plan override, for tuning and tests; pos_ids and
    rope_base > 0: RoPE inside the call (the tree's K rows of k_cache are
    rotated in place); req_to_token [B, stride] int32: K/V rows through a token
    table (kv_start may then be None).  Any of these goes through
    tree_attn_verify_ex."""
    import torch
    T, hq, d = q.shape
    rows, hkv, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_cache / v_cache shapes disagree")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    code = _dtype_code(q)
    B = cu_nodes.numel() - 1
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n)
    for t, n in ((cu_nodes, "cu_nodes"), (kv_start, "kv_start"), (prefix_len, "prefix_len")):
        if t is not None or n != "kv_start" or req_to_token is None:
            _need(t, n, torch.int32)
    if req_to_token is not None:
        _need(req_to_token, "req_to_token", torch.int32, B * int(req_to_token.shape[-1]))
    if rope_base:
        _need(pos_ids, "pos_ids", torch.int32, T)
    _need(anc, "anc", torch.int64, T * ((max_nodes + 63) // 64))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", q.dtype, q.numel())
    err = torch.zeros(1, dtype=torch.int32, device=q.device) if err is None else err
    inputs = _inputs(pos_ids, rope_base, req_to_token)
    ws_bytes = tree_attn_verify_workspace_size(B, T, max_nodes, max_prefix, hq, hkv, d, code, splits, order, waves,
                                               inputs)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = d ** -0.5
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_nodes), _ptr(kv_start), _ptr(prefix_len),
            _ptr(anc), B, T, max_nodes, max_prefix, rows, hq, hkv, d, float(scale), code)
    tail = (_ptr(out), _ptr(workspace), ws_have, _ptr(err))
    ov = _override(splits, order, waves)
    if ov is None and inputs is None:
        _check("tree_attn_verify", lib().tree_attn_verify(*head, *tail, _stream(stream)))
    else:
        _check("tree_attn_verify_ex", lib().tree_attn_verify_ex(
            *head, C.byref(inputs) if inputs is not None else None, *tail,
            C.byref(ov) if ov is not None else None, _stream(stream)))
    return out


TV_NOALLOC_SCRATCH_BYTES = 80 << 20


def tree_attn_verify_noalloc(q, k_cache, v_cache, cu_nodes, kv_start, prefix_len, anc, max_nodes: int,
                             max_prefix: int, scale: float | None = None, out=None, err=None, stream=None):
    """tree_attn_verify with no workspace: the library's static per-GPU scratch
    buffer holds the split partials (calls on one GPU must not overlap)."""
    import torch
    T, hq, d = q.shape
    rows, hkv, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_cache / v_cache shapes disagree")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    code = _dtype_code(q)
    B = cu_nodes.numel() - 1
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n)
    for t, n in ((cu_nodes, "cu_nodes"), (kv_start, "kv_start"), (prefix_len, "prefix_len")):
        _need(t, n, torch.int32)
    _need(anc, "anc", torch.int64, T * ((max_nodes + 63) // 64))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", q.dtype, q.numel())
    err = torch.zeros(1, dtype=torch.int32, device=q.device) if err is None else err
    if scale is None:
        scale = d ** -0.5
    _check("tree_attn_verify_noalloc", lib().tree_attn_verify_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_nodes), _ptr(kv_start), _ptr(prefix_len),
        _ptr(anc), B, T, max_nodes, max_prefix, rows, hq, hkv, d, float(scale), code, _ptr(out),
        _ptr(err), _stream(stream)))
    return out


def tree_accept_greedy(parent, draft_tokens, target_tokens, root_target, cu_nodes, max_depth: int,
                       accept_len=None, accept_idx=None, next_token=None, err=None, stream=None):
    """-> (accept_len int32 [B], accept_idx int32 [B, max_depth], next_token int32 [B], err)."""
    import torch
    B = cu_nodes.numel() - 1
    T = parent.numel()
    dev = parent.device
    for t, n in ((parent, "parent"), (draft_tokens, "draft_tokens"), (target_tokens, "target_tokens"),
                 (root_target, "root_target"), (cu_nodes, "cu_nodes")):
        _need(t, n, torch.int32)
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    accept_idx = (torch.empty((B, max_depth), dtype=torch.int32, device=dev)
                  if accept_idx is None else accept_idx)
    next_token = torch.empty(B, dtype=torch.int32, device=dev) if next_token is None else next_token
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    _need(accept_idx, "accept_idx", torch.int32, B * max_depth)
    _check("tree_accept_greedy", lib().tree_accept_greedy(
        _ptr(parent), _ptr(draft_tokens), _ptr(target_tokens), _ptr(root_target), _ptr(cu_nodes),
        B, T, max_depth, _ptr(accept_len), _ptr(accept_idx), _ptr(next_token), _ptr(err),
        _stream(stream)))
    return accept_len, accept_idx, next_token, err


def kv_compact_path(k_cache, v_cache, cu_nodes, kv_start, prefix_len, accept_len, accept_idx,
                    max_depth: int, total_nodes: int, new_kv_len=None, err=None, stream=None):
    """Gathers the accepted rows in place; -> (new_kv_len int32 [B], err)."""
    import torch
    rows, hkv, d = k_cache.shape
    code = _dtype_code(k_cache)
    B = cu_nodes.numel() - 1
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.numel())
    for t, n in ((cu_nodes, "cu_nodes"), (kv_start, "kv_start"), (prefix_len, "prefix_len"),
                 (accept_len, "accept_len"), (accept_idx, "accept_idx")):
        _need(t, n, torch.int32)
    new_kv_len = torch.empty(B, dtype=torch.int32, device=k_cache.device) if new_kv_len is None else new_kv_len
    err = torch.zeros(1, dtype=torch.int32, device=k_cache.device) if err is None else err
    _check("kv_compact_path", lib().kv_compact_path(
        _ptr(k_cache), _ptr(v_cache), _ptr(cu_nodes), _ptr(kv_start), _ptr(prefix_len),
        _ptr(accept_len), _ptr(accept_idx), B, total_nodes, max_depth, rows, hkv, d, code,
        _ptr(new_kv_len), _ptr(err), _stream(stream)))
    return new_kv_len, err


def tree_accept_commit(parent, draft_tokens, target_tokens, root_target, cu_nodes, kv_start, prefix_len,
                       k_cache, v_cache, max_depth: int, accept_len=None, accept_idx=None, next_token=None,
                       new_kv_len=None, err=None, stream=None):
    """tree_accept_greedy then kv_compact_path in one launch; gathers the
    accepted rows in place; -> (accept_len, accept_idx, next_token, new_kv_len, err)."""
    import torch
    rows, hkv, d = k_cache.shape
    code = _dtype_code(k_cache)
    B = cu_nodes.numel() - 1
    T = parent.numel()
    dev = k_cache.device
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.numel())
    for t, n in ((parent, "parent"), (draft_tokens, "draft_tokens"), (target_tokens, "target_tokens"),
                 (root_target, "root_target"), (cu_nodes, "cu_nodes"), (kv_start, "kv_start"),
                 (prefix_len, "prefix_len")):
        _need(t, n, torch.int32)
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    accept_idx = (torch.empty((B, max_depth), dtype=torch.int32, device=dev)
                  if accept_idx is None else accept_idx)
    next_token = torch.empty(B, dtype=torch.int32, device=dev) if next_token is None else next_token
    new_kv_len = torch.empty(B, dtype=torch.int32, device=dev) if new_kv_len is None else new_kv_len
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    _need(accept_idx, "accept_idx", torch.int32, B * max_depth)
    _check("tree_accept_commit", lib().tree_accept_commit(
        _ptr(parent), _ptr(draft_tokens), _ptr(target_tokens), _ptr(root_target), _ptr(cu_nodes),
        _ptr(kv_start), _ptr(prefix_len), B, T, max_depth, rows, hkv, d, code, _ptr(k_cache),
        _ptr(v_cache), _ptr(accept_len), _ptr(accept_idx), _ptr(next_token), _ptr(new_kv_len),
        _ptr(err), _stream(stream)))
    return accept_len, accept_idx, next_token, new_kv_len, err


def tree_select_topb(score, parent, token, budget: int, beta: float = 0.0, tree_parent=None,
                     tree_token=None, n_real=None, err=None, stream=None):
    """score float32 / parent int32 / token int32 [B, D, L] -> (tree_parent int32
    [B, budget], tree_token int32 [B, budget], n_real int32 [B], err)."""
    import torch
    if score.dim() != 3 or tuple(parent.shape) != tuple(score.shape) or tuple(token.shape) != tuple(score.shape):
        raise ValueError("score, parent and token must share one [batch, depth, lanes] shape")
    B, D, L = score.shape
    dev = score.device
    _need(score, "score", torch.float32)
    _need(parent, "parent", torch.int32)
    _need(token, "token", torch.int32)
    tree_parent = torch.empty((B, budget), dtype=torch.int32, device=dev) if tree_parent is None else tree_parent
    tree_token = torch.empty((B, budget), dtype=torch.int32, device=dev) if tree_token is None else tree_token
    n_real = torch.empty(B, dtype=torch.int32, device=dev) if n_real is None else n_real
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    _need(tree_parent, "tree_parent", torch.int32, B * budget)
    _need(tree_token, "tree_token", torch.int32, B * budget)
    _need(n_real, "n_real", torch.int32, B)
    _check("tree_select_topb", lib().tree_select_topb(
        _ptr(score), _ptr(parent), _ptr(token), B, D, L, budget, float(beta), _ptr(tree_parent),
        _ptr(tree_token), _ptr(n_real), _ptr(err), _stream(stream)))
    return tree_parent, tree_token, n_real, err


def tree_target_argmax(logits, token=None, stream=None):
    """logits [rows, vocab] (float32 or bfloat16) -> token int32 [rows]: the
    lowest index of each row's maximum (NaN ranks highest)."""
    import torch
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, vocab]")
    rows, vocab = logits.shape
    code = _dtype_code(logits)
    _need(logits, "logits")
    token = torch.empty(rows, dtype=torch.int32, device=logits.device) if token is None else token
    _need(token, "token", torch.int32, rows)
    _check("tree_target_argmax", lib().tree_target_argmax(_ptr(logits), rows, vocab, code, _ptr(token),
                                                          _stream(stream)))
    return token


def tree_target_sample_workspace_size(rows: int, vocab: int) -> int:
    return int(lib().tree_target_sample_workspace_size(rows, vocab))


def tree_target_sample(logits, temperature: float, u, token=None, workspace=None, stream=None):
    """logits [rows, vocab] (float32 or bfloat16), u [rows] float64 uniforms
    -> token int32 [rows]: the inverse-transform sample of
    softmax(logits / temperature) at u."""
    import torch
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, vocab]")
    rows, vocab = logits.shape
    code = _dtype_code(logits)
    _need(logits, "logits")
    _need(u, "u", torch.float64, rows)
    token = torch.empty(rows, dtype=torch.int32, device=logits.device) if token is None else token
    _need(token, "token", torch.int32, rows)
    ws_bytes = tree_target_sample_workspace_size(rows, vocab)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=logits.device)
    _check("tree_target_sample", lib().tree_target_sample(
        _ptr(logits), rows, vocab, code, float(temperature), _ptr(u), _ptr(token), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return token


def tree_accept_stochastic(parent, draft_tokens, cu_nodes, root_logits, node_logits, temperature: float, root_q,
                           node_q, u_accept, u_final, max_depth: int, err=None, workspace=None, stream=None):
    """The stochastic tree walk: root_logits [B, V] / node_logits [T, V]
    (float32 or bfloat16), root_q [B, V] / node_q [T, V] float32 draft
    probabilities, u_accept [T] / u_final [B] float64 uniforms ->
    (accept_len [B], accept_idx [B, max_depth], next_token [B], err)."""
    import torch
    B, V = root_logits.shape
    T = int(parent.numel())
    code = _dtype_code(root_logits)
    dev = root_logits.device
    for t, n in ((parent, "parent"), (draft_tokens, "draft_tokens"), (cu_nodes, "cu_nodes")):
        _need(t, n, torch.int32)
    _need(root_logits, "root_logits", None, B * V)
    _need(node_logits, "node_logits", root_logits.dtype, T * V)
    _need(root_q, "root_q", torch.float32, B * V)
    _need(node_q, "node_q", torch.float32, T * V)
    _need(u_accept, "u_accept", torch.float64, T)
    _need(u_final, "u_final", torch.float64, B)
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    aidx = torch.empty((B, max_depth), dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    ws_bytes = int(lib().tree_accept_stochastic_workspace_size(B, T, V))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check("tree_accept_stochastic", lib().tree_accept_stochastic(
        _ptr(parent), _ptr(draft_tokens), _ptr(cu_nodes), B, T, max_depth, _ptr(root_logits), _ptr(node_logits),
        code, float(temperature), _ptr(root_q), _ptr(node_q), V, _ptr(u_accept), _ptr(u_final), _ptr(alen),
        _ptr(aidx), _ptr(nxt), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(err),
        _stream(stream)))
    return alen, aidx, nxt, err


def tree_rope_apply(q, k_cache, pos_ids, cu_nodes, kv_start, prefix_len, base: float = 1.0e6, err=None,
                    stream=None):
    """Rotates q [T, hq, d] and the tree's K rows of k_cache [rows, hkv, d] in
    place by pos_ids [T]; -> err."""
    import torch
    T, hq, d = q.shape
    rows, hkv, d2 = k_cache.shape
    if d2 != d or k_cache.dtype != q.dtype:
        raise ValueError("q and k_cache disagree in head_dim or dtype")
    code = _dtype_code(q)
    B = cu_nodes.numel() - 1
    _need(q, "q")
    _need(k_cache, "k_cache")
    for t, n in ((cu_nodes, "cu_nodes"), (kv_start, "kv_start"), (prefix_len, "prefix_len")):
        _need(t, n, torch.int32)
    _need(pos_ids, "pos_ids", torch.int32, T)
    err = torch.zeros(1, dtype=torch.int32, device=q.device) if err is None else err
    _check("tree_rope_apply", lib().tree_rope_apply(
        _ptr(q), _ptr(k_cache), _ptr(pos_ids), _ptr(cu_nodes), _ptr(kv_start), _ptr(prefix_len), B, T, rows,
        hq, hkv, d, float(base), code, _ptr(err), _stream(stream)))
    return err


def kv_rollback_token_table(req_to_token, tree_slots, cu_nodes, prefix_len, accept_len, accept_idx,
                            max_depth: int, total_nodes: int, new_len=None, freed_slots=None, n_freed=None,
                            err=None, stream=None):
    """Updates req_to_token [B, stride] in place; -> (new_len [B],
    freed_slots [T], n_freed [B], err)."""
    import torch
    B, stride = req_to_token.shape
    dev = req_to_token.device
    for t, n in ((req_to_token, "req_to_token"), (cu_nodes, "cu_nodes"), (prefix_len, "prefix_len"),
                 (accept_len, "accept_len"), (accept_idx, "accept_idx"), (tree_slots, "tree_slots")):
        _need(t, n, torch.int32)
    new_len = torch.empty(B, dtype=torch.int32, device=dev) if new_len is None else new_len
    freed_slots = (torch.empty(max(total_nodes, 1), dtype=torch.int32, device=dev)
                   if freed_slots is None else freed_slots)
    n_freed = torch.empty(B, dtype=torch.int32, device=dev) if n_freed is None else n_freed
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    _check("kv_rollback_token_table", lib().kv_rollback_token_table(
        _ptr(req_to_token), stride, _ptr(tree_slots), _ptr(cu_nodes), _ptr(prefix_len), _ptr(accept_len),
        _ptr(accept_idx), B, total_nodes, max_depth, _ptr(new_len), _ptr(freed_slots), _ptr(n_freed), _ptr(err),
        _stream(stream)))
    return new_len, freed_slots, n_freed, err


# ---------------------------------------------------------------------------
# Tree-aware Gated-DeltaNet verification (tree_gdn_conv, tree_gdn_verify,
# tree_gdn_commit).  q, k and v are [T, H, 128] bf16 tensors sharing one row
# stride, e.g. the views gdn_split() takes of tree_gdn_conv's output.
# ---------------------------------------------------------------------------

def gdn_split(y, hk: int, hv: int, d: int = 128):
    """Views (q, k, v) of a mixed [T, 2*hk*d + hv*d] row: q, then k, then v."""
    T = y.shape[0]
    q = y[:, :hk * d].unflatten(1, (hk, d))
    k = y[:, hk * d:2 * hk * d].unflatten(1, (hk, d))
    v = y[:, 2 * hk * d:].unflatten(1, (hv, d))
    assert v.shape == (T, hv, d)
    return q, k, v


def _rows_stride(ts, names):
    """Common row stride of [T, H, d] bf16 tensors with unit channel stride."""
    import torch
    rs = None
    for t, n in zip(ts, names):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
        if t.dtype != torch.bfloat16 or t.dim() != 3:
            raise TypeError(f"{n} must be a [T, H, d] bfloat16 tensor")
        if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{n} must have contiguous heads")
        s = t.stride(0) if t.shape[0] > 1 else None
        if s is not None:
            if rs is not None and s != rs:
                raise ValueError("q, k and v must share one row stride")
            rs = s
    if rs is None:
        rs = max(t.shape[1] * t.shape[2] for t in ts)
    return rs


def tree_gdn_conv(x, conv_state, weight, parent, cu_nodes, y=None, err=None, stream=None):
    """x [T, C] bf16, conv_state [B, K-1, C] bf16, weight [C, K] bf16 ->
    (y [T, C] bf16, err)."""
    import torch
    T, Cc = x.shape
    B = cu_nodes.numel() - 1
    K = weight.shape[1]
    for t, n in ((x, "x"), (conv_state, "conv_state"), (weight, "weight")):
        _need(t, n, torch.bfloat16)
    _need(parent, "parent", torch.int32, T)
    _need(cu_nodes, "cu_nodes", torch.int32)
    y = torch.empty_like(x) if y is None else y
    _need(y, "y", torch.bfloat16, T * Cc)
    err = torch.zeros(1, dtype=torch.int32, device=x.device) if err is None else err
    _check("tree_gdn_conv", lib().tree_gdn_conv(
        _ptr(x), _ptr(conv_state), _ptr(weight), _ptr(parent), _ptr(cu_nodes), B, T, Cc, K, _ptr(y), _ptr(err),
        _stream(stream)))
    return y, err


def tree_gdn_verify(q, k, v, g, beta, state, parent, cu_nodes, max_depth: int, scale: float | None = None,
                    l2norm: bool = True, out=None, err=None, stream=None):
    """q, k [T, hk, 128], v [T, hv, 128] bf16 (one row stride); g, beta [T, hv]
    float32; state [B, hv, 128, 128] float32 -> (out [T, hv, 128] float32, err)."""
    import torch
    T, hk, d = q.shape
    hv = v.shape[1]
    B = cu_nodes.numel() - 1
    rs = _rows_stride((q, k, v), ("q", "k", "v"))
    for t, n in ((g, "g"), (beta, "beta"), (state, "state")):
        _need(t, n, torch.float32)
    _need(parent, "parent", torch.int32, T)
    _need(cu_nodes, "cu_nodes", torch.int32)
    scale = d ** -0.5 if scale is None else scale
    out = torch.empty((T, hv, d), dtype=torch.float32, device=q.device) if out is None else out
    _need(out, "out", torch.float32, T * hv * d)
    err = torch.zeros(1, dtype=torch.int32, device=q.device) if err is None else err
    _check("tree_gdn_verify", lib().tree_gdn_verify(
        _ptr(q), _ptr(k), _ptr(v), rs, _ptr(g), _ptr(beta), _ptr(state), _ptr(parent), _ptr(cu_nodes), B, T,
        max_depth, hk, hv, d, float(scale), int(bool(l2norm)), _ptr(out), _ptr(err), _stream(stream)))
    return out, err


def tree_gdn_commit(state, conv_state, x, k, v, g, beta, cu_nodes, accept_len, accept_idx, max_depth: int,
                    l2norm: bool = True, err=None, stream=None):
    """Advances state [B, hv, 128, 128] float32 and conv_state [B, K-1, C] bf16
    in place by each request's accepted path -> err."""
    import torch
    T, Cc = x.shape
    B = cu_nodes.numel() - 1
    hk, hv, d = k.shape[1], v.shape[1], k.shape[2]
    rs = _rows_stride((k, v), ("k", "v"))
    _need(state, "state", torch.float32)
    _need(conv_state, "conv_state", torch.bfloat16)
    _need(x, "x", torch.bfloat16)
    for t, n in ((g, "g"), (beta, "beta")):
        _need(t, n, torch.float32)
    for t, n in ((cu_nodes, "cu_nodes"), (accept_len, "accept_len"), (accept_idx, "accept_idx")):
        _need(t, n, torch.int32)
    K = conv_state.shape[1] + 1
    err = torch.zeros(1, dtype=torch.int32, device=state.device) if err is None else err
    _check("tree_gdn_commit", lib().tree_gdn_commit(
        _ptr(state), _ptr(conv_state), _ptr(x), _ptr(k), _ptr(v), rs, _ptr(g), _ptr(beta), _ptr(cu_nodes),
        _ptr(accept_len), _ptr(accept_idx), B, T, max_depth, hk, hv, d, Cc, K, int(bool(l2norm)), _ptr(err),
        _stream(stream)))
    return err
