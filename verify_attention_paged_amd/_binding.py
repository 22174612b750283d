"""ctypes binding of the C ABI in include/vap.h (argument marshalling only).

Every computation runs in the HIP library ``lib/libvap.so``; this module checks tensor
dtypes, devices and shapes, passes ``data_ptr()`` values and torch's current HIP stream, and
turns negative return codes into ``VapError``.  There is no fallback: if the library is
missing or the device is not gfx950, calls raise.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import re

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libvap.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vap.h")

VAP_OK, VAP_EINVAL, VAP_ENOSPC, VAP_EHIP, VAP_ENODEV = 0, -1, -2, -3, -4
DERR_BLOCK_ID, DERR_LENS, DERR_TOTAL_Q, DERR_DRAFT_ID, DERR_EMPTY_ROW, DERR_TREE, DERR_TEMP, DERR_SYNC = (
    0x1, 0x2, 0x4, 0x8, 0x10, 0x20, 0x40, 0x80)
TIMER_ATTENTION, TIMER_VERIFY, TIMER_TREE_VERIFY, TIMER_KV_APPEND, TIMER_KV_COMMIT = 0, 1, 2, 3, 4
TIMER_LOGIT_STATS, TIMER_VERIFY_LOGITS, TIMER_TREE_DRAW = 5, 6, 7


class VapError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (code {code})")
        self.code = code


class AttnShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


_vp, _sz, _i32, _pi32, _pdbl = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)
_pshape = ctypes.POINTER(AttnShape)

SIGNATURES = {
    "vap_attn_workspace_bytes": (_sz, [_pshape]),
    "vap_attn_workspace_min_bytes": (_sz, [_pshape]),
    "paged_attn_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _pshape, _vp, _sz, _vp]),
    "paged_attn_step_u8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _pshape, _vp, _sz, _vp]),
    "paged_attn_step_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _pshape, _vp, _sz, _vp]),
    "paged_attn_step_tree": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _pshape, _vp, _sz, _vp]),
    "vap_verify_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "spec_verify": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "spec_verify_static": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "vap_verify_logits_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "spec_verify_logits": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "vap_tree_verify_workspace_bytes": (_sz, [_i32]),
    "spec_verify_tree": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "vap_kv_workspace_bytes": (_sz, []),
    "kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _pshape, _vp, _sz, _vp]),
    "kv_commit": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _pshape, _vp, _sz, _vp]),
    "vap_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "vap_get_device_error": (ctypes.c_int, [_vp, _vp, _pi32, ctypes.c_int]),
    "vap_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "vap_last_error_message": (ctypes.c_char_p, []),
    "vap_timer_enable": (ctypes.c_int, [ctypes.c_int]),
    "vap_timer_read": (ctypes.c_int, [ctypes.c_int, _pdbl, _pi32, ctypes.c_int]),
    "vap_stream_copy": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
    "vap_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _vp]),
    "vap_device_info": (ctypes.c_int, [_pi32, ctypes.c_char_p, _sz]),
}

_lib = None


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions declared in include/vap.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


def load_library(path: str = LIB_PATH):
    """Load libvap.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise VapError(VAP_ENODEV, f"HIP library {path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int) -> None:
    if rc != VAP_OK:
        lib = load_library()
        msg = lib.vap_last_error_message().decode() or lib.vap_strerror(rc).decode()
        raise VapError(rc, msg)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(device: torch.device):
    """Context making `device` current for a library call (no switch when it already is: the
    switch costs more host time than the call's own work)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _need(t: torch.Tensor, name: str, dtype, ndim: int | None = None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")


# ---------------------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------------------

def attn_shape(q: torch.Tensor, kv_pool: torch.Tensor, block_tables: torch.Tensor,
               scale: float = 0.0) -> AttnShape:
    T, Hq, D = q.shape
    two, NB, BS, Hkv, D2 = kv_pool.shape
    B, MB = block_tables.shape
    if two != 2 or D2 != D:
        raise ValueError(f"kv_pool must be [2, num_blocks, block_size, Hkv, {D}], got {tuple(kv_pool.shape)}")
    return AttnShape(B, Hq, Hkv, D, BS, NB, MB, T, float(scale))


def attn_workspace(shape: AttnShape, device=None) -> torch.Tensor:
    """Zero-filled device workspace sized for ``shape`` on ``device``."""
    lib = load_library()
    device = torch.device(device or "cuda")
    with torch.cuda.device(device):
        n = lib.vap_attn_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        _check(VAP_EINVAL)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def paged_attn_step(q, kv_pool, block_tables, ctx_lens, q_lens, out=None, *, scale: float = 0.0,
                    workspace: torch.Tensor | None = None, stream=None, kv_scales=None,
                    tree_mask=None, fp8: bool = False) -> torch.Tensor:
    """Paged attention for one ragged batch; see ``paged_attn_step`` in include/vap.h.

    q bf16 [T, Hq, D]; kv_pool bf16 [2, NB, bs, Hkv, D]; block_tables int32 [B, MB];
    ctx_lens, q_lens int32 [B]; returns out fp32 [T, Hq, D].  With ``kv_scales`` (fp32
    [NB, Hkv, bs, 4]) the pool holds uint8 codes and ``paged_attn_step_u8`` is called, or with
    ``fp8=True`` E4M3 codes and ``paged_attn_step_fp8``.  With ``tree_mask`` (int64 [T] holding
    uint64 ancestor masks) ``paged_attn_step_tree`` is called (bf16 or uint8 codes).
    """
    lib = load_library()
    dev = q.device
    kv8 = kv_scales is not None
    if fp8 and (not kv8 or tree_mask is not None):
        raise ValueError("fp8 needs kv_scales and no tree_mask")
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_pool, "kv_pool", torch.uint8 if kv8 else torch.bfloat16, 5, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, 1, dev)
    _need(q_lens, "q_lens", torch.int32, 1, dev)
    shape = attn_shape(q, kv_pool, block_tables, scale)
    if kv8:
        _need(kv_scales, "kv_scales", torch.float32, 4, dev)
        if tuple(kv_scales.shape) != (shape.num_blocks, shape.num_kv_heads, shape.block_size, 4):
            raise ValueError("kv_scales must be [num_blocks, Hkv, block_size, 4]")
    if ctx_lens.numel() != shape.num_seqs or q_lens.numel() != shape.num_seqs:
        raise ValueError("ctx_lens and q_lens need one entry per block-table row")
    if tree_mask is not None:
        _need(tree_mask, "tree_mask", torch.int64, 1, dev)
        if tree_mask.numel() != shape.total_q:
            raise ValueError("tree_mask needs one entry per query row")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 3, dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    if workspace is None:
        workspace = attn_workspace(shape, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    with _on(dev):
        if tree_mask is not None:
            rc = lib.paged_attn_step_tree(q.data_ptr(), kv_pool.data_ptr(), kv_scales.data_ptr() if kv8 else None,
                                          block_tables.data_ptr(), ctx_lens.data_ptr(), q_lens.data_ptr(),
                                          tree_mask.data_ptr(), out.data_ptr(), ctypes.byref(shape),
                                          workspace.data_ptr(), workspace.numel(), _stream(stream))
        elif kv8:
            fn = lib.paged_attn_step_fp8 if fp8 else lib.paged_attn_step_u8
            rc = fn(q.data_ptr(), kv_pool.data_ptr(), kv_scales.data_ptr(), block_tables.data_ptr(),
                    ctx_lens.data_ptr(), q_lens.data_ptr(), out.data_ptr(), ctypes.byref(shape),
                    workspace.data_ptr(), workspace.numel(), _stream(stream))
        else:
            rc = lib.paged_attn_step(q.data_ptr(), kv_pool.data_ptr(), block_tables.data_ptr(),
                                     ctx_lens.data_ptr(), q_lens.data_ptr(), out.data_ptr(),
                                     ctypes.byref(shape), workspace.data_ptr(), workspace.numel(),
                                     _stream(stream))
    _check(rc)
    return out


# ---------------------------------------------------------------------------------------
# speculative verification
# ---------------------------------------------------------------------------------------

def verify_workspace(num_seqs: int, k: int, vocab: int, device=None) -> torch.Tensor:
    lib = load_library()
    n = lib.vap_verify_workspace_bytes(num_seqs, k, vocab)
    if n == 0:
        _check(VAP_EINVAL)
    return torch.zeros(n, dtype=torch.uint8, device=torch.device(device or "cuda"))


def _verify_args(p, q, draft_ids, uniforms, out_ids, n_accepted):
    """Checks of spec_verify's tensors; returns (B, k, V, out_ids, n_accepted, q ptr, ids ptr)."""
    dev = p.device
    _need(p, "p", torch.float32, 3)
    B, k1, V = p.shape
    k = k1 - 1
    _need(uniforms, "uniforms", torch.float32, 2, dev)
    if tuple(uniforms.shape) != (B, k + 1):
        raise ValueError("uniforms must be [B, k+1]")
    if k > 0:
        _need(q, "q", torch.float32, 3, dev)
        _need(draft_ids, "draft_ids", torch.int32, 2, dev)
        if tuple(q.shape) != (B, k, V) or tuple(draft_ids.shape) != (B, k):
            raise ValueError("q must be [B, k, V] and draft_ids [B, k]")
    if out_ids is None:
        out_ids = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_ids, "out_ids", torch.int32, 2, dev)
    _need(n_accepted, "n_accepted", torch.int32, 1, dev)
    qp = q.data_ptr() if k > 0 else None
    ip = draft_ids.data_ptr() if k > 0 else None
    return B, k, V, out_ids, n_accepted, qp, ip


def spec_verify(p, q, draft_ids, uniforms, out_ids=None, n_accepted=None, *,
                workspace: torch.Tensor | None = None, stream=None):
    """Modified rejection sampling; see ``spec_verify`` in include/vap.h.

    p fp32 [B, k+1, V]; q fp32 [B, k, V]; draft_ids int32 [B, k]; uniforms fp32 [B, k+1].
    Returns (out_ids int32 [B, k+1], n_accepted int32 [B]).
    """
    lib = load_library()
    dev = p.device
    B, k, V, out_ids, n_accepted, qp, ip = _verify_args(p, q, draft_ids, uniforms, out_ids, n_accepted)
    if workspace is None:
        workspace = verify_workspace(B, k, V, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    with _on(dev):
        rc = lib.spec_verify(p.data_ptr(), qp, ip, uniforms.data_ptr(), out_ids.data_ptr(),
                             n_accepted.data_ptr(), B, k, V, workspace.data_ptr(),
                             workspace.numel(), _stream(stream))
    _check(rc)
    return out_ids, n_accepted


def spec_verify_static(p, q, draft_ids, uniforms, out_ids, n_accepted, *, device_error=None, stream=None):
    """spec_verify without a workspace (the library's static device scratch); see
    ``spec_verify_static`` in include/vap.h.  Outputs are given by the caller; ``device_error``
    is an optional int32 [1] device tensor receiving the VAP_DERR_* bits."""
    lib = load_library()
    dev = p.device
    B, k, V, out_ids, n_accepted, qp, ip = _verify_args(p, q, draft_ids, uniforms, out_ids, n_accepted)
    ep = None
    if device_error is not None:
        _need(device_error, "device_error", torch.int32, 1, dev)
        ep = device_error.data_ptr()
    with _on(dev):
        rc = lib.spec_verify_static(p.data_ptr(), qp, ip, uniforms.data_ptr(), out_ids.data_ptr(),
                                    n_accepted.data_ptr(), B, k, V, ep, _stream(stream))
    _check(rc)
    return out_ids, n_accepted


def verify_logits_workspace(num_seqs: int, k: int, vocab: int, device=None) -> torch.Tensor:
    lib = load_library()
    n = lib.vap_verify_logits_workspace_bytes(num_seqs, k, vocab)
    if n == 0:
        _check(VAP_EINVAL)
    return torch.zeros(n, dtype=torch.uint8, device=torch.device(device or "cuda"))


def spec_verify_logits(target_logits, draft_logits, draft_ids, uniforms, temperatures, out_ids=None,
                       n_accepted=None, *, workspace: torch.Tensor | None = None, stream=None):
    """Verification from logits; see ``spec_verify_logits`` in include/vap.h.

    target_logits fp32 [B, k+1, V]; draft_logits fp32 [B, k, V]; draft_ids int32 [B, k];
    uniforms fp32 [B, k+1]; temperatures fp32 [B] (0 = greedy).
    Returns (out_ids int32 [B, k+1], n_accepted int32 [B]).
    """
    lib = load_library()
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, 3)
    B, k1, V = target_logits.shape
    k = k1 - 1
    _need(uniforms, "uniforms", torch.float32, 2, dev)
    _need(temperatures, "temperatures", torch.float32, 1, dev)
    if tuple(uniforms.shape) != (B, k + 1) or temperatures.numel() != B:
        raise ValueError("uniforms must be [B, k+1] and temperatures [B]")
    if k > 0:
        _need(draft_logits, "draft_logits", torch.float32, 3, dev)
        _need(draft_ids, "draft_ids", torch.int32, 2, dev)
        if tuple(draft_logits.shape) != (B, k, V) or tuple(draft_ids.shape) != (B, k):
            raise ValueError("draft_logits must be [B, k, V] and draft_ids [B, k]")
    if out_ids is None:
        out_ids = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_ids, "out_ids", torch.int32, 2, dev)
    _need(n_accepted, "n_accepted", torch.int32, 1, dev)
    if workspace is None:
        workspace = verify_logits_workspace(B, k, V, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    with _on(dev):
        rc = lib.spec_verify_logits(target_logits.data_ptr(), draft_logits.data_ptr() if k > 0 else None,
                                    draft_ids.data_ptr() if k > 0 else None, uniforms.data_ptr(),
                                    temperatures.data_ptr(), out_ids.data_ptr(), n_accepted.data_ptr(), B, k, V,
                                    workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(rc)
    return out_ids, n_accepted


def tree_verify_workspace(num_seqs: int, device=None) -> torch.Tensor:
    n = load_library().vap_tree_verify_workspace_bytes(num_seqs)
    if n == 0:
        _check(VAP_EINVAL)
    return torch.zeros(n, dtype=torch.uint8, device=torch.device(device or "cuda"))


def spec_verify_tree(p, q, parents, tokens, uniforms, out_ids=None, out_path=None, n_accepted=None, *,
                     workspace: torch.Tensor | None = None, stream=None):
    """Verification of draft token trees; see ``spec_verify_tree`` in include/vap.h.

    p, q fp32 [B, N, V]; parents, tokens int32 [B, N]; uniforms fp32 [B, N].
    Returns (out_ids int32 [B, N], out_path int32 [B, N], n_accepted int32 [B]).
    """
    lib = load_library()
    dev = p.device
    _need(p, "p", torch.float32, 3)
    B, N, V = p.shape
    _need(q, "q", torch.float32, 3, dev)
    if tuple(q.shape) != (B, N, V):
        raise ValueError("q must have the shape of p")
    for t, name, dt in ((parents, "parents", torch.int32), (tokens, "tokens", torch.int32),
                        (uniforms, "uniforms", torch.float32)):
        _need(t, name, dt, 2, dev)
        if tuple(t.shape) != (B, N):
            raise ValueError(f"{name} must be [B, N]")
    if out_ids is None:
        out_ids = torch.empty((B, N), dtype=torch.int32, device=dev)
    if out_path is None:
        out_path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    for t, name in ((out_ids, "out_ids"), (out_path, "out_path")):
        _need(t, name, torch.int32, 2, dev)
    _need(n_accepted, "n_accepted", torch.int32, 1, dev)
    if workspace is None:
        workspace = tree_verify_workspace(B, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    with _on(dev):
        rc = lib.spec_verify_tree(p.data_ptr(), q.data_ptr(), parents.data_ptr(), tokens.data_ptr(),
                                  uniforms.data_ptr(), out_ids.data_ptr(), out_path.data_ptr(),
                                  n_accepted.data_ptr(), B, N, V, workspace.data_ptr(), workspace.numel(),
                                  _stream(stream))
    _check(rc)
    return out_ids, out_path, n_accepted


# ---------------------------------------------------------------------------------------
# KV append / commit
# ---------------------------------------------------------------------------------------

def kv_workspace(device=None) -> torch.Tensor:
    n = load_library().vap_kv_workspace_bytes()
    return torch.zeros(n, dtype=torch.uint8, device=torch.device(device or "cuda"))


def _kv_checks(kv_pool, kv_scales, block_tables, ctx_lens, q_lens, dev):
    kv8 = kv_scales is not None
    _need(kv_pool, "kv_pool", torch.uint8 if kv8 else torch.bfloat16, 5, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, 1, dev)
    _need(q_lens, "q_lens", torch.int32, 1, dev)
    two, NB, BS, Hkv, D = kv_pool.shape
    if two != 2:
        raise ValueError(f"kv_pool must be [2, num_blocks, block_size, Hkv, D], got {tuple(kv_pool.shape)}")
    if kv8:
        _need(kv_scales, "kv_scales", torch.float32, 4, dev)
        if tuple(kv_scales.shape) != (NB, Hkv, BS, 4):
            raise ValueError("kv_scales must be [num_blocks, Hkv, block_size, 4]")
    B = block_tables.shape[0]
    if ctx_lens.numel() != B or q_lens.numel() != B:
        raise ValueError("ctx_lens and q_lens need one entry per block-table row")


def kv_append(k_new, v_new, kv_pool, block_tables, ctx_lens, q_lens, *, kv_scales=None,
              workspace: torch.Tensor | None = None, stream=None) -> None:
    """Write new K/V rows into the paged pool in place; see ``kv_append`` in include/vap.h.

    k_new, v_new bf16 [T, Hkv, D]; kv_pool bf16 [2, NB, bs, Hkv, D] (or uint8 codes with
    ``kv_scales`` fp32 [NB, Hkv, bs, 4], both written); block_tables int32 [B, MB]; ctx_lens
    (counting the new rows) and q_lens int32 [B].
    """
    lib = load_library()
    dev = kv_pool.device
    _kv_checks(kv_pool, kv_scales, block_tables, ctx_lens, q_lens, dev)
    _need(k_new, "k_new", torch.bfloat16, 3, dev)
    _need(v_new, "v_new", torch.bfloat16, 3, dev)
    _, NB, BS, Hkv, D = kv_pool.shape
    if tuple(k_new.shape[1:]) != (Hkv, D) or k_new.shape != v_new.shape:
        raise ValueError(f"k_new and v_new must be [T, {Hkv}, {D}]")
    B, MB = block_tables.shape
    shape = AttnShape(B, Hkv, Hkv, D, BS, NB, MB, k_new.shape[0], 0.0)
    if workspace is None:
        workspace = kv_workspace(dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    with _on(dev):
        rc = lib.kv_append(k_new.data_ptr(), v_new.data_ptr(), kv_pool.data_ptr(),
                           kv_scales.data_ptr() if kv_scales is not None else None, block_tables.data_ptr(),
                           ctx_lens.data_ptr(), q_lens.data_ptr(), ctypes.byref(shape), workspace.data_ptr(),
                           workspace.numel(), _stream(stream))
    _check(rc)


def kv_commit(kv_pool, block_tables, ctx_lens, q_lens, n_accepted, *, path=None, kv_scales=None,
              out_ctx_lens=None, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Keep the accepted draft tokens; see ``kv_commit`` in include/vap.h.

    n_accepted int32 [B]; path None (a chain) or int32 [B, stride] of accepted tree nodes
    (spec_verify_tree's out_path).  The pool (and ``kv_scales``) change in place; returns the
    committed lengths int32 [B] (``out_ctx_lens``, which may be ``ctx_lens`` itself).
    """
    lib = load_library()
    dev = kv_pool.device
    _kv_checks(kv_pool, kv_scales, block_tables, ctx_lens, q_lens, dev)
    _need(n_accepted, "n_accepted", torch.int32, 1, dev)
    B, MB = block_tables.shape
    if n_accepted.numel() != B:
        raise ValueError("n_accepted needs one entry per block-table row")
    stride = 0
    if path is not None:
        _need(path, "path", torch.int32, 2, dev)
        if path.shape[0] != B:
            raise ValueError("path must be [B, stride]")
        stride = path.shape[1]
    if out_ctx_lens is None:
        out_ctx_lens = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_ctx_lens, "out_ctx_lens", torch.int32, 1, dev)
    _, NB, BS, Hkv, D = kv_pool.shape
    shape = AttnShape(B, Hkv, Hkv, D, BS, NB, MB, 0, 0.0)
    if workspace is None:
        workspace = kv_workspace(dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    with _on(dev):
        rc = lib.kv_commit(kv_pool.data_ptr(), kv_scales.data_ptr() if kv_scales is not None else None,
                           block_tables.data_ptr(), ctx_lens.data_ptr(), q_lens.data_ptr(),
                           path.data_ptr() if path is not None else None, stride, n_accepted.data_ptr(),
                           out_ctx_lens.data_ptr(), ctypes.byref(shape), workspace.data_ptr(), workspace.numel(),
                           _stream(stream))
    _check(rc)
    return out_ctx_lens


# ---------------------------------------------------------------------------------------
# workspace, errors, measurement helpers
# ---------------------------------------------------------------------------------------

def workspace_init(workspace: torch.Tensor, stream=None) -> None:
    _check(load_library().vap_workspace_init(workspace.data_ptr(), workspace.numel(), _stream(stream)))


def get_device_error(workspace: torch.Tensor, stream=None, clear: bool = False) -> int:
    err = ctypes.c_int32(0)
    with torch.cuda.device(workspace.device):
        _check(load_library().vap_get_device_error(workspace.data_ptr(), _stream(stream),
                                                   ctypes.byref(err), int(clear)))
    return int(err.value)


def timer_enable(on: bool = True) -> None:
    _check(load_library().vap_timer_enable(int(on)))


def timer_read(kind: int, reset: bool = True):
    """(summed milliseconds, number of recorded kernels) of timer `kind`."""
    total = ctypes.c_double(0.0)
    count = ctypes.c_int32(0)
    _check(load_library().vap_timer_read(kind, ctypes.byref(total), ctypes.byref(count), int(reset)))
    return total.value, int(count.value)


def stream_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    if dst.numel() * dst.element_size() < src.numel() * src.element_size():
        raise ValueError("dst smaller than src")
    nbytes = src.numel() * src.element_size()
    _check(load_library().vap_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream(stream)))


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    _check(load_library().vap_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream(stream)))


def device_info():
    n = ctypes.c_int32(0)
    buf = ctypes.create_string_buffer(64)
    _check(load_library().vap_device_info(ctypes.byref(n), buf, 64))
    return int(n.value), buf.value.decode()
