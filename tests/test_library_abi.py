"""The C-ABI library loads, exports every symbol include/vap.h declares, and rejects bad
arguments on the host before touching a device (CPU only; no kernel is launched)."""

import ctypes
import os

import pytest

import verify_attention_paged_amd as vap
from verify_attention_paged_amd import _binding as B


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vap.LIB_PATH):
        from verify_attention_paged_amd.build import build
        build()
    return vap.load_library()


def test_exports_every_declared_symbol(lib):
    names = vap.header_functions()
    assert {"paged_attn_step", "paged_attn_step_u8", "paged_attn_step_tree", "spec_verify", "spec_verify_tree", "kv_append", "kv_commit", "vap_attn_workspace_bytes", "vap_verify_workspace_bytes",
            "vap_get_device_error", "vap_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.SIGNATURES), "binding signatures out of sync with the header"


def test_strerror_and_codes(lib):
    assert lib.vap_strerror(0) == b"ok"
    assert lib.vap_strerror(-2) == b"workspace too small"
    assert lib.vap_strerror(-99) == b"unknown error"


def _shape(**kw):
    base = dict(num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                num_blocks=35, max_blocks_per_seq=16, total_q=4, scale=0.0)
    base.update(kw)
    return vap.AttnShape(**base)


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(block_size=8), dict(num_q_heads=6, num_kv_heads=4),
                                 dict(num_seqs=-1), dict(num_seqs=9000), dict(total_q=-1),
                                 dict(num_blocks=0), dict(scale=float("nan")), dict(scale=-1.0),
                                 dict(num_kv_heads=0)])
def test_attention_shape_rejected_on_host(lib, bad):
    s = _shape(**bad)
    assert lib.vap_attn_workspace_min_bytes(ctypes.byref(s)) == 0
    rc = lib.paged_attn_step(None, None, None, None, None, None, ctypes.byref(s), None, 0, None)
    assert rc == B.VAP_EINVAL
    assert lib.vap_last_error_message()


def test_attention_null_pointers_and_empty_batch(lib):
    s = _shape()
    assert lib.paged_attn_step(None, None, None, None, None, None, None, None, 0, None) == B.VAP_EINVAL
    assert lib.paged_attn_step(None, None, None, None, None, None, ctypes.byref(s), None, 0, None) == B.VAP_EINVAL
    empty = _shape(num_seqs=0, total_q=0)
    assert lib.paged_attn_step(None, None, None, None, None, None, ctypes.byref(empty), None, 0, None) == B.VAP_OK
    bad_empty = _shape(num_seqs=0, total_q=3)
    assert lib.paged_attn_step(None, None, None, None, None, None, ctypes.byref(bad_empty), None, 0, None) == B.VAP_EINVAL


def test_u8_attention_null_pointers_and_empty_batch(lib):
    s = B.AttnShape(4, 8, 2, 64, 16, 35, 16, 4, 0.0)
    fake = ctypes.c_void_p(16)        # never dereferenced: the host check fails first
    assert lib.paged_attn_step_u8(None, None, None, None, None, None, None, ctypes.byref(s), None, 0, None) == B.VAP_EINVAL
    # codes given but no scales
    assert lib.paged_attn_step_u8(fake, fake, None, fake, fake, fake, fake, ctypes.byref(s), fake, 1 << 20, None) == B.VAP_EINVAL
    empty = B.AttnShape(0, 8, 2, 64, 16, 35, 16, 0, 0.0)
    assert lib.paged_attn_step_u8(None, None, None, None, None, None, None, ctypes.byref(empty), None, 0, None) == B.VAP_OK


def test_tree_verify_rejected_on_host(lib):
    ws = lib.vap_tree_verify_workspace_bytes(4)
    assert ws >= 256 + 4 * (32 + 256 * 8 + 4) and ws % 256 == 0
    assert lib.vap_tree_verify_workspace_bytes(-1) == 0
    assert lib.vap_tree_verify_workspace_bytes(8) > ws
    assert lib.spec_verify_tree(None, None, None, None, None, None, None, None, 4, 65, 10, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify_tree(None, None, None, None, None, None, None, None, 4, 0, 10, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify_tree(None, None, None, None, None, None, None, None, 4, 8, 0, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify_tree(None, None, None, None, None, None, None, None, 4, 8, (1 << 20) + 1, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify_tree(None, None, None, None, None, None, None, None, 4, 8, 10, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify_tree(None, None, None, None, None, None, None, None, 0, 8, 10, None, 0, None) == B.VAP_OK


def test_kv_append_and_commit_rejected_on_host(lib):
    s = B.AttnShape(4, 8, 2, 64, 16, 35, 16, 4, 0.0)
    fake = ctypes.c_void_p(256)       # never dereferenced: the host check fails first
    ws = lib.vap_kv_workspace_bytes()
    assert ws >= 4
    append = lambda *a: lib.kv_append(*a)
    # NULL pool / workspace, small workspace, misaligned new rows, bad shape
    assert append(fake, fake, None, None, fake, fake, fake, ctypes.byref(s), fake, ws, None) == B.VAP_EINVAL
    assert append(fake, fake, fake, None, fake, fake, fake, ctypes.byref(s), fake, 2, None) == B.VAP_ENOSPC
    assert append(ctypes.c_void_p(258), fake, fake, None, fake, fake, fake, ctypes.byref(s), fake, ws, None) == B.VAP_EINVAL
    assert append(fake, fake, fake, None, None, fake, fake, ctypes.byref(s), fake, ws, None) == B.VAP_EINVAL
    bad = B.AttnShape(4, 8, 2, 96, 16, 35, 16, 4, 0.0)
    assert append(fake, fake, fake, None, fake, fake, fake, ctypes.byref(bad), fake, ws, None) == B.VAP_EINVAL
    empty = B.AttnShape(0, 8, 2, 64, 16, 35, 16, 0, 0.0)
    assert append(None, None, None, None, None, None, None, ctypes.byref(empty), None, 0, None) == B.VAP_OK
    bad_empty = B.AttnShape(0, 8, 2, 64, 16, 35, 16, 3, 0.0)
    assert append(None, None, None, None, None, None, None, ctypes.byref(bad_empty), None, 0, None) == B.VAP_EINVAL
    commit = lambda *a: lib.kv_commit(*a)
    assert commit(None, None, fake, fake, fake, None, 0, fake, fake, ctypes.byref(s), fake, ws, None) == B.VAP_EINVAL
    assert commit(fake, None, fake, fake, fake, None, 0, None, fake, ctypes.byref(s), fake, ws, None) == B.VAP_EINVAL
    assert commit(fake, None, fake, fake, fake, fake, 0, fake, fake, ctypes.byref(s), fake, ws, None) == B.VAP_EINVAL
    assert commit(fake, None, fake, fake, fake, None, 0, fake, fake, ctypes.byref(s), fake, 0, None) == B.VAP_ENOSPC
    assert commit(None, None, None, None, None, None, 0, None, None, ctypes.byref(empty), None, 0, None) == B.VAP_OK


def test_verify_logits_rejected_on_host(lib):
    f = lib.spec_verify_logits
    assert lib.vap_verify_logits_workspace_bytes(16, 4, 128256) > 0
    assert lib.vap_verify_logits_workspace_bytes(16, 65, 100) == 0
    assert lib.vap_verify_logits_workspace_bytes(16, 4, (1 << 20) + 1) == 0
    assert f(None, None, None, None, None, None, None, 4, 65, 10, None, 0, None) == B.VAP_EINVAL
    assert f(None, None, None, None, None, None, None, 4, 4, 0, None, 0, None) == B.VAP_EINVAL
    assert f(None, None, None, None, None, None, None, 4, 4, 10, None, 0, None) == B.VAP_EINVAL
    fake = ctypes.c_void_p(256)
    # temperatures missing
    assert f(fake, fake, fake, fake, None, fake, fake, 4, 4, 10, fake, 1 << 20, None) == B.VAP_EINVAL
    # workspace too small
    assert f(fake, fake, fake, fake, fake, fake, fake, 4, 4, 10, fake, 64, None) == B.VAP_ENOSPC
    assert f(None, None, None, None, None, None, None, 0, 4, 10, None, 0, None) == B.VAP_OK


def _a256(x):
    return (x + 255) // 256 * 256


def test_verifier_workspace_layouts(lib):
    """Header, then one record per sequence (its ticket first, then its data: 256 fp64 chunk
    sums; for a tree also the walk's end state and the 16 x 16 chunk sums its workgroups
    share); the logits workspace puts the statistics partials (16 bytes per row and 2048-token
    chunk) before the records."""
    rec = 16 + 8 * 256
    walk = 8 * 256
    for B in (1, 7, 1000, 1 << 22):
        assert lib.vap_verify_workspace_bytes(B, 4, 128256) == _a256(256 + B * rec)
        assert lib.vap_tree_verify_workspace_bytes(B) == _a256(256 + B * (rec + 32 + walk))
    for B, k, V in ((1, 4, 1 << 20), (1000, 0, 4), (16, 4, 128256), (3, 64, 2049)):
        part = B * (2 * k + 1) * ((V + 2047) // 2048) * 16
        assert lib.vap_verify_logits_workspace_bytes(B, k, V) == _a256(_a256(256 + part) + B * rec)


def test_workspace_sizes_are_consistent(lib):
    s = _shape(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, num_blocks=6000,
               max_blocks_per_seq=512, total_q=64)
    lo = lib.vap_attn_workspace_min_bytes(ctypes.byref(s))
    hi = lib.vap_attn_workspace_bytes(ctypes.byref(s))
    assert 0 < lo < hi and lo % 256 == 0 and hi % 256 == 0
    assert lib.vap_verify_workspace_bytes(16, 4, 128256) > 0
    assert lib.vap_verify_workspace_bytes(16, 65, 100) == 0
    assert lib.vap_verify_workspace_bytes(-1, 4, 100) == 0


def test_verify_rejected_on_host(lib):
    assert lib.spec_verify(None, None, None, None, None, None, 4, 65, 10, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify(None, None, None, None, None, None, 4, 4, 0, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify(None, None, None, None, None, None, 4, 4, 10, None, 0, None) == B.VAP_EINVAL
    assert lib.spec_verify(None, None, None, None, None, None, 0, 4, 10, None, 0, None) == B.VAP_OK


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(4, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vap.paged_attn_step(q, q, q, q, q)
