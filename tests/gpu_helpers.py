"""Helpers shared by the GPU parity tests: device transfer, oracle calls, tolerance check."""

from __future__ import annotations

import functools

import numpy as np
import torch

import workloads
from oracle import attention as OA

# attention parity bar: |gpu - ref| <= ATOL + RTOL * |ref| elementwise (bf16 inputs, fp32 accumulation)
ATOL = 2e-3
RTOL = 1e-2


def device():
    return torch.device("cuda:0")


def to_device(inp: workloads.AttnInputs, dev=None):
    """Device copies of the inputs as keyword arguments of ``vap.paged_attn_step`` (with
    ``kv_scales`` for an 8-bit cache)."""
    dev = dev or device()
    d = dict(q=inp.q.to(dev), kv_pool=inp.kv_pool.to(dev), block_tables=inp.block_tables.to(dev),
             ctx_lens=inp.ctx_lens.to(dev), q_lens=inp.q_lens.to(dev))
    if inp.kv_scales is not None:
        d["kv_scales"] = inp.kv_scales.to(dev)
    if inp.fp8:
        d["fp8"] = True
    return d


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a CPU bf16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_rows(inp: workloads.AttnInputs, rows=None, scale=None) -> dict:
    if inp.fp8:
        return OA.paged_attention_fp8(bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(),
                                      inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy(),
                                      scale=scale, rows=rows)
    if inp.kv_scales is not None:
        return OA.paged_attention_u8(bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(),
                                     inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy(),
                                     scale=scale, rows=rows)
    return OA.paged_attention_bf16(bits(inp.q), bits(inp.kv_pool), inp.block_tables.numpy(),
                                   inp.ctx_lens.numpy(), inp.q_lens.numpy(), scale=scale, rows=rows)


def assert_close_rows(out: torch.Tensor, ref: dict, what: str = "") -> float:
    """Compare GPU rows out[t, h] with oracle rows, every element; returns the worst
    |err| / bound (a NaN or infinite output counts as a failure)."""
    o = out.detach().cpu().numpy().astype(np.float64)
    keys = list(ref.keys())
    if not keys:
        return 0.0
    t_idx = np.fromiter((k[0] for k in keys), dtype=np.int64, count=len(keys))
    h_idx = np.fromiter((k[1] for k in keys), dtype=np.int64, count=len(keys))
    r = np.stack([ref[k] for k in keys])
    err = np.abs(o[t_idx, h_idx] - r)
    ratio = err / (ATOL + RTOL * np.abs(r))
    ratio = np.where(np.isfinite(ratio), ratio, np.inf).max(axis=1)
    i = int(np.argmax(ratio))
    worst = float(ratio[i])
    assert worst <= 1.0, f"{what}: row {keys[i]} exceeds |err| <= {ATOL} + {RTOL}|ref| by x{worst:.3f}"
    return worst


def assert_full_parity(out: torch.Tensor, inp: workloads.AttnInputs, ref: dict, what: str = "") -> float:
    """Every (row, head) of the batch is in ``ref`` and every element of out is within the bar."""
    assert len(ref) == inp.total_q * inp.num_q_heads, f"{what}: oracle covers {len(ref)} pairs"
    worst = assert_close_rows(out, ref, what)
    print(f"{what}: {len(ref)} (row, head) pairs, worst |err|/bound {worst:.3f}", flush=True)
    return worst


@functools.lru_cache(maxsize=None)
def config_inputs(name: str, kv_format: str = "bf16") -> workloads.AttnInputs:
    return workloads.attention_config(name, kv_format=kv_format)


@functools.lru_cache(maxsize=4)
def config_oracle(name: str, kv_format: str = "bf16") -> dict:
    """The oracle's output for every (row, head) of a named workload (computed once per
    process, on the CPU, single-threaded NumPy; tree workloads under their tree masks)."""
    from oracle import attention as OA_
    inp = config_inputs(name, kv_format)
    tm = None if inp.tree_mask is None else inp.tree_mask.numpy()
    args = (inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy())
    if inp.fp8:
        return OA_.paged_attention_fp8(bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(), *args, tree_mask=tm)
    if inp.kv_scales is not None:
        return OA_.paged_attention_u8(bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(), *args, tree_mask=tm)
    return OA_.paged_attention_bf16(bits(inp.q), bits(inp.kv_pool), *args, tree_mask=tm)
