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
    return d


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a CPU bf16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_rows(inp: workloads.AttnInputs, rows=None, scale=None) -> dict:
    if inp.kv_scales is not None:
        return OA.paged_attention_u8(bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(),
                                     inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy(),
                                     scale=scale, rows=rows)
    return OA.paged_attention_bf16(bits(inp.q), bits(inp.kv_pool), inp.block_tables.numpy(),
                                   inp.ctx_lens.numpy(), inp.q_lens.numpy(), scale=scale, rows=rows)


def assert_close_rows(out: torch.Tensor, ref: dict, what: str = "") -> float:
    """Compare GPU rows out[t, h] with oracle rows; returns the worst |err| / bound."""
    o = out.detach().cpu().numpy().astype(np.float64)
    worst = 0.0
    worst_key = None
    for (t, h), r in ref.items():
        err = np.abs(o[t, h] - r)
        bound = ATOL + RTOL * np.abs(r)
        ratio = float(np.max(err / bound))
        if not np.isfinite(ratio):
            ratio = np.inf
        if ratio > worst:
            worst, worst_key = ratio, (t, h)
    assert worst <= 1.0, f"{what}: row {worst_key} exceeds |err| <= {ATOL} + {RTOL}|ref| by x{worst:.3f}"
    return worst


def sample_rows(inp: workloads.AttnInputs, n: int, seed: int = 0):
    """(row, head) pairs to check at full size: every row of the longest and shortest sequences
    (all heads of one row), plus n random pairs; includes every verify/prefill edge row."""
    rng = np.random.default_rng(seed)
    L = inp.ctx_lens.numpy()
    Q = inp.q_lens.numpy()
    starts = np.concatenate([[0], np.cumsum(Q)])
    Hq = inp.num_q_heads
    picks = set()
    for s in (int(np.argmax(L)), int(np.argmin(L))):
        for h in range(Hq):
            picks.add((int(starts[s] + Q[s] - 1), h))
        picks.add((int(starts[s]), int(rng.integers(Hq))))
    for s in np.nonzero(Q > 1)[0][:6]:
        for i in (0, int(Q[s]) // 2, int(Q[s]) - 1):
            picks.add((int(starts[s] + i), int(rng.integers(Hq))))
    T = int(starts[-1])
    for _ in range(n):
        picks.add((int(rng.integers(T)), int(rng.integers(Hq))))
    return sorted(picks)


@functools.lru_cache(maxsize=None)
def config_inputs(name: str, kv_format: str = "bf16") -> workloads.AttnInputs:
    return workloads.attention_config(name, kv_format=kv_format)
