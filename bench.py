#!/usr/bin/env python3
"""Benchmark of the paged decode/verify attention step and the speculative verifier on one GPU.

Default run (one JSON line on stdout):
  * value: HBM GB/s of paged_attn_step on the Llama-3-8B-shaped decode batch (64 sequences,
    32 q / 8 kv heads, head_dim 128, 16-token blocks, lognormal context lengths), i.e. the
    algorithmic bytes of one step divided by its time, with K steps timed back to back;
  * verify step: paged_attn_step + spec_verify on the speculative-verify batch (16 sequences,
    q_len 5, vocab 128256) -> verified tokens/s and the verifier's own GB/s;
  * roofline: the attention kernel's average duration from HIP events recorded on its own
    stream (the library's kernel timer) against the 8 TB/s HBM peak;
  * logits_verify_step: spec_verify_logits on the verify batch's logits (temperature 1), beside
    torch's softmax followed by spec_verify;
  * kv_cache: kv_append of the decode batch's new rows (bf16 and 8-bit), append + attention
    back to back, and kv_commit of the tree step's accepted paths;
  * attention_configs: every attention workload (decode, verify, 70B share, mixed step, tree
    batch; bf16, 8-bit integer and FP8 KV) with its algorithmic bytes, step and kernel time, GB/s and
    fraction of the HBM peak;
  * spec_verify_sweep: spec_verify at vocabulary 128256 over batch sizes 16 .. 1024;
  * cpu_baseline: the fp64 CPU oracle on the same decode batch, on up to 16 host cores (forked
    workers, before the GPU is touched; the host's core count beside it), with the one-core
    rate, and the verifier oracle's tokens/s on one core.

Inputs are resident in HBM before timing starts.  The KV pool (and the verifier's
probability rows) are rotated over several device copies so that consecutive steps never
find their bytes in the 256 MB Infinity Cache.

Other modes: --mode copy (streaming copy kernel: the measured HBM ceiling), --mode attn-only /
verify-only (one kernel family, for profiling).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode/verify attention HBM GB/s (% of peak); verified tokens/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_llama3_8b_decode_traffic.txt")
KERNEL_SOURCES = ["verify_attention_paged_amd/csrc/attn_paged.hip",
                  "verify_attention_paged_amd/csrc/attn_internal.h",
                  "verify_attention_paged_amd/csrc/vap_common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------
# algorithmic bytes (what the method must move; no padding, no partials)
# ---------------------------------------------------------------------------------------

def attn_bytes(ctx_lens, q_lens, Hq, Hkv, D, bs) -> int:
    total = 0
    for L, Q in zip(ctx_lens, q_lens):
        L, Q = int(L), int(Q)
        total += 4 * L * Hkv * D          # K and V rows (bf16), each KV head once for all its rows
        total += 2 * Q * Hq * D           # q (bf16)
        total += 4 * Q * Hq * D           # out (fp32)
        total += 4 * ((L + bs - 1) // bs) + 8   # block ids and the two lengths
    return total


def attn_bytes_u8(ctx_lens, q_lens, Hq, Hkv, D, bs) -> int:
    """Algorithmic bytes of one step over an 8-bit KV cache: one code per K and V element,
    16 bytes of (scale, zero) pairs per token and KV head, q, out, block ids, lengths."""
    total = 0
    for L, Q in zip(ctx_lens, q_lens):
        total += 2 * L * Hkv * D + 16 * L * Hkv
        total += 2 * Q * Hq * D + 4 * Q * Hq * D
        total += 4 * ((L + bs - 1) // bs) + 8
    return total


def verify_bytes(n_accepted, k, V) -> int:
    total = 0
    for n in n_accepted:
        total += 8 * k + 4 * (k + 1) + 4 * k + 4 * (k + 2)   # gathers, uniforms, ids, outputs
        total += 8 * V if int(n) < k else 4 * V                 # residual row pair or bonus row
    return total


def kv_append_bytes(T, B, Hkv, D, u8) -> int:
    """New K and V rows read as bf16, written as bf16 or as codes + one (scale, zero) pair each,
    plus the lengths, the q_lens scan and one block id per row."""
    written = 2 * T * Hkv * D + 16 * T * Hkv if u8 else 4 * T * Hkv * D
    return 4 * T * Hkv * D + written + 8 * B + 4 * T


def kv_commit_bytes(n_moved, B, Hkv, D, u8) -> int:
    """Each moved row's K and V (and scales) read and written once, plus lengths, counts, paths."""
    row = (2 * Hkv * D + 16 * Hkv) if u8 else 4 * Hkv * D
    return 2 * n_moved * row + 16 * B


def logits_verify_bytes(n_accepted, temps, k, V) -> int:
    """Statistics pass: every target row, and the draft rows of sampled (T > 0) sequences, read
    once; verification: the gathers and the row pair (or bonus row) drawn from, read again."""
    total = 0
    for n, T in zip(n_accepted, temps):
        rows = (k + 1) + (k if T > 0 else 0)
        total += 4 * V * rows + 16 * rows
        total += 8 * k + 4 * (k + 1) + 4 * k + 4 * (k + 2) + 4
        if T > 0:
            total += 8 * V if n < k else 4 * V
    return total


def code_only(text: str) -> str:
    """C/C++ source with comments and blank lines removed, so that a comment edit does not
    count as a kernel change."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def tree_verify_bytes(parents, path, n_accepted, V) -> int:
    """Rows the tree walk must read: at every visited node where a child was rejected, its
    target and draft rows (8V); at the final node without a rejection, its target row (4V);
    plus the two gathered values per accept test, the tree, the uniforms and the outputs."""
    total = 0
    for par, pth, n in zip(parents, path, n_accepted):
        par = list(par)
        N = len(par)
        visited = [0] + [int(x) for x in pth[:int(n)]]
        tests = 0
        for i, u in enumerate(visited):
            kids = [c for c in range(1, N) if par[c] == u]
            if i < len(visited) - 1:
                rejected = sum(1 for c in kids if c < visited[i + 1])
                tests += rejected + 1
            else:
                rejected = len(kids)
                tests += rejected
            total += 8 * V if rejected else (4 * V if i == len(visited) - 1 else 0)
        total += 8 * tests + 12 * N + 8 * N + 4
    return total


def kernel_source_hash() -> str:
    """Fingerprint of the attention kernel's code (comments ignored); the committed counter
    summary is valid only for the fingerprint it records."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per attention launch from the committed counter summary, if it was taken on
    the current kernel source (else None)."""
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------------------
# device-side setup
# ---------------------------------------------------------------------------------------

def rotating_copies(t, min_bytes):
    """Enough device copies of `t` that cycling through them spans at least `min_bytes`."""
    import torch
    n = max(2, math.ceil(min_bytes / max(1, t.numel() * t.element_size())))
    return [t] + [t.clone() for _ in range(n - 1)]


def setup_attention(name, dev, kv_format="bf16"):
    """Device inputs of a named workload; the KV pool (and for 8-bit KV its scales) is copied
    until the copies span at least 1 GiB, so consecutive steps never hit in the 256 MB MALL."""
    import torch
    import workloads
    import verify_attention_paged_amd as vap
    inp = workloads.attention_config(name, kv_format=kv_format)
    d = dict(q=inp.q.to(dev), block_tables=inp.block_tables.to(dev), ctx_lens=inp.ctx_lens.to(dev),
             q_lens=inp.q_lens.to(dev))
    pools = rotating_copies(inp.kv_pool.to(dev), 1 << 30)
    scales = [inp.kv_scales.to(dev) for _ in pools] if inp.kv_scales is not None else None
    out = torch.empty(inp.q.shape, dtype=torch.float32, device=dev)
    ws = vap.attn_workspace(vap.attn_shape(d["q"], pools[0], d["block_tables"]), dev)
    size = attn_bytes_u8 if inp.kv_scales is not None else attn_bytes
    nbytes = size(inp.ctx_lens.tolist(), inp.q_lens.tolist(), inp.num_q_heads, inp.num_kv_heads,
                  inp.head_dim, inp.block_size)
    d["scales"] = scales
    d["tree_mask"] = inp.tree_mask.to(dev) if inp.tree_mask is not None else None
    d["fp8"] = inp.fp8
    return inp, d, pools, out, ws, nbytes


# Within a timed region, one step in TIMER_EVERY launches its kernels with the library's timer
# events (launch-stamped start/stop events): a launch that carries them also signals its
# completion, which cost about 4.6 us per decode step, so stamping every launch would time
# the instrumentation along with the step.  Kernel durations are the mean over the stamped
# launches of the same timed region.
TIMER_EVERY = 8


def time_loop(fn, steps, warmup, sample_timer=False):
    """Milliseconds per step over `steps` calls after `warmup` untimed ones (stream events
    around the loop), and the wall time.  With sample_timer, the library's kernel timer is on
    for steps 0, TIMER_EVERY, 2 TIMER_EVERY, ... of the timed loop only, and off afterwards."""
    import torch
    import verify_attention_paged_amd as vap
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        if sample_timer:
            vap.timer_enable(i % TIMER_EVERY == 0)
        fn(warmup + i)
    if sample_timer:
        vap.timer_enable(False)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / max(steps, 1), wall


def graph_loop(step, variants, steps, warmup, skip=False):
    """Milliseconds per step when each step is one HIP graph replay: step(j) is captured once
    for each of the `variants` rotating input copies (kernel timers off, after one eager call
    of each on a side stream) and step i replays graph i % variants.  Nothing in a step
    allocates or clears memory with memset nodes, so replays do exactly the eager work.  None
    when `skip`."""
    import torch
    if skip:
        return None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for j in range(variants):
            step(j)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for j in range(variants):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(j)
        graphs.append(g)
    torch.cuda.synchronize()
    ms, _ = time_loop(lambda i: graphs[i % variants].replay(), steps, warmup)
    del graphs
    torch.cuda.synchronize()
    return ms


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host's cores
# ---------------------------------------------------------------------------------------

_CPU_JOB = None   # (q bits, pool bits, tables, ctx_lens, q_lens, sequences per worker), shared by fork


def _cpu_worker(args):
    """One pool worker: the oracle on its share of the batch's sequences (a sub-batch with their
    query rows, block tables and lengths; the pool is shared), repeated until `budget_s` has
    passed; returns (shares done, seconds)."""
    import time as _t
    from threadpoolctl import threadpool_limits
    from oracle import attention as OA
    import numpy as np
    i, budget_s = args
    qb, pb, tables, L, Q, shares = _CPU_JOB
    seqs = shares[i]
    starts = np.concatenate([[0], np.cumsum(Q)])
    q_sub = np.concatenate([qb[starts[s]:starts[s + 1]] for s in seqs]) if seqs else qb[:0]
    t_sub, L_sub, Q_sub = tables[seqs], L[seqs], Q[seqs]
    done = 0
    t0 = _t.perf_counter()
    with threadpool_limits(1):
        while True:
            OA.paged_attention_bf16(q_sub, pb, t_sub, L_sub, Q_sub)
            done += 1
            if _t.perf_counter() - t0 >= budget_s:
                break
    return done, _t.perf_counter() - t0


def cpu_baseline_all_cores(inp, budget_s=10.0):
    """The oracle on all the host cores this benchmark may use (at most 16): each worker process
    takes a share of the batch's sequences (balanced by context length, all heads of a
    sequence together) and repeats it for about budget_s.  Must run before the process touches
    the GPU: the workers are forked."""
    import multiprocessing as mp
    import numpy as np
    import torch
    global _CPU_JOB
    P = max(1, min(16, os.cpu_count() or 1))
    L, Q = inp.ctx_lens.numpy(), inp.q_lens.numpy()
    load = [0.0] * P
    shares = [[] for _ in range(P)]
    share_bytes = [0] * P
    Hq, Hkv, D, bs = inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.block_size
    for s in sorted(range(len(L)), key=lambda s: -int(L[s]) * int(Q[s])):   # longest first
        w = int(np.argmin(load))
        load[w] += float(L[s]) * float(Q[s])
        shares[w].append(s)
        share_bytes[w] += attn_bytes([L[s]], [Q[s]], Hq, Hkv, D, bs)
    _CPU_JOB = (inp.q.view(torch.int16).numpy().view(np.uint16), inp.kv_pool.view(torch.int16).numpy().view(np.uint16),
                inp.block_tables.numpy(), L, Q, shares)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(P) as pool:
        res = pool.map(_cpu_worker, [(i, budget_s) for i in range(P)])
    wall = time.perf_counter() - t0
    _CPU_JOB = None
    # each worker's share of the algorithmic bytes times the shares it completed, over the
    # pool's wall time
    done_bytes = sum(share_bytes[i] * res[i][0] for i in range(P))
    return {"value": round(done_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": P, "kind": "oracle",
            "sample": f"whole {inp.name} batch split over {P} forked worker processes by context length "
                      f"(fp64 NumPy, 1 BLAS thread each), about {budget_s:.0f} s per worker, "
                      f"{wall:.1f} s wall"}


def cpu_baseline(inp, nbytes, budget_s=10.0):
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import attention as OA
    qb = inp.q.view(torch.int16).numpy().view(np.uint16)
    pb = inp.kv_pool.view(torch.int16).numpy().view(np.uint16)
    tables, L, Q = inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy()
    passes = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        while True:
            OA.paged_attention_bf16(qb, pb, tables, L, Q)
            passes += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes * passes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole {inp.name} batch ({inp.num_seqs} sequences, all {inp.num_q_heads} heads, "
                      f"fp64 NumPy, 1 BLAS thread), {passes} passes in {dt:.1f} s"}


# ---------------------------------------------------------------------------------------
# modes
# ---------------------------------------------------------------------------------------

def run_copy(args, dev):
    import torch
    import verify_attention_paged_amd as vap
    nbytes = args.copy_mib << 20
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dsts = [torch.empty_like(src) for _ in range(2)]
    ms, wall = time_loop(lambda i: vap.stream_copy(dsts[i % 2], src), args.steps, args.warmup)
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "ms_per_copy": round(ms, 5),
                      "GB_per_s": round(gbs, 2), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}))


def run_attention_only(args, dev, name):
    import verify_attention_paged_amd as vap
    inp, d, pools, out, ws, nbytes = setup_attention(name, dev, args.kv_format)
    sc = d["scales"]
    step = lambda i: vap.paged_attn_step(d["q"], pools[i % len(pools)], d["block_tables"], d["ctx_lens"],
                                         d["q_lens"], out=out, workspace=ws,
                                         kv_scales=None if sc is None else sc[i % len(pools)],
                                         tree_mask=d["tree_mask"], fp8=d["fp8"])
    vap.timer_enable(True)
    time_loop(step, 0, args.warmup)
    vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    ms, wall = time_loop(step, args.steps, 0, sample_timer=True)
    kms, cnt = vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    vap.timer_enable(False)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"mode": "attn-only", "workload": name, "kv_format": args.kv_format, "bytes": nbytes,
                      "ms_per_step": round(ms, 5),
                      "GB_per_s": round(gbs, 2), "kernel_ms": round(kms / max(cnt, 1), 5),
                      "kernel_GB_per_s": round(nbytes / (kms / max(cnt, 1) * 1e-3) / 1e9, 2)}))


ATTN_CONFIG_NAMES = ["llama3_8b_decode", "spec_verify_step", "llama70b_share", "mixed_step", "tree_verify_step"]


def measure_attention(name, dev, args, kv_format="bf16"):
    """One attention workload in the benchmark's launch configuration: K steps back to back
    (inputs resident, pools rotated past the MALL), the whole step (attention + combine
    kernels) by stream events and the attention kernel by the library's kernel timer."""
    import verify_attention_paged_amd as vap
    inp, d, pools, out, ws, nbytes = setup_attention(name, dev, kv_format)
    sc = d["scales"]
    step = lambda i: vap.paged_attn_step(d["q"], pools[i % len(pools)], d["block_tables"], d["ctx_lens"],
                                         d["q_lens"], out=out, workspace=ws,
                                         kv_scales=None if sc is None else sc[i % len(pools)],
                                         tree_mask=d["tree_mask"], fp8=d["fp8"])
    vap.timer_enable(True)
    time_loop(step, 0, args.warmup)
    vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    ms, _ = time_loop(step, args.steps, 0, sample_timer=True)
    kms, cnt = vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    vap.timer_enable(False)
    if vap.get_device_error(ws):
        raise RuntimeError(f"device reported a data error on {name} ({kv_format})")
    kms /= max(1, cnt)
    gbs, kgbs = nbytes / (ms * 1e-3) / 1e9, nbytes / (kms * 1e-3) / 1e9
    flops = sum(4 * inp.head_dim * inp.num_q_heads * sum(int(L) - int(Q) + i + 1 for i in range(int(Q)))
                for L, Q in zip(inp.ctx_lens.tolist(), inp.q_lens.tolist()))
    log(f"{name} ({kv_format}): step {ms * 1e3:.1f} us -> {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of peak); "
        f"attention kernel {kms * 1e3:.1f} us -> {kgbs:.0f} GB/s ({kgbs / HBM_PEAK_GBS:.3f})")
    del pools, sc
    return {"kv_format": kv_format, "seqs": inp.num_seqs, "rows": inp.total_q, "tokens": int(inp.ctx_lens.sum()),
            "bytes_per_step": nbytes, "flops_per_step": flops, "ms_per_step": round(ms, 5),
            "GB_per_s": round(gbs, 2), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "attention_kernel_ms": round(kms, 5), "kernel_GB_per_s": round(kgbs, 2),
            "kernel_frac_of_peak": round(kgbs / HBM_PEAK_GBS, 4),
            "rows_per_s": round(inp.total_q / (ms * 1e-3), 1)}


SWEEP_BATCHES = (16, 64, 256, 1024)


def spec_verify_sweep(dev, args):
    """spec_verify at vocabulary 128256, k = 4, over batch sizes: the verify batch's 16 sequences
    tiled B/16 times (same rows, so the same acceptance and bytes per sequence), probability
    rows rotated past the MALL."""
    import torch
    import verify_attention_paged_amd as vap
    import workloads
    ver = workloads.verify_config("spec_verify_step")
    res = {}
    for B in SWEEP_BATCHES:
        r = B // ver.num_seqs
        p = ver.p.to(dev).repeat(r, 1, 1)
        ps = rotating_copies(p, 768 << 20)
        qs = [ver.q.to(dev).repeat(r, 1, 1) for _ in ps]
        ids, uni = ver.draft_ids.to(dev).repeat(r, 1), ver.uniforms.to(dev).repeat(r, 1)
        out_ids = torch.empty((B, ver.k + 1), dtype=torch.int32, device=dev)
        n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
        ws = vap.verify_workspace(B, ver.k, ver.vocab, dev)
        step = lambda i: vap.spec_verify(ps[i % len(ps)], qs[i % len(qs)], ids, uni, out_ids, n_acc, workspace=ws)
        vap.timer_enable(True)
        time_loop(step, 0, args.warmup)
        vap.timer_read(vap.TIMER_VERIFY, reset=True)
        ms, _ = time_loop(step, args.steps, 0)   # every launch stamped: the kernel time is the figure here
        kms, cnt = vap.timer_read(vap.TIMER_VERIFY, reset=True)
        vap.timer_enable(False)
        kms /= max(1, cnt)
        n_host = n_acc.cpu().numpy()
        nbytes = verify_bytes(n_host, ver.k, ver.vocab)
        emitted = int((n_host + 1).sum())
        kgbs = nbytes / (kms * 1e-3) / 1e9
        log(f"spec_verify B={B}: kernel {kms * 1e3:.2f} us -> {kgbs:.0f} GB/s ({kgbs / HBM_PEAK_GBS:.3f} of peak), "
            f"{emitted / (kms * 1e-3) / 1e6:.1f} M tokens/s; {ms * 1e3:.2f} us per call")
        res[str(B)] = {"bytes": nbytes, "kernel_ms": round(kms, 5), "ms_per_call": round(ms, 5),
                       "kernel_GB_per_s": round(kgbs, 2), "kernel_frac_of_peak": round(kgbs / HBM_PEAK_GBS, 4),
                       "tokens_emitted": emitted, "tokens_per_s": round(emitted / (kms * 1e-3), 1)}
        del ps, qs, p
        torch.cuda.synchronize()
    return res


def cpu_verifier_baseline(budget_s=5.0):
    """The sequential fp64 verifier oracle on the verify batch (16 sequences, k 4, vocab 128256)
    on one core: tokens emitted per second and GB/s-equivalent of the same algorithmic bytes."""
    import numpy as np
    import workloads
    from threadpoolctl import threadpool_limits
    from oracle import spec_verify as OS
    ver = workloads.verify_config("spec_verify_step")
    p = ver.p.numpy().astype(np.float64)
    q = ver.q.numpy().astype(np.float64)
    ids, u = ver.draft_ids.numpy(), ver.uniforms.numpy().astype(np.float64)
    passes, emitted, nbytes = 0, 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        while True:
            _, n = OS.spec_verify(p, q, ids, u)
            passes += 1
            emitted += int((n + 1).sum())
            nbytes += verify_bytes(n, ver.k, ver.vocab)
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    return {"tokens_per_s": round(emitted / dt, 1), "GB_per_s": round(nbytes / dt / 1e9, 4), "cores": 1,
            "kind": "oracle",
            "sample": f"whole spec_verify_step batch (16 sequences, k 4, vocab 128256, fp64 NumPy, 1 BLAS "
                      f"thread), {passes} passes in {dt:.1f} s"}


def run_default(args, dev):
    import numpy as np
    import torch
    import verify_attention_paged_amd as vap
    import workloads

    # ---- decode step (the headline workload)
    inp, d, pools, out, ws, nbytes = setup_attention("llama3_8b_decode", dev)
    log(f"decode batch: {inp.num_seqs} seqs, {int(inp.ctx_lens.sum())} tokens, {nbytes / 1e6:.1f} MB/step, "
        f"{len(pools)} pool copies")
    step = lambda i: vap.paged_attn_step(d["q"], pools[i % len(pools)], d["block_tables"], d["ctx_lens"],
                                         d["q_lens"], out=out, workspace=ws)
    vap.timer_enable(True)
    time_loop(step, 0, args.warmup)
    vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    ms, wall = time_loop(step, args.steps, 0, sample_timer=True)
    kms_total, kcount = vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    if vap.get_device_error(ws):
        raise RuntimeError("device reported a data error on the decode batch")
    kernel_ms = kms_total / max(1, kcount)
    vap.timer_enable(False)
    gms = graph_loop(step, len(pools), args.steps, args.warmup, args.no_graphs)
    vap.timer_enable(True)
    value = nbytes / (ms * 1e-3) / 1e9
    kernel_gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    log(f"decode step {ms * 1e3:.1f} us -> {value:.1f} GB/s; attention kernel {kernel_ms * 1e3:.1f} us "
        f"-> {kernel_gbs:.1f} GB/s ({wall:.2f} s wall for {args.steps} steps)"
        + (f"; as HIP graph replays {gms * 1e3:.1f} us -> {nbytes / (gms * 1e-3) / 1e9:.1f} GB/s" if gms else ""))

    # ---- speculative verify step: attention (q_len 5) + spec_verify (vocab 128256)
    vinp, vd, vpools, vout, vws, vnbytes = setup_attention("spec_verify_step", dev)
    ver = workloads.verify_config("spec_verify_step")
    p = ver.p.to(dev)
    ps = rotating_copies(p, 768 << 20)
    qs = [ver.q.to(dev) for _ in range(len(ps))]
    ids, uni = ver.draft_ids.to(dev), ver.uniforms.to(dev)
    out_ids = torch.empty((ver.num_seqs, ver.k + 1), dtype=torch.int32, device=dev)
    n_acc = torch.empty((ver.num_seqs,), dtype=torch.int32, device=dev)
    sws = vap.verify_workspace(ver.num_seqs, ver.k, ver.vocab, dev)

    def vstep(i):
        vap.paged_attn_step(vd["q"], vpools[i % len(vpools)], vd["block_tables"], vd["ctx_lens"], vd["q_lens"],
                            out=vout, workspace=vws)
        vap.spec_verify(ps[i % len(ps)], qs[i % len(qs)], ids, uni, out_ids, n_acc, workspace=sws)

    time_loop(vstep, 0, args.warmup)
    vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    vap.timer_read(vap.TIMER_VERIFY, reset=True)
    vms, _ = time_loop(vstep, args.steps, 0, sample_timer=True)
    vattn_ms, c0 = vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    sv_ms, c1 = vap.timer_read(vap.TIMER_VERIFY, reset=True)
    vap.timer_enable(False)
    vgms = graph_loop(vstep, max(len(vpools), len(ps)), args.steps, args.warmup, args.no_graphs)
    n_host = n_acc.cpu().numpy()
    emitted = int((n_host + 1).sum())
    sv_bytes = verify_bytes(n_host, ver.k, ver.vocab)
    sv_kernel_ms = sv_ms / max(1, c1)
    verify_tok_s = emitted / (vms * 1e-3)
    log(f"verify step {vms * 1e3:.1f} us" + (f", as HIP graph replays {vgms * 1e3:.1f} us" if vgms else "") +
        f" ({emitted} tokens emitted, acceptance "
        f"{float(n_host.sum()) / (ver.k * ver.num_seqs):.3f}); spec_verify kernel {sv_kernel_ms * 1e3:.2f} us "
        f"-> {sv_bytes / (sv_kernel_ms * 1e-3) / 1e9:.1f} GB/s; verify attention kernel "
        f"{vattn_ms / max(1, c0) * 1e3:.1f} us -> {vnbytes / (vattn_ms / max(1, c0) * 1e-3) / 1e9:.1f} GB/s")

    # ---- tree verify step: tree-masked attention (16 x 16-node trees) + spec_verify_tree
    tinp, td, tpools, tout, tws, tnbytes = setup_attention("tree_verify_step", dev)
    tver = workloads.tree_verify_config("tree_verify_step")
    tmask = torch.from_numpy(np.concatenate([workloads.tree_masks(pr) for pr in tver.parents.numpy()])).to(dev)
    tps = rotating_copies(tver.p.to(dev), 768 << 20)
    tqs = [tver.q.to(dev) for _ in range(len(tps))]
    tpar, ttok, tuni = tver.parents.to(dev), tver.tokens.to(dev), tver.uniforms.to(dev)
    t_ids = torch.empty((tver.num_seqs, tver.num_nodes), dtype=torch.int32, device=dev)
    t_path = torch.empty_like(t_ids)
    t_n = torch.empty((tver.num_seqs,), dtype=torch.int32, device=dev)
    tvws = vap.tree_verify_workspace(tver.num_seqs, dev)

    def tstep(i):
        vap.paged_attn_step(td["q"], tpools[i % len(tpools)], td["block_tables"], td["ctx_lens"], td["q_lens"],
                            out=tout, workspace=tws, tree_mask=tmask)
        vap.spec_verify_tree(tps[i % len(tps)], tqs[i % len(tqs)], tpar, ttok, tuni, t_ids, t_path, t_n,
                             workspace=tvws)

    vap.timer_enable(True)
    time_loop(tstep, 0, args.warmup)
    vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    vap.timer_read(vap.TIMER_TREE_VERIFY, reset=True)
    vap.timer_read(vap.TIMER_TREE_DRAW, reset=True)
    tms, _ = time_loop(tstep, args.steps, 0, sample_timer=True)
    tattn_ms, tc0 = vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    tsv_ms, tc1 = vap.timer_read(vap.TIMER_TREE_VERIFY, reset=True)
    tdr_ms, tc2 = vap.timer_read(vap.TIMER_TREE_DRAW, reset=True)
    vap.timer_enable(False)
    tgms = graph_loop(tstep, max(len(tpools), len(tps)), args.steps, args.warmup, args.no_graphs)
    tn_host = t_n.cpu().numpy()
    t_emitted = int((tn_host + 1).sum())
    tsv_bytes = tree_verify_bytes(tver.parents.numpy(), t_path.cpu().numpy(), tn_host, tver.vocab)
    tsv_walk_ms = tsv_ms / max(1, tc1)
    tsv_draw_ms = tdr_ms / max(1, tc2)
    tsv_kernel_ms = tsv_walk_ms + tsv_draw_ms
    tree_tok_s = t_emitted / (tms * 1e-3)
    log(f"tree verify step {tms * 1e3:.1f} us" + (f", as HIP graph replays {tgms * 1e3:.1f} us" if tgms else "") +
        f" ({t_emitted} tokens emitted, {tn_host.mean():.2f} accepted per "
        f"sequence); tree attention kernel {tattn_ms / max(1, tc0) * 1e3:.1f} us; spec_verify_tree walk "
        f"{tsv_walk_ms * 1e3:.1f} us + draw {tsv_draw_ms * 1e3:.1f} us -> "
        f"{tsv_bytes / (tsv_kernel_ms * 1e-3) / 1e9:.1f} GB/s")

    # ---- decode step over an 8-bit KV cache (same lengths and shapes)
    qinp, qd, qpools, qout, qws, qnbytes = setup_attention("llama3_8b_decode", dev, kv_format="u8")
    qstep = lambda i: vap.paged_attn_step(qd["q"], qpools[i % len(qpools)], qd["block_tables"], qd["ctx_lens"],
                                          qd["q_lens"], out=qout, workspace=qws,
                                          kv_scales=qd["scales"][i % len(qpools)])
    vap.timer_enable(True)
    time_loop(qstep, 0, args.warmup)
    vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    qms, _ = time_loop(qstep, args.steps, 0, sample_timer=True)
    qk_total, qk_count = vap.timer_read(vap.TIMER_ATTENTION, reset=True)
    vap.timer_enable(False)
    if vap.get_device_error(qws):
        raise RuntimeError("device reported a data error on the 8-bit decode batch")
    qkernel_ms = qk_total / max(1, qk_count)
    log(f"8-bit KV decode step {qms * 1e3:.1f} us ({ms / qms:.2f}x the bf16 step) -> "
        f"{qnbytes / (qms * 1e-3) / 1e9:.1f} GB/s of {qnbytes / 1e6:.1f} MB; attention kernel "
        f"{qkernel_ms * 1e3:.1f} us -> {qnbytes / (qkernel_ms * 1e-3) / 1e9:.1f} GB/s")

    # ---- verification from logits (spec_verify_step logits, T = 1), and the unfused path
    lver = workloads.logits_verify_config("spec_verify_step")
    zps = rotating_copies(lver.zp.to(dev), 768 << 20)
    zqs = [lver.zq.to(dev) for _ in range(len(zps))]
    lids, luni, ltemps = lver.draft_ids.to(dev), lver.uniforms.to(dev), lver.temps.to(dev)
    l_out = torch.empty((lver.num_seqs, lver.k + 1), dtype=torch.int32, device=dev)
    l_n = torch.empty((lver.num_seqs,), dtype=torch.int32, device=dev)
    lws = vap.verify_logits_workspace(lver.num_seqs, lver.k, lver.vocab, dev)
    lstep = lambda i: vap.spec_verify_logits(zps[i % len(zps)], zqs[i % len(zqs)], lids, luni, ltemps, l_out, l_n,
                                             workspace=lws)
    vap.timer_enable(True)
    time_loop(lstep, 0, args.warmup)
    vap.timer_read(vap.TIMER_LOGIT_STATS, reset=True)
    vap.timer_read(vap.TIMER_VERIFY_LOGITS, reset=True)
    lms, _ = time_loop(lstep, args.steps, 0, sample_timer=True)
    st_ms, sc = vap.timer_read(vap.TIMER_LOGIT_STATS, reset=True)
    lv_ms, lc = vap.timer_read(vap.TIMER_VERIFY_LOGITS, reset=True)
    vap.timer_enable(False)
    if vap.get_device_error(lws):
        raise RuntimeError("device reported a data error in spec_verify_logits")
    ln_host = l_n.cpu().numpy()
    lbytes = logits_verify_bytes(ln_host, lver.temps.numpy(), lver.k, lver.vocab)
    stats_bytes = 4 * lver.vocab * (2 * lver.k + 1) * lver.num_seqs
    st_kernel, lv_kernel = st_ms / max(1, sc), lv_ms / max(1, lc)
    # the unfused alternative: probability rows written by torch's softmax, then spec_verify
    p_buf = torch.empty_like(zps[0])
    q_buf = torch.empty_like(zqs[0])
    uws = vap.verify_workspace(lver.num_seqs, lver.k, lver.vocab, dev)

    def ustep(i):
        torch.softmax(zps[i % len(zps)], dim=-1, out=p_buf)
        torch.softmax(zqs[i % len(zqs)], dim=-1, out=q_buf)
        vap.spec_verify(p_buf, q_buf, lids, luni, l_out, l_n, workspace=uws)

    time_loop(ustep, 0, args.warmup)
    ums, _ = time_loop(ustep, args.steps, 0)
    log(f"verify from logits: {lms * 1e3:.1f} us per call (statistics kernel {st_kernel * 1e3:.1f} us -> "
        f"{stats_bytes / (st_kernel * 1e-3) / 1e9:.0f} GB/s, verify kernel {lv_kernel * 1e3:.1f} us); "
        f"torch softmax + spec_verify {ums * 1e3:.1f} us")
    logits_line = {"workload": "spec_verify_step logits: 16 seqs, k 4, vocab 128256, target and draft logits fp32, "
                               "temperature 1",
                   "ms_per_call": round(lms, 5), "bytes": lbytes,
                   "stats_kernel_ms": round(st_kernel, 5), "stats_bytes": stats_bytes,
                   "stats_GB_per_s": round(stats_bytes / (st_kernel * 1e-3) / 1e9, 2),
                   "verify_kernel_ms": round(lv_kernel, 5),
                   "unfused_torch_softmax_plus_spec_verify_ms": round(ums, 5)}

    # ---- KV append (before attention) and commit (after verification)
    kinp = inp
    T, Hkv, D = kinp.total_q, kinp.num_kv_heads, kinp.head_dim
    k_new, v_new = (x.to(dev) for x in workloads.new_kv_rows(1, T, Hkv, D))
    kvws = vap.kv_workspace(dev)
    app = lambda i: vap.kv_append(k_new, v_new, pools[i % len(pools)], d["block_tables"], d["ctx_lens"],
                                  d["q_lens"], workspace=kvws)
    app8 = lambda i: vap.kv_append(k_new, v_new, qpools[i % len(qpools)], qd["block_tables"], qd["ctx_lens"],
                                   qd["q_lens"], kv_scales=qd["scales"][i % len(qpools)], workspace=kvws)

    def app_step(i):
        app(i)
        step(i)

    vap.timer_enable(True)
    res = {}
    for key, fn in (("bf16", app), ("u8", app8)):
        time_loop(fn, 0, args.warmup)
        vap.timer_read(vap.TIMER_KV_APPEND, reset=True)
        call_ms, _ = time_loop(fn, args.steps, 0, sample_timer=True)
        ktot, kcnt = vap.timer_read(vap.TIMER_KV_APPEND, reset=True)
        res[key] = (call_ms, ktot / max(1, kcnt))
    time_loop(app_step, 0, args.warmup)
    as_ms, _ = time_loop(app_step, args.steps, 0, sample_timer=True)
    # commit the tree step's accepted paths (as the tree verifier left them) on one tree pool
    out_lens = torch.empty_like(td["ctx_lens"])
    com = lambda i: vap.kv_commit(tpools[0], td["block_tables"], td["ctx_lens"], td["q_lens"], t_n, path=t_path,
                                  out_ctx_lens=out_lens, workspace=kvws)
    time_loop(com, 0, args.warmup)
    vap.timer_read(vap.TIMER_KV_COMMIT, reset=True)
    com_ms, _ = time_loop(com, args.steps, 0, sample_timer=True)
    ctot, ccnt = vap.timer_read(vap.TIMER_KV_COMMIT, reset=True)
    vap.timer_enable(False)
    if vap.get_device_error(kvws):
        raise RuntimeError("device reported a data error in kv_append / kv_commit")
    moved = sum(int(sum(1 for i in range(int(nn)) if tp[i] != i + 1)) for tp, nn in zip(t_path.cpu().numpy(), tn_host))
    ab = kv_append_bytes(T, kinp.num_seqs, Hkv, D, False)
    ab8 = kv_append_bytes(T, kinp.num_seqs, Hkv, D, True)
    cb = kv_commit_bytes(moved, tinp.num_seqs, tinp.num_kv_heads, tinp.head_dim, False)
    ckern = ctot / max(1, ccnt)
    log(f"kv_append decode batch: bf16 {res['bf16'][1] * 1e3:.2f} us kernel ({res['bf16'][0] * 1e3:.2f} us/call), "
        f"u8 {res['u8'][1] * 1e3:.2f} us kernel; append + attention {as_ms * 1e3:.1f} us vs attention alone "
        f"{ms * 1e3:.1f} us; kv_commit tree step {ckern * 1e3:.2f} us kernel ({moved} rows moved)")
    kv_line = {"workload": "kv_append of the llama3_8b_decode batch's 64 new rows (8 kv heads, head_dim 128), "
                           "bf16 and 8-bit; kv_commit of the tree_verify_step batch's accepted paths",
               "append_bf16_kernel_ms": round(res["bf16"][1], 5), "append_bf16_ms_per_call": round(res["bf16"][0], 5),
               "append_bf16_bytes": ab, "append_bf16_GB_per_s": round(ab / (res["bf16"][1] * 1e-3) / 1e9, 2),
               "append_u8_kernel_ms": round(res["u8"][1], 5), "append_u8_bytes": ab8,
               "decode_step_with_append_ms": round(as_ms, 5),
               "commit_tree_kernel_ms": round(ckern, 5), "commit_rows_moved": moved, "commit_bytes": cb}

    # ---- every attention workload in one table (configs 2-5 and the tree batch; bf16 and 8-bit)
    configs = {}
    if not args.no_configs:
        for nm in ATTN_CONFIG_NAMES:
            configs[nm] = measure_attention(nm, dev, args)
            if nm != "tree_verify_step":
                configs[nm + " u8"] = measure_attention(nm, dev, args, kv_format="u8")
                configs[nm + " fp8"] = measure_attention(nm, dev, args, kv_format="fp8")
    # ---- spec_verify over batch sizes (vocabulary 128256)
    sweep = spec_verify_sweep(dev, args) if not args.no_configs else None

    # ---- CPU baseline (oracle), rank 0 at N = 1 only
    cpu = None
    cpu_verify = None
    if not args.no_cpu_baseline:
        one = cpu_baseline(inp, nbytes, args.cpu_seconds)
        log(f"cpu oracle, 1 core: {one['value']} GB/s ({one['sample']})")
        cpu = dict(getattr(args, "cpu_all", None) or one)
        if cpu is not one and cpu.get("cores") != 1:
            log(f"cpu oracle, {cpu['cores']} cores: {cpu['value']} GB/s ({cpu['sample']})")
            cpu["single_core_value"] = one["value"]
            cpu["single_core_sample"] = one["sample"]
        cpu["host_cores"] = os.cpu_count()
        cpu_verify = cpu_verifier_baseline(min(5.0, args.cpu_seconds))
        log(f"cpu verifier oracle, 1 core: {cpu_verify['tokens_per_s']} tokens/s, {cpu_verify['GB_per_s']} GB/s")
        cpu["verifier"] = cpu_verify

    traffic = read_traffic()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "graph_ms_per_step": round(gms, 5) if gms else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_decode: 64 decode seqs, 32 q / 8 kv heads, head_dim 128, "
                               "block 16, ctx lognormal(1024, 1) in [16, 8192], pool 1.2x live blocks",
                   "tokens": int(inp.ctx_lens.sum()), "bytes_per_step": nbytes, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s_per_layer": round(inp.num_seqs / (ms * 1e-3), 1),
        "verified_tokens_per_s": round(verify_tok_s, 1),
        "verified_tokens_per_s_graph": round(emitted / (vgms * 1e-3), 1) if vgms else None,
        "verify_step": {"workload": "spec_verify_step: 16 seqs, q_len 5, 32/8 heads, head_dim 128, ctx "
                                    "uniform [512, 4096]; spec_verify vocab 128256, k 4",
                        "ms_per_step": round(vms, 5), "graph_ms_per_step": round(vgms, 5) if vgms else None,
                        "tokens_emitted": emitted,
                        "acceptance_rate": round(float(n_host.sum()) / (ver.k * ver.num_seqs), 4),
                        "sampler_tokens_per_s": round(emitted / (sv_kernel_ms * 1e-3), 1),
                        "attention_kernel_ms": round(vattn_ms / max(1, c0), 5),
                        "attention_GB_per_s": round(vnbytes / (vattn_ms / max(1, c0) * 1e-3) / 1e9, 2),
                        "spec_verify_kernel_ms": round(sv_kernel_ms, 5),
                        "spec_verify_GB_per_s": round(sv_bytes / (sv_kernel_ms * 1e-3) / 1e9, 2),
                        "spec_verify_bytes": sv_bytes},
        "tree_verify_step": {"workload": "tree_verify_step: 16 seqs verifying 16-node random token trees "
                                         "(tree-masked attention, 32/8 heads, head_dim 128, ctx uniform "
                                         "[512, 4096]) then spec_verify_tree over vocab 128256",
                             "ms_per_step": round(tms, 5), "graph_ms_per_step": round(tgms, 5) if tgms else None,
                             "tokens_emitted": t_emitted,
                             "mean_accepted": round(float(tn_host.mean()), 3),
                             "verified_tokens_per_s": round(tree_tok_s, 1),
                             "verified_tokens_per_s_graph": round(t_emitted / (tgms * 1e-3), 1) if tgms else None,
                             "attention_kernel_ms": round(tattn_ms / max(1, tc0), 5),
                             "spec_verify_tree_kernel_ms": round(tsv_kernel_ms, 5),
                             "spec_verify_tree_walk_ms": round(tsv_walk_ms, 5),
                             "spec_verify_tree_draw_ms": round(tsv_draw_ms, 5),
                             "spec_verify_tree_bytes": tsv_bytes},
        "kv8_decode_step": {"workload": "llama3_8b_decode with uint8 K/V codes and per-token (scale, zero) "
                                        "pairs, dequantised in the kernel",
                            "ms_per_step": round(qms, 5), "bytes_per_step": qnbytes,
                            "GB_per_s": round(qnbytes / (qms * 1e-3) / 1e9, 2),
                            "attention_kernel_ms": round(qkernel_ms, 5),
                            "speedup_vs_bf16_step": round(ms / qms, 3)},
        "kv_cache": kv_line,
        "logits_verify_step": logits_line,
        "attention_configs": configs or None,
        "spec_verify_sweep": sweep,
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "attn_main_kernel<128,16,1>",
                     "kernel_ms": round(kernel_ms, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["default", "copy", "attn-only", "verify-only"], default="default")
    ap.add_argument("--workload", default="llama3_8b_decode")
    ap.add_argument("--kv-format", choices=["bf16", "u8", "fp8"], default="bf16", help="KV cache format (attn-only mode)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graphs", action="store_true", help="skip the HIP graph timings (eager steps only)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload attention table and the spec_verify batch sweep")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the step has no cross-GPU part in this library "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    cpu_all = None
    if args.mode == "default" and not args.no_cpu_baseline:
        # the all-cores oracle leg forks its workers, so it runs before anything touches the GPU
        import workloads
        cpu_all = cpu_baseline_all_cores(workloads.attention_config("llama3_8b_decode"), args.cpu_seconds)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    args.cpu_all = cpu_all
    if args.mode == "copy":
        run_copy(args, dev)
    elif args.mode == "attn-only":
        run_attention_only(args, dev, args.workload)
    elif args.mode == "verify-only":
        run_verify_only(args, dev)
    else:
        run_default(args, dev)


def run_verify_only(args, dev):
    import torch
    import verify_attention_paged_amd as vap
    import workloads
    ver = workloads.verify_config("spec_verify_step")
    ps = rotating_copies(ver.p.to(dev), 768 << 20)
    qs = [ver.q.to(dev) for _ in range(len(ps))]
    ids, uni = ver.draft_ids.to(dev), ver.uniforms.to(dev)
    out_ids = torch.empty((ver.num_seqs, ver.k + 1), dtype=torch.int32, device=dev)
    n_acc = torch.empty((ver.num_seqs,), dtype=torch.int32, device=dev)
    sws = vap.verify_workspace(ver.num_seqs, ver.k, ver.vocab, dev)
    step = lambda i: vap.spec_verify(ps[i % len(ps)], qs[i % len(qs)], ids, uni, out_ids, n_acc, workspace=sws)
    vap.timer_enable(True)
    time_loop(step, 0, args.warmup)
    vap.timer_read(vap.TIMER_VERIFY, reset=True)
    ms, _ = time_loop(step, args.steps, 0, sample_timer=True)
    kms, cnt = vap.timer_read(vap.TIMER_VERIFY, reset=True)
    n = n_acc.cpu().numpy()
    nbytes = verify_bytes(n, ver.k, ver.vocab)
    print(json.dumps({"mode": "verify-only", "bytes": nbytes, "ms_per_call": round(ms, 5),
                      "kernel_ms": round(kms / max(cnt, 1), 5),
                      "kernel_GB_per_s": round(nbytes / (kms / max(cnt, 1) * 1e-3) / 1e9, 2)}))


if __name__ == "__main__":
    main()
