"""CPU checks of the benchmark's byte accounting and of its counter-summary fingerprint.

The roofline fraction that bench.py reports divides these algorithmic byte counts by a
measured kernel time, so each formula is checked here against a sum of the sizes of the
arrays the operation must read or write (numpy nbytes of arrays with the tensors' shapes and
dtypes), not against a retyped copy of the formula.
"""

import numpy as np
import pytest

import bench
import workloads
from workloads import generate as G


def _attn_touched_bytes(ctx_lens, q_lens, Hq, Hkv, D, bs, kv_dtype=np.uint16, scales=False):
    total = 0
    for L, Q in zip(ctx_lens, q_lens):
        L, Q = int(L), int(Q)
        k = np.empty((L, Hkv, D), dtype=kv_dtype)         # this sequence's K rows
        v = np.empty((L, Hkv, D), dtype=kv_dtype)         # and V rows
        q = np.empty((Q, Hq, D), dtype=np.uint16)         # bf16 query rows
        out = np.empty((Q, Hq, D), dtype=np.float32)      # fp32 output rows
        table = np.empty(-(-L // bs), dtype=np.int32)     # block ids actually used
        lens = np.empty(2, dtype=np.int32)                # ctx_len and q_len
        total += k.nbytes + v.nbytes + q.nbytes + out.nbytes + table.nbytes + lens.nbytes
        if scales:
            total += np.empty((L, Hkv, 4), dtype=np.float32).nbytes   # (scale, zero) of K and of V
    return total


@pytest.mark.parametrize("name", ["tiny", "llama3_8b_decode", "spec_verify_step", "llama70b_share", "mixed_step"])
def test_attention_bytes_match_the_arrays_touched(name):
    L, Q, (Hq, Hkv, D, bs, _) = G.config_lengths(name)
    assert bench.attn_bytes(L, Q, Hq, Hkv, D, bs) == _attn_touched_bytes(L, Q, Hq, Hkv, D, bs)
    assert bench.attn_bytes_u8(L, Q, Hq, Hkv, D, bs) == _attn_touched_bytes(L, Q, Hq, Hkv, D, bs,
                                                                             kv_dtype=np.uint8, scales=True)


def test_decode_batch_bytes_are_the_documented_figure():
    # 64 sequences, 79095 cached tokens, 8 KV heads of 128 dims: the per-launch figure that the
    # roofline line and the traffic summary quote
    L, Q, (Hq, Hkv, D, bs, _) = G.config_lengths("llama3_8b_decode")
    assert int(np.sum(L)) == 79095
    assert bench.attn_bytes(L, Q, Hq, Hkv, D, bs) == 325566396


def test_verify_bytes_match_the_arrays_touched():
    rng = np.random.default_rng(3)
    k, V = 4, 1000
    n = rng.integers(0, k + 1, size=32)
    total = 0
    for ni in n:
        gathers = np.empty(2 * k, dtype=np.float32)        # p(x_i) and q(x_i)
        uniforms = np.empty(k + 1, dtype=np.float32)
        ids = np.empty(k, dtype=np.int32)
        outs = np.empty(k + 2, dtype=np.int32)             # k + 1 emitted ids and the count
        rows = np.empty((2 if ni < k else 1, V), dtype=np.float32)   # residual pair or bonus row
        total += gathers.nbytes + uniforms.nbytes + ids.nbytes + outs.nbytes + rows.nbytes
    assert bench.verify_bytes(n, k, V) == total


def test_kernel_fingerprint_ignores_comments_only():
    src = "int f(int x) {\n  // double it\n  return 2 * x; /* twice */\n}\n"
    assert bench.code_only(src) == bench.code_only(src.replace("double it", "twice x"))
    assert bench.code_only(src) != bench.code_only(src.replace("2 * x", "3 * x"))


def test_traffic_is_read_only_for_the_current_kernel(tmp_path, monkeypatch):
    good = tmp_path / "traffic.txt"
    good.write_text("# header\nhbm_bytes_per_launch = 12345\n"
                    f"kernel_source_sha256_16 = {bench.kernel_source_hash()}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.read_traffic() == 12345.0
    stale = tmp_path / "stale.txt"
    stale.write_text("hbm_bytes_per_launch = 12345\nkernel_source_sha256_16 = 0000000000000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic() is None

