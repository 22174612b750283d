"""CPU oracle for paged decode/verify attention and speculative verification.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (``verify_attention_paged_amd``);
the two meet only through the seeded input generators in ``workloads/``.

The oracle is deliberately plain and slow: NumPy in float64, one query row or one sequence at a
time, written from the definitions on the source pages:

  [P1] "Continuous Batching and Speculative Decoding: How Modern LLM Serving Engines Actually
       Work" (syslabs.in)
  [P2] "Speculative Decoding and Continuous Batching for High-Throughput LLM Serving"
       (mohashari.github.io)
  [P3] the tempatgunting.com article on LLM inference optimisation and batching (untitled)
  [P4] "Continuous Batching & Speculative Decoding" (neuralmasteryai.com)
  [P5] "Continuous batching: how vLLM and friends keep GPUs fed" (martinuke0.github.io)

Modules:
  attention    -- paged KV address translation and causal softmax attention (fp64)
  spec_verify  -- sequential modified rejection sampling with residual resampling (fp64)
  tree_verify  -- the same rule walked over a draft token tree (fp64)
  logits_verify -- verification from logits: temperature, softmax (fp64), then spec_verify;
                  temperature 0 is the greedy (one-hot) limit
  kv_cache     -- writing new K/V rows into the paged pool (bf16 copy, 8-bit per-token
                  quantisation in fp32) and committing accepted draft tokens

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms, invariants the
pages fix, library routines and hand-worked fixtures under ``tests/golden/``.
"""

from . import attention, kv_cache, logits_verify, spec_verify, tree_verify  # noqa: F401
