"""The bench's algorithmic byte counts (the numerator of roofline.achieved)
follow the KV-size formula the pages print in full: 2 (K and V) x KV heads x
head_dim x bytes per element for each cached token ("Inference Engineering,
Part 2", "The KV cache"), plus the query and output rows (CPU only)."""
import numpy as np

import bench
from paged_kv_decode_reshape_amd import workloads as W


def test_decode_bytes_follow_the_kv_formula():
    step = W.custom("acct", seed=3, dtype="bf16", hq=32, hkv=8, d=128, ctx=[1, 17, 300, 1000])
    ab = bench.algorithmic_bytes(step)
    tokens = int(step.context_lens.sum())
    assert ab["decode_kv"] == 2 * 8 * 128 * 2 * tokens
    assert ab["decode_qo"] == 2 * 4 * 32 * 128 * 2
    assert ab["append"] == 2 * 4 * 8 * 128 * (2 + 2)          # read new K, V rows + write them
    # e4m3 cache: one byte per cached element; queries, outputs and new rows stay bf16
    ab8 = bench.algorithmic_bytes(step, "fp8")
    assert ab8["decode_kv"] == ab["decode_kv"] // 2
    assert ab8["decode_qo"] == ab["decode_qo"]
    assert ab8["append"] == 2 * 4 * 8 * 128 * (2 + 1)


def test_shared_prefix_counts_each_prompt_once():
    groups = [(64, [70, 100, 64 + 33]), (0, [5])]
    step = W.shared_prefix("acct_sh", seed=4, dtype="bf16", hq=8, hkv=2, d=64, groups=groups)
    plain = bench.algorithmic_bytes(step)
    shared = bench.algorithmic_bytes(step, shared=True)
    per_token = 2 * 2 * 64 * 2
    assert plain["decode_kv"] == per_token * (70 + 100 + 97 + 5)
    assert shared["decode_kv"] == per_token * (64 + (70 - 64) + (100 - 64) + (97 - 64) + 5)


def test_prefill_flops_count_unmasked_pairs():
    # one 4-row chunk on 6 cached tokens: rows see 7, 8, 9, 10 keys
    step = W.custom("acct_pf", seed=5, dtype="bf16", hq=4, hkv=1, d=64, ctx=[10], q_lens=[4])
    ab = bench.algorithmic_bytes(step)
    assert ab["prefill_flops"] == 4 * 4 * 64 * (7 + 8 + 9 + 10)
