"""GPU parity of decode over shared prefixes (paged_attention_decode_shared)
against the CPU oracle.

Sequences in a group share the physical blocks of a common prefix (parallel
sampling, a common system prompt; "The Serving Playbook", "Sharing is a
reference count"). Sharing changes how the work is organised, not what is
computed: every sequence's output is the oracle's decode over its own block
table. Bar: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| (bf16 queries and outputs,
fp32 accumulation). The step's pool starts NaN-filled, so a read of a slot no
sequence wrote, or of a table entry past a sequence's last block (they point
at a NaN block), would poison the output.
"""
import numpy as np
import pytest

import oracle
from oracle import fp8 as f8
from paged_kv_decode_reshape_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import full_refs
    from gpu_harness import DevicePool, assert_close, to_f32


def oracle_decode(step, seqs=None, k_scale=None, v_scale=None):
    pk = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    pv = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    for key, value, slots in ((step.cached_key, step.cached_value, step.cached_slots),
                              (step.new_key, step.new_value, step.new_slots)):
        k, v = key.f32, value.f32
        if k_scale is not None:
            k, v = f8.quantize_dequantize(k, k_scale), f8.quantize_dequantize(v, v_scale)
        oracle.append(pk, pv, k, v, slots)
    bt, cl = step.decode_inputs()
    return oracle.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale, seqs=seqs)


# Groups chosen to hit the edges: a prefix ending inside a block (copied per
# member), a group with more members than one wavefront's columns hold, a
# singleton whose whole context is one shared partition, empty and unshared
# sequences, and prefixes shorter than a partition.
GROUPS = [
    (40, [41, 60, 100]),
    (0, [5]),
    (256, [256]),
    (130, [131 + 7 * i for i in range(19)]),
    (640, [641, 700, 1000, 1500]),
    (1, [1, 2]),
    (0, [0]),
    (300, [301, 555]),
    (512, [513]),
]


def shared_step(name, seed, hq, hkv, d, groups=GROUPS):
    return W.shared_prefix(name, seed=seed, dtype="bf16", hq=hq, hkv=hkv, d=d, groups=groups)


@pytest.mark.parametrize("hq,hkv,d,part", [
    (32, 8, 128, 0), (32, 8, 128, 64), (8, 1, 128, 128), (6, 2, 128, 64),
    (4, 4, 64, 64), (16, 4, 64, 256), (14, 2, 64, 192), (10, 2, 128, 64)])
def test_shared_parity_bf16(hq, hkv, d, part):
    step = shared_step(f"sh{hq}_{hkv}_{d}_{part}", 900 + hq + d + part, hq, hkv, d)
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode_shared(part))
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(step), "bf16", step.name)


@pytest.mark.parametrize("hq,hkv,d,part", [(32, 8, 128, 0), (6, 2, 64, 64), (8, 8, 128, 128)])
def test_shared_parity_fp8(hq, hkv, d, part):
    step = shared_step(f"sh8_{hq}_{hkv}_{d}_{part}", 940 + hq + d + part, hq, hkv, d)
    ks, vs = 1.0 / 96, 1.0 / 32
    pool = DevicePool(step, kv="fp8", k_scales=[ks], v_scales=[vs])
    pool.fill()
    out = to_f32(pool.decode_shared(part))
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(step, k_scale=ks, v_scale=vs), "bf16", step.name)


def test_shared_without_sharing_equals_oracle():
    """Every sequence its own group with prefix 0: the prefix kernel does no
    attention work and the result is plain fixed-partition decode."""
    step = shared_step("sh_none", 961, 32, 8, 128)
    nseq = len(step.context_lens)
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode_shared(64, groups=np.arange(nseq + 1), prefix_lens=np.zeros(nseq)))
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(step), "bf16", step.name)


def test_shared_prefix_longer_than_a_member():
    """A prefix length past the contexts is clamped to the first member's
    context (its table supplies the shared block ids) and to each member's
    own. Here the clamped lengths' whole partitions (128 and 64 tokens) lie
    inside the blocks the members really share, so the result is still each
    sequence's own decode."""
    step = shared_step("sh_clamp", 962, 32, 8, 128, groups=[(130, [131, 140, 200]), (64, [65, 70])])
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode_shared(64, prefix_lens=[5000, 5000]))
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(step), "bf16", step.name)


def test_shared_repeat_and_reuse_workspace():
    """Two calls in a row with different groupings on one workspace give the
    same answer: the per-sequence shared counts are rewritten on every call."""
    step = shared_step("sh_rep", 963, 16, 4, 128)
    pool = DevicePool(step)
    pool.fill()
    a = to_f32(pool.decode_shared(64))
    nseq = len(step.context_lens)
    b = to_f32(pool.decode_shared(64, groups=np.arange(nseq + 1), prefix_lens=np.zeros(nseq)))
    torch.cuda.synchronize()
    ref = oracle_decode(step)
    assert_close(a, ref, "bf16", "grouped")
    assert_close(b, ref, "bf16", "ungrouped")


def test_parallel_sampling_step():
    """The B = 256 parallel-sampling step the bench times (32 prompts of 2000
    tokens x 8 samples, Llama-8B shapes), in the same launch configuration,
    every output row."""
    step = full_refs.step("parallel")
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode_shared(0))
    torch.cuda.synchronize()
    assert_close(out, full_refs.decode_ref("parallel"), "bf16", step.name)


def test_shared_empty_groups():
    """Empty groups (equal consecutive group starts), first and last among
    them, with large prefix lengths, change nothing: they have no members."""
    step = shared_step("sh_empty", 964, 32, 8, 128)
    gs, pl = step.info["group_starts"], step.info["prefix_lens"]
    new_gs, new_pl = [0], []
    for k in range(len(pl)):
        new_gs.append(int(gs[k]))                       # an empty group before each real one
        new_pl.append(4096)
        new_gs.append(int(gs[k + 1]))
        new_pl.append(int(pl[k]))
    new_gs.append(int(gs[-1]))                          # and an empty group at the end
    new_pl.append(4096)
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode_shared(64, groups=new_gs, prefix_lens=new_pl))
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(step), "bf16", step.name)
