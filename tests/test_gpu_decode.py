"""GPU parity of the KV append and paged decode attention against the CPU oracle.

Every call goes through the C-ABI library. Bar: append bit-exact; attention
|gpu - oracle| <= 2e-3 + 1e-2 |oracle| for bf16, <= 1e-5 for fp32.
"""
import numpy as np
import pytest

import oracle
from paged_kv_decode_reshape_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import full_refs
    from gpu_harness import COUNTER_BYTES, DevicePool, POISON_BITS, assert_close, int_tensor, to_device, to_f32


def oracle_decode(step, seqs=None, lens=None, tables=None, query=None, scale=None):
    pk = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim, np.float32)
    pv = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim, np.float32)
    oracle.append(pk, pv, step.cached_key.f32, step.cached_value.f32, step.cached_slots)
    oracle.append(pk, pv, step.new_key.f32, step.new_value.f32, step.new_slots)
    bt, cl = step.decode_inputs()
    bt = bt if tables is None else tables
    cl = cl if lens is None else lens
    q = step.decode_query.f32 if query is None else query
    return oracle.paged_decode(q, pk, pv, bt, cl, step.scale if scale is None else scale, seqs=seqs)


def run_and_check(step, partition_size=None, seqs=None):
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode(partition_size))
    torch.cuda.synchronize()
    ref = oracle_decode(step, seqs=seqs)
    idx = slice(None) if seqs is None else list(seqs)
    return assert_close(out[idx], ref[idx], step.dtype, step.name)


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_append_bit_exact(dtype, d):
    step = W.custom(f"app_{dtype}_{d}", seed=101, dtype=dtype, hq=4, hkv=2, d=d,
                    ctx=[1, 16, 17, 40, 100])
    # drop a few cached tokens: negative slots must be skipped
    step.cached_slots = step.cached_slots.copy()
    step.cached_slots[::7] = -1
    pool = DevicePool(step)
    pool.fill()
    kbits, vbits = pool.decode_pool()
    bits_dt = np.uint16 if dtype == "bf16" else np.uint32
    ref_k = np.full(kbits.shape, POISON_BITS[dtype], dtype=bits_dt)
    ref_v = np.full(vbits.shape, POISON_BITS[dtype], dtype=bits_dt)
    for vals_k, vals_v, slots in ((step.cached_key, step.cached_value, step.cached_slots),
                                  (step.new_key, step.new_value, step.new_slots)):
        keep = slots >= 0
        blk, off = slots[keep] // 16, slots[keep] % 16
        ref_k[blk, off] = vals_k.bits[keep].view(bits_dt)
        ref_v[blk, off] = vals_v.bits[keep].view(bits_dt)
    assert np.array_equal(kbits, ref_k)
    assert np.array_equal(vbits, ref_v)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_decode_tiny_fp32():
    step = W.tiny_fp32()
    run_and_check(step)
    run_and_check(step, partition_size=64)     # split every sequence longer than 64


@pytest.mark.parametrize("batch,context", W.QWEN_GRID)
def test_decode_qwen_grid(batch, context):
    run_and_check(W.qwen_layer(batch, context))


def check_full(kind, partition_size=None):
    """A full-size workload in the launch configuration bench.py times, every
    output row against the oracle."""
    step = full_refs.step(kind)
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode(partition_size))
    torch.cuda.synchronize()
    return assert_close(out, full_refs.decode_ref(kind), step.dtype, step.name)


def test_decode_llama8b_b256():
    """B = 256 Llama-8B-shaped layer, lognormal contexts, churned block
    tables, balanced split: all 256 x 32 output rows."""
    check_full("llama8b")


def test_decode_long_context_split():
    step = W.long_context()
    assert step.partition_size == 512
    run_and_check(step)


def test_decode_long_context_balanced():
    """The 8 x 32768-token step with the default balanced split: 64 rows over
    the GPU's resident waves, each row combined from dozens of pieces by the
    workgroup-shared reduction."""
    step = W.long_context()
    run_and_check(step, partition_size=0)


def test_decode_mixed_step_decode_part():
    """The 128 decodes of the mixed chunked-prefill step, every row."""
    check_full("mixed")


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (3, 1), (5, 1), (6, 2), (7, 1), (8, 1), (16, 2)])
def test_decode_group_sizes(hq, hkv):
    step = W.custom(f"g{hq}_{hkv}", seed=200 + hq, dtype="bf16", hq=hq, hkv=hkv, d=128,
                    ctx=[1, 15, 16, 17, 63, 64, 65, 300])
    run_and_check(step)
    run_and_check(step, partition_size=128)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128), ("f32", 64)])
def test_decode_dtypes_head_dims(dtype, d):
    step = W.custom(f"{dtype}{d}", seed=300 + d, dtype=dtype, hq=8, hkv=2, d=d,
                    ctx=[2, 33, 64, 129, 700])
    run_and_check(step)
    run_and_check(step, partition_size=64)


@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 8), (128, 8, 8), (128, 24, 8), (64, 64, 8), (128, 64, 8)])
def test_decode_in_launch_combine(d, hq, hkv):
    """1024 rows for about 2048 resident wavefronts (a row per eight waves or
    more, so the partition launch combines its split rows itself), 1..400
    tokens each: rows span two or three waves, and several hundred of them
    have every piece inside one four-wave workgroup (combined through LDS
    when G * D <= 512: the first four cases) while as many are cut between
    workgroups (combined through the workspace; the last case, G * D = 1024,
    takes that path for all)."""
    ctx = np.random.Generator(np.random.PCG64(700 + hq)).integers(1, 401, 128).tolist()
    step = W.custom(f"fc{d}_{hq}_{hkv}", seed=700 + hq, dtype="bf16", hq=hq, hkv=hkv, d=d, ctx=ctx)
    run_and_check(step)


def test_decode_balanced_batch_limit():
    """4096 sequences, the most the balanced split takes (its window prefix
    then fills 16 KiB of dynamic LDS beside the LDS partials), with empty
    and short contexts."""
    ctx = np.random.Generator(np.random.PCG64(760)).integers(0, 97, 4096).tolist()
    step = W.custom("b4096", seed=760, dtype="bf16", hq=4, hkv=1, d=128, ctx=ctx)
    run_and_check(step)


@pytest.mark.parametrize("part", [-1, 0, 64, 128, 192, 512])
def test_decode_partition_sizes_agree(part):
    step = W.custom("parts", seed=400, dtype="bf16", hq=8, hkv=2, d=128,
                    ctx=[1, 64, 65, 511, 512, 513, 1500, 3000], boost_k_fraction=0.05)
    run_and_check(step, partition_size=part)


def test_decode_empty_and_tiny_contexts():
    step = W.custom("empty", seed=500, dtype="bf16", hq=4, hkv=1, d=128, ctx=[0, 1, 0, 2, 17])
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode(64))
    ref = oracle_decode(step)
    assert np.array_equal(out[0], np.zeros_like(out[0])) and np.array_equal(out[2], out[0])
    assert_close(out, ref, "bf16", "empty")


def test_decode_context_one_is_exact():
    """ctx = 1: the output is the appended V row, bit for bit."""
    step = W.custom("one", seed=501, dtype="bf16", hq=8, hkv=2, d=128, ctx=[1, 1, 1])
    pool = DevicePool(step)
    pool.fill()
    out = pool.decode().view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(3):
        for i in range(8):
            assert np.array_equal(out[b, i], step.new_value.bits[b, i // 4])


def test_decode_block_permutation_bit_identical():
    step = W.custom("perm", seed=502, dtype="bf16", hq=8, hkv=2, d=128, ctx=[5, 16, 47, 300, 1000])
    pool = DevicePool(step)
    pool.fill()
    out1 = pool.decode(128).cpu()
    perm = np.random.default_rng(9).permutation(step.num_blocks)
    step2 = W.custom("perm", seed=502, dtype="bf16", hq=8, hkv=2, d=128, ctx=[5, 16, 47, 300, 1000])
    step2.block_tables = perm[step2.block_tables].astype(np.int32)
    step2.cached_slots = perm[step2.cached_slots // 16] * 16 + step2.cached_slots % 16
    step2.new_slots = perm[step2.new_slots // 16] * 16 + step2.new_slots % 16
    pool2 = DevicePool(step2)
    pool2.fill()
    out2 = pool2.decode(128).cpu()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_decode_aliased_tables_equal_outputs():
    """Two sequences whose tables point at the same blocks, with equal queries and
    lengths, give identical outputs (prefix sharing)."""
    step = W.custom("alias", seed=503, dtype="bf16", hq=8, hkv=2, d=128, ctx=[300, 50, 700])
    pool = DevicePool(step)
    pool.fill()
    bt, cl = step.decode_inputs()
    bt2 = np.concatenate([bt, bt[:1]]).astype(np.int32)
    cl2 = np.concatenate([cl, cl[:1]]).astype(np.int32)
    q = np.concatenate([step.decode_query.bits, step.decode_query.bits[:1]])
    qv = W.Values("bf16", q)
    out = pool.decode(128, query=to_device(qv), tables=bt2, lens=cl2).cpu()
    assert torch.equal(out[0].view(torch.int16), out[3].view(torch.int16))
    ref = oracle_decode(step, lens=cl2, tables=bt2, query=qv.f32)
    assert_close(to_f32(out), ref, "bf16", "alias")


def test_decode_large_scores_do_not_overflow():
    """scale = 3 gives scores of a few hundred: exp() overflows in fp32 unless the
    running maximum is right."""
    step = W.custom("big", seed=504, dtype="bf16", hq=8, hkv=2, d=128, ctx=[700, 1200, 90])
    pool = DevicePool(step)
    pool.fill()
    for part in (-1, 128):
        out = to_f32(pool.decode(part, scale=3.0))
        ref = oracle_decode(step, scale=3.0)
        assert_close(out, ref, "bf16", f"big part={part}")


def test_decode_poisoned_unused_entries():
    """Unused table entries point at a NaN block and last-block tails hold NaN;
    nothing leaks into the output (checked by assert_close's finiteness test)."""
    step = W.custom("poison", seed=505, dtype="bf16", hq=4, hkv=1, d=128, ctx=[1, 17, 33, 250])
    assert (step.block_tables[0, 1:] == step.poison_block).all()
    run_and_check(step)
    run_and_check(step, partition_size=64)


def test_decode_workspace_reuse_counters_return_to_zero():
    """One zero-filled workspace serves a run of decode calls of different
    batches, splits and variants. The completion counters at its start are
    zero after every call, and every output matches the oracle. The contexts
    make rows that span many wavefronts' shares and shares that are empty."""
    a = W.custom("ws_a", seed=520, dtype="bf16", hq=32, hkv=8, d=128, ctx=[3000, 1, 700, 5000, 64, 0, 129])
    rng = np.random.default_rng(521)
    b = W.custom("ws_b", seed=522, dtype="bf16", hq=8, hkv=2, d=64,
                 ctx=rng.integers(1, 2500, size=64).tolist())
    c = W.custom("ws_c", seed=523, dtype="bf16", hq=32, hkv=8, d=128, ctx=[900, 3, 4100], q_lens=[3, 3, 3])
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda:0")
    pools = {}
    for step in (a, b, c):
        pools[step.name] = DevicePool(step)
        pools[step.name].fill()
    refs = {a.name: oracle_decode(a), b.name: oracle_decode(b)}
    for step, part in [(a, 0), (b, 0), (a, 128), (b, -1), (a, 0), (b, 64), (b, 0)]:
        out = to_f32(pools[step.name].decode(part, ws=ws))
        torch.cuda.synchronize()
        assert not ws[:COUNTER_BYTES].any(), f"{step.name} part={part}: counters left non-zero"
        assert_close(out, refs[step.name], "bf16", f"{step.name} part={part}")
    # several query rows per sequence (combined by the separate reduction), then plain decode again
    out = to_f32(pools[c.name].decode_multi(3, 0, ws=ws))
    torch.cuda.synchronize()
    assert not ws[:COUNTER_BYTES].any()
    pk = oracle.new_pool(c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    pv = oracle.new_pool(c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
    oracle.append(pk, pv, c.cached_key.f32, c.cached_value.f32, c.cached_slots)
    oracle.append(pk, pv, c.new_key.f32, c.new_value.f32, c.new_slots)
    bt, cl = c.prefill_inputs()
    assert_close(out, oracle.paged_prefill_chunk(c.prefill_query.f32, c.cu_q_lens, pk, pv, bt, cl, c.scale),
                 "bf16", "multi")
    out = to_f32(pools[a.name].decode(0, ws=ws))
    torch.cuda.synchronize()
    assert not ws[:COUNTER_BYTES].any()
    assert_close(out, refs[a.name], "bf16", "a after multi")
