"""paged_attention_decode_noalloc: decode with the library's own scratch
workspace, for callers that cannot allocate (graph capture, serving loops).

Through the C ABI it must give exactly paged_attention_decode's output (same
kernels, same split) and the oracle's within the bf16 bar, on consecutive
calls of different sizes -- the second smaller than the first, then the first
again -- since every call shares the one scratch array and must leave its
completion counters zero for the next. A call whose workspace would exceed
the array is refused on the host, before anything is launched.
"""
import numpy as np
import pytest

from paged_kv_decode_reshape_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_reshape_amd as pkv
    import oracle
    from gpu_harness import DevicePool, assert_close, int_tensor, to_device, to_f32


def _oracle(step):
    pk = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    pv = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    oracle.append(pk, pv, step.cached_key.f32, step.cached_value.f32, step.cached_slots)
    oracle.append(pk, pv, step.new_key.f32, step.new_value.f32, step.new_slots)
    bt, cl = step.decode_inputs()
    return oracle.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale)


def _noalloc(pool, step, part):
    bt, cl = step.decode_inputs()
    out = torch.full((len(cl), step.num_q_heads, step.head_dim), 5.0, dtype=torch.bfloat16, device="cuda:0")
    pkv.paged_attention_decode_noalloc(pool.handle, 0, out, to_device(step.decode_query), int_tensor(bt),
                                       int_tensor(cl), len(cl), step.num_q_heads, bt.shape[1], step.scale, part)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("part", [0, 128])
def test_noalloc_equals_decode_on_consecutive_calls(part):
    # 96 sequences with the balanced split; 48 with 128-token partitions, whose
    # summaries (sequences x heads x partitions) must fit the scratch array
    nbig = 96 if part == 0 else 48
    big = W.custom("na_big", seed=1800, dtype="bf16", hq=32, hkv=8, d=128,
                   ctx=np.random.default_rng(1800).integers(1, 3000, size=nbig).tolist())
    small = W.custom("na_small", seed=1801, dtype="bf16", hq=8, hkv=2, d=64, ctx=[1, 70, 5, 900, 33])
    pools = {}
    for st in (big, small):
        pools[st.name] = DevicePool(st)
        pools[st.name].fill()
    first = None
    for st in (big, small, big):
        got = _noalloc(pools[st.name], st, part)
        ref = pools[st.name].decode(part)          # caller workspace
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), st.name
        assert_close(to_f32(got), _oracle(st), "bf16", st.name)
        if st is big:
            if first is None:
                first = got.clone()
            else:
                assert torch.equal(got.view(torch.int16), first.view(torch.int16))


def test_noalloc_refuses_a_workspace_past_the_scratch_array():
    # 256 sequences of up to 8192 tokens in 64-token partitions: ~545 MB of
    # partial summaries, far past the scratch array; refused on the host.
    h = pkv.kv_pool_create(1, 4096, 16, 8, 128, pkv.BF16, [256], [512])
    try:
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_attention_decode_noalloc(h, 0, 256, 256, 256, 256, 256, 32, 512, 0.1, 64)
        assert e.value.status == -4 and "scratch" in str(e.value)
    finally:
        pkv.kv_pool_destroy(h)
