"""GPU parity of decode with several query rows per sequence
(paged_attention_decode_multi) against the CPU oracle.

Row j of a sequence with T rows and context ctx sits at position ctx - T + j
and attends causally to keys 0 .. ctx - T + j: the oracle's prefill-chunk
attention with every chunk of length T. Bar: |gpu - oracle| <= 2e-3 +
1e-2 |oracle| (bf16 queries and outputs, fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
from oracle import fp8 as f8
from paged_kv_decode_reshape_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_reshape_amd as pkv
    from gpu_harness import DevicePool, assert_close, int_tensor, to_device, to_f32


def oracle_multi(step, k_scale=None, v_scale=None, rows=None):
    pk = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    pv = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    for key, value, slots in ((step.cached_key, step.cached_value, step.cached_slots),
                              (step.new_key, step.new_value, step.new_slots)):
        k, v = key.f32, value.f32
        if k_scale is not None:
            k, v = f8.quantize_dequantize(k, k_scale), f8.quantize_dequantize(v, v_scale)
        oracle.append(pk, pv, k, v, slots)
    bt, cl = step.prefill_inputs()
    return oracle.paged_prefill_chunk(step.prefill_query.f32, step.cu_q_lens, pk, pv, bt, cl, step.scale,
                                      rows=rows)


def multi_step(name, seed, hq, hkv, d, tq, ctx):
    ctx = [c for c in ctx if c >= tq]
    return W.custom(name, seed=seed, dtype="bf16", hq=hq, hkv=hkv, d=d, ctx=ctx, q_lens=[tq] * len(ctx))


@pytest.mark.parametrize("hq,hkv,d,tq,part", [
    (32, 8, 128, 4, 0), (32, 8, 128, 2, 128), (32, 8, 128, 3, -1), (8, 1, 128, 2, 0),
    (4, 4, 64, 16, 0), (4, 4, 64, 16, 64), (6, 2, 128, 5, 0), (16, 4, 64, 4, 0)])
def test_multi_parity_bf16(hq, hkv, d, tq, part):
    step = multi_step(f"mq{hq}_{hkv}_{d}_{tq}", 800 + hq + d + tq, hq, hkv, d, tq,
                      [1, 2, 5, 15, 16, 17, 63, 64, 65, 300, 1000])
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode_multi(tq, part))
    torch.cuda.synchronize()
    assert_close(out, oracle_multi(step), "bf16", step.name)


@pytest.mark.parametrize("hq,hkv,d,tq,part", [(32, 8, 128, 4, 0), (6, 2, 128, 5, 64), (8, 8, 64, 8, -1)])
def test_multi_parity_fp8(hq, hkv, d, tq, part):
    step = multi_step(f"mq8_{hq}_{hkv}_{d}_{tq}", 820 + hq + d + tq, hq, hkv, d, tq,
                      [4, 9, 16, 33, 64, 129, 700])
    ks, vs = 1.0 / 96, 1.0 / 32
    pool = DevicePool(step, kv="fp8", k_scales=[ks], v_scales=[vs])
    pool.fill()
    out = to_f32(pool.decode_multi(tq, part))
    torch.cuda.synchronize()
    assert_close(out, oracle_multi(step, ks, vs), "bf16", step.name)


def test_multi_one_row_is_decode():
    """queries_per_seq = 1 gives paged_attention_decode's output, bit for bit."""
    step = multi_step("mq1", 840, 32, 8, 128, 1, [1, 17, 64, 65, 900, 2000])
    pool = DevicePool(step)
    pool.fill()
    a = pool.decode_multi(1, 0)
    bt, cl = step.prefill_inputs()
    b = pool.decode(0, query=to_device(step.prefill_query), tables=bt, lens=cl)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_multi_llama8b_b256_lognormal():
    """B=256 Llama-8B-shaped layer, lognormal contexts, 4 query rows each:
    every output row."""
    rng = np.random.default_rng(7)
    ctx = W.lognormal_lengths(rng, 256).astype(int).tolist()
    step = multi_step("mq_llama", 850, 32, 8, 128, 4, ctx)
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.decode_multi(4, 0))
    torch.cuda.synchronize()
    assert_close(out, oracle_multi(step), "bf16", step.name)


@pytest.mark.parametrize("hq,hkv,tq,kv", [
    (32, 8, 5, "bf16"), (32, 8, 6, "bf16"), (32, 8, 7, "bf16"), (32, 8, 8, "bf16"),
    (64, 8, 3, "bf16"), (64, 8, 4, "bf16"), (32, 8, 8, "fp8"), (64, 8, 3, "fp8"), (16, 16, 17, "bf16")])
def test_multi_more_rows_than_one_tile(hq, hkv, tq, kv):
    """queries_per_seq x (query heads per KV head) > 16: the rows of a
    sequence run as an equal-length chunk on the prefill-chunk kernel.
    Speculative verification of up to 7 draft tokens at G = 4 and 3 at G = 8;
    an empty context gives zero rows."""
    ctx = [0, tq, tq + 1, 16, 17, 63, 64, 65, 300, 1000, 2500]
    step = W.custom(f"mq_big{hq}_{hkv}_{tq}_{kv}", seed=870 + hq + tq, dtype="bf16", hq=hq, hkv=hkv, d=128,
                    ctx=[c for c in ctx if c >= tq], q_lens=[tq] * len([c for c in ctx if c >= tq]))
    ks, vs = (1.0 / 96, 1.0 / 32) if kv == "fp8" else (None, None)
    pool = DevicePool(step, kv=kv, k_scales=None if ks is None else [ks], v_scales=None if vs is None else [vs])
    pool.fill()
    out = to_f32(pool.decode_multi(tq, 0))
    torch.cuda.synchronize()
    assert_close(out, oracle_multi(step, ks, vs), "bf16", step.name)
    # an empty context: zero rows
    bt, cl = step.prefill_inputs()
    cl0 = cl.copy()
    cl0[0] = 0
    q = to_device(step.prefill_query)
    nseq = len(cl)
    o2 = torch.full((nseq * tq, hq, 128), 3.0, dtype=torch.bfloat16, device="cuda:0")
    pkv.paged_attention_decode_multi(pool.handle, 0, o2, q, tq, int_tensor(bt), int_tensor(cl0), nseq, hq,
                                     bt.shape[1], step.scale, 0, None, 0)
    torch.cuda.synchronize()
    assert (o2[:tq].float() == 0).all()
    assert_close(to_f32(o2[tq:]), out[tq:], "bf16", "rows after the empty context")
