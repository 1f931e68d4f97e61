"""paged_attention_decode_append (append and decode in one call) against the
two-call sequence reshape_and_cache + paged_attention_decode, and against the
oracle.

Each sequence's new token sits at position context_lens[b] - 1, its slot given
by the block table. The fused call must leave the pool bit-identical to the
append (bf16 bits, or e4m3 codes) and produce bit-identical outputs; both
must match the oracle's decode to the bf16 bar |gpu - oracle| <= 2e-3 +
1e-2 |oracle|.
"""
import numpy as np
import pytest

import oracle
from oracle import fp8 as f8
from paged_kv_decode_reshape_amd import workloads as W
import paged_kv_decode_reshape_amd as pkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_harness import DEV, TORCH_DT, DevicePool, assert_close, int_tensor, raw_bits, to_device, to_f32


def _fused(pool, step, part):
    s = step
    bt, cl = s.decode_inputs()
    nseq = len(cl)
    out = torch.empty((nseq, s.num_q_heads, s.head_dim), dtype=TORCH_DT[s.dtype], device=DEV)
    wsb = pkv.paged_attention_decode_workspace_bytes(pool.handle, nseq, s.num_q_heads, bt.shape[1], part)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=DEV)
    # the step's new rows in sequence order (one per sequence with ctx >= 1)
    hkv, d = s.num_kv_heads, s.head_dim
    k = np.zeros((nseq, hkv, d), np.uint16)
    v = np.zeros((nseq, hkv, d), np.uint16)
    live = np.flatnonzero(cl > 0)
    assert len(live) == len(s.new_slots)
    k[live], v[live] = s.new_key.bits, s.new_value.bits
    pkv.paged_attention_decode_append(pool.handle, 0, out, to_device(s.decode_query),
                                      to_device(W.Values("bf16", k)), to_device(W.Values("bf16", v)),
                                      int_tensor(bt), int_tensor(cl), nseq, s.num_q_heads, bt.shape[1], s.scale,
                                      part, ws, wsb)
    return out


def _check(step, kv, part):
    ks, vs = 1.0 / 96, 1.0 / 32
    mk = (lambda: DevicePool(step, kv="fp8", k_scales=[ks], v_scales=[vs])) if kv == "fp8" else \
        (lambda: DevicePool(step))
    two, one = mk(), mk()
    two.fill()
    ref_out = to_f32(two.decode(part))
    one.fill(include_new=False)
    got = to_f32(_fused(one, step, part))
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(one.k[0]), raw_bits(two.k[0])), "K pool differs from the append"
    assert np.array_equal(raw_bits(one.v[0]), raw_bits(two.v[0])), "V pool differs from the append"
    assert np.array_equal(got, ref_out), "outputs differ from append + decode"
    return got, ks, vs


@pytest.mark.parametrize("kv,hq,hkv,d,part,bs", [
    ("bf16", 32, 8, 128, 0, 16), ("bf16", 32, 8, 128, 128, 16), ("bf16", 12, 2, 128, 512, 16),
    ("bf16", 8, 8, 64, -1, 16), ("bf16", 12, 2, 128, -1, 16), ("bf16", 32, 8, 128, 0, 32),
    ("fp8", 32, 8, 128, 0, 16), ("fp8", 6, 2, 64, 64, 16), ("fp8", 64, 8, 128, -1, 32)])
def test_fused_append_matches_two_calls(kv, hq, hkv, d, part, bs):
    ctx = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 257, 700, 1500]
    step = W.custom(f"fuse_{kv}_{hq}_{d}_{part}_{bs}", seed=1600 + hq + d + bs, dtype="bf16", hq=hq, hkv=hkv,
                    d=d, ctx=ctx, block_size=bs)
    got, ks, vs = _check(step, kv, part)
    pk = oracle.new_pool(step.num_blocks, step.block_size, hkv, d)
    pv = oracle.new_pool(step.num_blocks, step.block_size, hkv, d)
    for key, value, slots in ((step.cached_key, step.cached_value, step.cached_slots),
                              (step.new_key, step.new_value, step.new_slots)):
        kk, vv = key.f32, value.f32
        if kv == "fp8":
            kk, vv = f8.quantize_dequantize(kk, ks), f8.quantize_dequantize(vv, vs)
        oracle.append(pk, pv, kk, vv, slots)
    bt, cl = step.decode_inputs()
    assert_close(got, oracle.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale), "bf16", step.name)


@pytest.mark.parametrize("batch,context,part", [(16, 128, -1), (16, 512, 0)])
def test_fused_append_qwen_step(batch, context, part):
    """Small Qwen-shaped steps in the launch configurations bench.py
    --config 2 --fused-append times."""
    _check(W.qwen_layer(batch, context), "bf16", part)


def test_fused_append_llama8b_step():
    """The B = 256 lognormal step."""
    _check(W.llama8b_continuous(), "bf16", 0)
