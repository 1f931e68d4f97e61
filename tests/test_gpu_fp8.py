"""GPU parity of the e4m3 (eight-bit) KV pool against the CPU oracle.

Every call goes through the C-ABI library with a PKV_FP8_E4M3 pool.
  * append: the stored codes equal the oracle's encoding of each bf16 input
    with the layer's 1/scale, bit for bit (saturation, subnormals, signed
    zero, NaN and infinity included);
  * decode and prefill: the output matches the oracle's attention over the
    values the pool stands for (decode(code) * scale, float64), to the bf16
    bar |gpu - oracle| <= 2e-3 + 1e-2 |oracle| (queries and outputs are bf16).
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
    from gpu_harness import DevicePool, POISON_BITS, assert_close, to_f32


def inv(scale):
    return np.float32(1.0) / np.float32(scale)


def oracle_pools(step, k_scale, v_scale):
    """Oracle pools holding the value each e4m3 code stands for."""
    pk = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    pv = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)
    for key, value, slots in ((step.cached_key, step.cached_value, step.cached_slots),
                              (step.new_key, step.new_value, step.new_slots)):
        oracle.append(pk, pv, f8.quantize_dequantize(key.f32, k_scale),
                      f8.quantize_dequantize(value.f32, v_scale), slots)
    return pk, pv


def fp8_pool(step, k_scale, v_scale):
    pool = DevicePool(step, kv="fp8", k_scales=[k_scale], v_scales=[v_scale])
    pool.fill()
    return pool


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

SPECIAL_BF16 = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x0000, 0x8000,   # NaN, inf, zeros
                         0x4600, 0xC600, 0x3700, 0xB700, 0x0001, 0x3C00],  # 8192, 2^-17, tiny, 2^-7
                        dtype=np.uint16)


def _with_specials(values: "W.Values", rng) -> "W.Values":
    bits = values.bits.copy().reshape(-1)
    pick = rng.choice(bits.size, size=min(bits.size, 4 * SPECIAL_BF16.size), replace=False)
    bits[pick] = np.resize(SPECIAL_BF16, pick.size)
    return W.Values("bf16", bits.reshape(values.bits.shape))


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_append_codes_bit_exact(d):
    step = W.custom(f"f8app{d}", seed=700 + d, dtype="bf16", hq=4, hkv=2, d=d,
                    ctx=[1, 16, 17, 40, 100])
    rng = np.random.default_rng(d)
    step.cached_key = _with_specials(step.cached_key, rng)
    step.cached_value = _with_specials(step.cached_value, rng)
    step.cached_slots = step.cached_slots.copy()
    step.cached_slots[::7] = -1                        # negative slots are skipped
    # two layers with their own scales; inputs x/scale run past 448 for the small scales
    scales = [(0.05, 3.0), (1.0, 1.0 / 96)]
    pool = DevicePool(step, num_layers=2, kv="fp8", k_scales=[s[0] for s in scales],
                      v_scales=[s[1] for s in scales])
    for layer in range(2):
        pool.fill(layer=layer)
    for layer, (ks, vs) in enumerate(scales):
        kbits, vbits = pool.decode_pool(layer)
        ref_k = np.full(kbits.shape, POISON_BITS["fp8"], dtype=np.uint8)
        ref_v = np.full(vbits.shape, POISON_BITS["fp8"], dtype=np.uint8)
        for vk, vv, slots in ((step.cached_key, step.cached_value, step.cached_slots),
                              (step.new_key, step.new_value, step.new_slots)):
            keep = slots >= 0
            blk, off = slots[keep] // 16, slots[keep] % 16
            ref_k[blk, off] = f8.fp8_e4m3_encode(vk.f32[keep], inv(ks))
            ref_v[blk, off] = f8.fp8_e4m3_encode(vv.f32[keep], inv(vs))
        for name, got, ref, src in (("K", kbits, ref_k, "key"), ("V", vbits, ref_v, "value")):
            bad = np.argwhere(got != ref)
            assert bad.size == 0, (f"layer {layer} {name}: {len(bad)} codes differ; first "
                                   + ", ".join(f"{tuple(i)} got {got[tuple(i)]:#04x} want {ref[tuple(i)]:#04x}"
                                               for i in bad[:6]))
        # the saturating cases were really exercised
        assert (kbits == 0x7E).any() and (kbits == 0xFE).any()


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def check_decode(step, k_scale, v_scale, partition_size=None, seqs=None):
    pool = fp8_pool(step, k_scale, v_scale)
    out = to_f32(pool.decode(partition_size))
    torch.cuda.synchronize()
    pk, pv = oracle_pools(step, k_scale, v_scale)
    bt, cl = step.decode_inputs()
    ref = oracle.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale, seqs=seqs)
    idx = slice(None) if seqs is None else list(seqs)
    return assert_close(out[idx], ref[idx], "bf16", step.name)


@pytest.mark.parametrize("hq,hkv,d,part", [
    (32, 8, 128, 0), (32, 8, 128, 128), (32, 8, 128, -1), (8, 2, 64, 0), (8, 2, 64, 64),
    (1, 1, 128, 0), (3, 1, 128, 0), (6, 2, 128, 64), (7, 1, 64, 0), (8, 1, 128, 0)])
def test_fp8_decode_parity(hq, hkv, d, part):
    step = W.custom(f"f8dec{hq}_{hkv}_{d}", seed=710 + hq + d, dtype="bf16", hq=hq, hkv=hkv, d=d,
                    ctx=[1, 15, 16, 17, 63, 64, 65, 300, 1000])
    check_decode(step, 1.0 / 96, 1.0 / 32, partition_size=part)


@pytest.mark.parametrize("batch,cmax", [(256, 200), (640, 100)])
def test_fp8_decode_in_launch_combine(batch, cmax):
    """Enough rows for the partition launch to combine its split rows itself.
    At 256 sequences the partials of rows held by one workgroup fit in LDS
    beside the window prefix at three workgroups per CU, and those rows meet
    there; at 640 the prefix leaves no room, and every split row goes through
    the workspace. Both give the oracle's result."""
    ctx = np.random.Generator(np.random.PCG64(761 + batch)).integers(1, cmax + 1, batch).tolist()
    step = W.custom(f"f8fc{batch}", seed=761 + batch, dtype="bf16", hq=8, hkv=2, d=128, ctx=ctx)
    check_decode(step, 1.0 / 96, 1.0 / 32)


def test_fp8_decode_unit_scales():
    """Scale 1: inputs near zero land on subnormal codes."""
    step = W.custom("f8dec_unit", seed=720, dtype="bf16", hq=8, hkv=2, d=128, ctx=[5, 77, 400])
    check_decode(step, 1.0, 1.0)


def test_fp8_decode_llama8b_b256():
    """The B=256 lognormal-length Llama-8B layer with an e4m3 pool (the
    scales bench.py --kv-dtype fp8 uses), every output row."""
    step = full_refs.step("llama8b")
    pool = fp8_pool(step, 1.0 / 80, 1.0 / 80)
    out = to_f32(pool.decode())
    torch.cuda.synchronize()
    assert_close(out, full_refs.decode_ref("llama8b", 1.0 / 80, 1.0 / 80), "bf16", step.name)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def check_prefill(step, k_scale, v_scale, rows=None):
    pool = fp8_pool(step, k_scale, v_scale)
    out = to_f32(pool.prefill())
    torch.cuda.synchronize()
    pk, pv = oracle_pools(step, k_scale, v_scale)
    bt, cl = step.prefill_inputs()
    ref = oracle.paged_prefill_chunk(step.prefill_query.f32, step.cu_q_lens, pk, pv, bt, cl,
                                     step.scale, rows=rows)
    idx = slice(None) if rows is None else list(rows)
    return assert_close(out[idx], ref[idx], "bf16", step.name)


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 128), (8, 2, 128), (8, 1, 64), (16, 2, 64), (2, 2, 128)])
def test_fp8_prefill_ragged_chunks(hq, hkv, d):
    ctx = [1, 20, 16, 100, 33, 130, 64, 257]
    q_lens = [1, 15, 16, 17, 33, 100, 64, 40]
    step = W.custom(f"f8pf{hq}_{hkv}_{d}", seed=730 + hq + d, dtype="bf16", hq=hq, hkv=hkv, d=d,
                    ctx=ctx, q_lens=q_lens)
    check_prefill(step, 1.0 / 96, 1.0 / 32)


def test_fp8_mixed_step():
    """The mixed chunked-prefill step with an e4m3 pool: the 512-token chunk
    and the 128 decodes, every output row."""
    step = full_refs.step("mixed")
    pool = fp8_pool(step, 1.0 / 80, 1.0 / 80)
    dec = to_f32(pool.decode())
    pre = to_f32(pool.prefill())
    torch.cuda.synchronize()
    ref_dec, ref_pre = full_refs.refs("mixed", 1.0 / 80, 1.0 / 80)
    assert_close(dec, ref_dec, "bf16", step.name + " decode")
    assert_close(pre, ref_pre, "bf16", step.name + " chunk")
