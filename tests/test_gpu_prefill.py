"""GPU parity of the MFMA prefill-chunk kernel against the CPU oracle.

Bar: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
from paged_kv_decode_reshape_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import full_refs
    from gpu_harness import DevicePool, assert_close, to_device, to_f32


def oracle_prefill(step, rows=None):
    pk = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim, np.float32)
    pv = oracle.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim, np.float32)
    oracle.append(pk, pv, step.cached_key.f32, step.cached_value.f32, step.cached_slots)
    oracle.append(pk, pv, step.new_key.f32, step.new_value.f32, step.new_slots)
    bt, cl = step.prefill_inputs()
    return oracle.paged_prefill_chunk(step.prefill_query.f32, step.cu_q_lens, pk, pv, bt, cl,
                                      step.scale, rows=rows)


def check(step, rows=None):
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.prefill())
    torch.cuda.synchronize()
    ref = oracle_prefill(step, rows)
    idx = slice(None) if rows is None else list(rows)
    return assert_close(out[idx], ref[idx], step.dtype, step.name)


def test_prefill_mixed_step_chunk():
    """The 512-token chunk on 2048 cached tokens (Hq=32, Hkv=8, D=128): all
    512 x 32 output rows."""
    step = full_refs.step("mixed")
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.prefill())
    torch.cuda.synchronize()
    assert_close(out, full_refs.prefill_ref("mixed"), step.dtype, step.name)


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 128), (8, 2, 128), (8, 1, 64), (16, 2, 64), (2, 2, 128)])
def test_prefill_ragged_chunks(hq, hkv, d):
    # chunk lengths: 1, a partial 16-row tile, exact tiles, whole sequences (nothing cached)
    ctx = [1, 20, 16, 100, 33, 130, 64, 257]
    q_lens = [1, 15, 16, 17, 33, 100, 64, 40]
    step = W.custom(f"pf{hq}_{hkv}_{d}", seed=600 + hq + d, dtype="bf16", hq=hq, hkv=hkv, d=d,
                    ctx=ctx, q_lens=q_lens)
    check(step)


def test_prefill_large_scores():
    """Large scores (scale 3): the running maximum must keep exp() in range."""
    step = W.custom("pfbig", seed=610, dtype="bf16", hq=8, hkv=2, d=128, ctx=[300, 90],
                    q_lens=[70, 90])
    step.scale = 3.0
    check(step)


def test_prefill_row_equals_decode():
    """Chunk row r attends exactly what a decode query at context ctx - T + r + 1 does."""
    step = W.custom("pfdec", seed=611, dtype="bf16", hq=8, hkv=2, d=128, ctx=[200], q_lens=[48])
    pool = DevicePool(step)
    pool.fill()
    out = to_f32(pool.prefill())
    bt, cl = step.prefill_inputs()
    t = int(step.cu_q_lens[1])
    rows = [0, 1, 17, 30, 47]
    q = step.prefill_query.bits[rows]
    lens = np.array([cl[0] - t + r + 1 for r in rows], dtype=np.int32)
    tables = np.repeat(bt[:1], len(rows), axis=0)
    dec = to_f32(pool.decode(-1, query=to_device(W.Values("bf16", np.ascontiguousarray(q))),
                             tables=tables, lens=lens))
    np.testing.assert_allclose(out[rows], dec, rtol=1e-2, atol=2e-3)


def test_prefill_poison_not_read():
    """NaN in unused slots and unused table entries never reaches the output."""
    step = W.custom("pfpoison", seed=612, dtype="bf16", hq=4, hkv=1, d=128, ctx=[17, 65, 3],
                    q_lens=[17, 10, 3])
    check(step)
