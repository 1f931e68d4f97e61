"""The mixed chunked-prefill step end to end, run as bench.py --config 5 runs it.

One sequence prefills a 512-token chunk on 2048 cached tokens while 128
sequences (contexts uniform in 128..4096) decode one token each, all in one
shared scattered pool (Hq=32, Hkv=8, D=128, bf16): one reshape_and_cache of
the step's 640 new tokens, then paged_attention_decode and
paged_attention_prefill_chunk, enqueued back to back on one stream with no
synchronization between them. Every output row of both calls is compared
with the oracle ("The Serving Playbook", "Chunked prefill": the chunk and the
decodes share one step over one cache).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import full_refs
    import paged_kv_decode_reshape_amd as pkv
    from gpu_harness import DevicePool, assert_close, int_tensor, to_device, to_f32


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mixed_step_end_to_end(kv):
    s = full_refs.step("mixed")
    scales = (1.0 / 80, 1.0 / 80) if kv == "fp8" else (None, None)
    pool = DevicePool(s, kv=kv, k_scales=None if kv == "bf16" else [scales[0]],
                      v_scales=None if kv == "bf16" else [scales[1]])
    pool.append(s.cached_key, s.cached_value, s.cached_slots)     # the cache before the step
    assert len(s.new_slots) == 640
    stream = torch.cuda.current_stream()
    new_k, new_v = to_device(s.new_key), to_device(s.new_value)
    slots = int_tensor(s.new_slots, torch.int64)
    bt, cl = s.decode_inputs()
    pbt, pcl = s.prefill_inputs()
    bt_d, cl_d, pbt_d, pcl_d, cu_d = int_tensor(bt), int_tensor(cl), int_tensor(pbt), int_tensor(pcl), \
        int_tensor(s.cu_q_lens)
    q, pq = to_device(s.decode_query), to_device(s.prefill_query)
    total = int(s.cu_q_lens[-1])
    out = torch.empty((len(cl), s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=q.device)
    pout = torch.empty((total, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=q.device)
    wsb = pkv.paged_attention_decode_workspace_bytes(pool.handle, len(cl), s.num_q_heads, bt.shape[1], 0)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=q.device)
    torch.cuda.synchronize()
    # the step
    pkv.reshape_and_cache(pool.handle, 0, new_k, new_v, slots, len(s.new_slots), stream)
    pkv.paged_attention_decode(pool.handle, 0, out, q, bt_d, cl_d, len(cl), s.num_q_heads, bt.shape[1],
                               s.scale, 0, ws, wsb, stream)
    pkv.paged_attention_prefill_chunk(pool.handle, 0, pout, pq, cu_d, pbt_d, pcl_d, len(pcl), total,
                                      int(np.max(np.diff(s.cu_q_lens))), s.num_q_heads, pbt.shape[1],
                                      s.scale, stream)
    torch.cuda.synchronize()
    ref_dec, ref_pre = full_refs.refs("mixed", *scales)
    assert_close(to_f32(out), ref_dec, "bf16", f"{s.name} decode ({kv} cache)")
    assert_close(to_f32(pout), ref_pre, "bf16", f"{s.name} chunk ({kv} cache)")
