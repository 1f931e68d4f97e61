"""GPU check of the library's kernel timing (pkv_timing_*): every timed launch
records one event pair stamped by the launch itself, kinds not selected record
nothing, and the results of timed calls equal those of untimed calls."""
import numpy as np
import pytest

from paged_kv_decode_reshape_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_reshape_amd as pkv
    from gpu_harness import DevicePool, raw_bits


def test_timed_launches_are_recorded_per_kind():
    step = W.custom("timing", seed=31, dtype="bf16", hq=8, hkv=2, d=128, ctx=[5, 300, 1200, 64],
                    q_lens=[0, 0, 0, 48])
    pool = DevicePool(step)
    pool.fill()
    ref = raw_bits(pool.decode(0))
    ref_p = raw_bits(pool.prefill())
    torch.cuda.synchronize()
    pkv.pkv_timing_enable(16, [pkv.KERNEL_DECODE_PARTITION, pkv.KERNEL_PREFILL])
    try:
        outs = [raw_bits(pool.decode(0)) for _ in range(3)]
        out_p = raw_bits(pool.prefill())
        pool.fill()                                   # appends: a kind not selected
        torch.cuda.synchronize()
        dec = pkv.pkv_timing_read_launches(pkv.KERNEL_DECODE_PARTITION, 16)
        pre = pkv.pkv_timing_read_launches(pkv.KERNEL_PREFILL, 16)
        app = pkv.pkv_timing_read_launches(pkv.KERNEL_APPEND, 16)
        n, total = pkv.pkv_timing_read(pkv.KERNEL_DECODE_PARTITION)
    finally:
        pkv.pkv_timing_disable()
    assert len(dec) == 3 and len(pre) == 1 and app == []
    assert n == 3 and abs(total - sum(dec)) < 1e-6
    assert all(0.0 < ms < 100.0 for ms in dec + pre), (dec, pre)
    for o in outs:
        assert np.array_equal(o, ref)
    assert np.array_equal(out_p, ref_p)


def test_timing_capacity_stops_recording():
    step = W.custom("timing_cap", seed=32, dtype="bf16", hq=4, hkv=1, d=64, ctx=[100, 7])
    pool = DevicePool(step)
    pool.fill()
    pkv.pkv_timing_enable(2, [pkv.KERNEL_DECODE_PARTITION])
    try:
        for _ in range(4):
            pool.decode(0)
        torch.cuda.synchronize()
        dec = pkv.pkv_timing_read_launches(pkv.KERNEL_DECODE_PARTITION, 8)
    finally:
        pkv.pkv_timing_disable()
    assert len(dec) == 2 and all(ms > 0.0 for ms in dec)
