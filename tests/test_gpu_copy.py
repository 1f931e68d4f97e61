"""GPU parity of copy_blocks (copy-on-write) against the oracle: bit-exact pool
contents on every layer, and a forked pair of sequences decoding to the
oracle's attention over what each of them logically holds."""
import numpy as np
import pytest

import oracle
from paged_kv_decode_reshape_amd import workloads as W
import paged_kv_decode_reshape_amd as pkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_harness import DevicePool, assert_close, int_tensor, to_f32, to_device, POISON_BITS


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_copy_blocks_bit_exact(kv):
    dtype = "f32" if kv == "f32" else "bf16"
    step = W.custom(f"cow_{kv}", seed=950, dtype=dtype, hq=8, hkv=2, d=64, ctx=[100, 37, 300])
    kw = {} if kv != "fp8" else dict(kv="fp8", k_scales=[0.05, 0.1, 1.0], v_scales=[0.5, 1.0, 2.0])
    pool = DevicePool(step, num_layers=3, **kw)
    for layer in range(3):
        pool.fill(layer=layer)
    before = [pool.decode_pool(layer) for layer in range(3)]
    nb = step.num_blocks
    rng = np.random.default_rng(0)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:7], perm[7:14]], axis=1).astype(np.int32)   # distinct sources and destinations
    pkv.copy_blocks(pool.handle, int_tensor(pairs), len(pairs))
    torch.cuda.synchronize()
    for layer in range(3):
        k, v = pool.decode_pool(layer)
        ek, ev = before[layer][0].copy(), before[layer][1].copy()
        for src, dst in pairs:
            ek[dst], ev[dst] = ek[src], ev[src]
        assert np.array_equal(k, ek) and np.array_equal(v, ev), f"layer {layer}"


def test_copy_on_write_fork_decodes():
    """Sequences 0 and 1 share a 40-token prompt; at the fork the partly filled
    third block is copied for sequence 1, each appends 6 tokens of its own,
    and both decode to the oracle's result on their own logical contents."""
    rng = np.random.default_rng(4)
    hq, hkv, d, bs = 8, 2, 128, 16
    step = W.custom("fork", seed=951, dtype="bf16", hq=hq, hkv=hkv, d=d, ctx=[46, 46, 400])   # pool of >= 10 blocks
    pool = DevicePool(step)
    prompt = W.make_values(rng.standard_normal((2, 40, hkv, d), dtype=np.float32), "bf16")
    tails = W.make_values(rng.standard_normal((2, 2, 6, hkv, d), dtype=np.float32), "bf16")
    shared = np.array([3, 7, 5]); private = 9
    tables = np.array([[3, 7, 5], [3, 7, private]], dtype=np.int32)
    pos = np.arange(40)
    slots = shared[pos // bs] * bs + pos % bs
    pool.append(W.Values("bf16", prompt.bits[0]), W.Values("bf16", prompt.bits[1]), slots)
    pkv.copy_blocks(pool.handle, int_tensor(np.array([[5, private]], np.int32)), 1)
    for sq in range(2):
        p2 = np.arange(40, 46)
        pool.append(W.Values("bf16", tails.bits[sq, 0]), W.Values("bf16", tails.bits[sq, 1]),
                    tables[sq][p2 // bs] * bs + p2 % bs)
    q = W.make_values(rng.standard_normal((2, hq, d), dtype=np.float32), "bf16")
    lens = np.array([46, 46], np.int32)
    out = to_f32(pool.decode(0, query=to_device(q), tables=tables, lens=lens))
    torch.cuda.synchronize()
    pk = oracle.new_pool(step.num_blocks, bs, hkv, d)
    pv = oracle.new_pool(step.num_blocks, bs, hkv, d)
    for sq in range(2):
        toks = np.arange(46)
        kk = np.concatenate([prompt.f32[0], tails.f32[sq, 0]])
        vv = np.concatenate([prompt.f32[1], tails.f32[sq, 1]])
        oracle.append(pk, pv, kk, vv, tables[sq][toks // bs] * bs + toks % bs)
        # the unshared view of sequence sq, written as if it owned its blocks
        ref = oracle.paged_decode(q.f32[sq:sq + 1], pk, pv, tables[sq:sq + 1], lens[sq:sq + 1], step.scale)
        assert_close(out[sq:sq + 1], ref, "bf16", f"fork seq {sq}")
