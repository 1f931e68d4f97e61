"""GPU check of the gather-ceiling entry point (paged_kv_gather_checksum).

The call reads the K/V words a decode call reads and folds them into one
XOR checksum per (sequence, KV head) row. Expected values come from the pool
read back to the host (the layout decoder of gpu_harness) and plain numpy:
for row (b, h), the XOR of every 32-bit word of K[t][h] and V[t][h] for
t < context_lens[b], the token at block_tables[b][t // bs], offset t % bs.
Integer work: compared bit for bit. Slots past a sequence's last token hold a
poison pattern, so a load or mask that strays past the context changes the
checksum.
"""
import numpy as np
import pytest

from paged_kv_decode_reshape_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_reshape_amd as pkv
    from gpu_harness import DEV, DevicePool, int_tensor


def expected_checksum(k, v, tables, lens, bs):
    """k, v: [num_blocks, bs, hkv, d] raw bits (uint8/uint16/uint32)."""
    hkv = k.shape[2]
    out = np.zeros((len(lens), hkv), np.uint32)
    for b, ctx in enumerate(lens):
        if ctx <= 0:
            continue
        t = np.arange(int(ctx))
        blk, off = tables[b, t // bs], t % bs
        for arr in (k, v):
            rows = np.ascontiguousarray(arr[blk, off])              # [ctx, hkv, d]
            words = rows.view(np.uint8).reshape(len(t), hkv, -1).view(np.uint32)
            out[b] ^= np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=2), axis=0)
    return out


def run_gather(pool, step, tables=None, lens=None, ws_extra=0):
    bt, cl = step.decode_inputs()
    bt = bt if tables is None else tables
    cl = cl if lens is None else lens
    n = len(cl)
    chk = torch.full((max(n, 1), step.num_kv_heads), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    wsb = (n + 1) * 4 + ws_extra
    ws = torch.full((wsb,), 0x77, dtype=torch.uint8, device=DEV)   # contents on entry are ignored
    pkv.paged_kv_gather_checksum(pool.handle, 0, chk, int_tensor(bt), int_tensor(cl), n, bt.shape[1], ws, wsb)
    torch.cuda.synchronize()
    return chk.cpu().numpy().view(np.uint32)[:n], bt, cl


def check(step, kv=None, **kw):
    pool = DevicePool(step, kv=kv)
    pool.fill()
    got, bt, cl = run_gather(pool, step, **kw)
    k, v = pool.decode_pool()
    ref = expected_checksum(k, v, bt, cl, step.block_size)
    bad = np.argwhere(got != ref)
    assert len(bad) == 0, f"{step.name}: {len(bad)} rows differ, first {bad[:5].tolist()}"
    return got


RAGGED = [1, 16, 17, 63, 64, 65, 129, 200, 1000, 0, 333]


@pytest.mark.parametrize("dtype,kv,d,bs", [
    ("bf16", None, 128, 16), ("bf16", None, 64, 16), ("bf16", None, 128, 32),
    ("f32", None, 64, 16), ("f32", None, 128, 16),
    ("bf16", "fp8", 128, 16), ("bf16", "fp8", 64, 16), ("bf16", "fp8", 128, 32)])
def test_gather_checksum_ragged(dtype, kv, d, bs):
    step = W.custom(f"gather_{dtype}_{kv}_{d}_{bs}", seed=900 + d + bs, dtype=dtype, hq=4, hkv=2, d=d,
                    ctx=RAGGED, block_size=bs)
    got = check(step, kv=kv)
    assert got[RAGGED.index(0)].tolist() == [0, 0]


def test_gather_checksum_rows_cut_between_waves():
    # More windows than resident waves with lengths that end mid-window and
    # mid-block, so shares cut rows at every kind of boundary.
    rng = np.random.default_rng(5)
    ctx = W.lognormal_lengths(rng, 700, median=900.0, sigma=1.2, lo=1, hi=8192)
    ctx[::37] = 0
    step = W.custom("gather_cut", seed=905, dtype="bf16", hq=8, hkv=8, d=128, ctx=ctx)
    check(step)


def test_gather_checksum_llama8b_b256_full():
    # The full decode workload of the bench (B=256, lognormal lengths, churned
    # pool), every row.
    check(W.llama8b_continuous())


def test_gather_checksum_llama8b_b256_fp8_full():
    check(W.llama8b_continuous(), kv="fp8")
