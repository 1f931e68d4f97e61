"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` takes the oracle module as an argument so the same checks can
be run against copies of the oracle with a planted mistake (see
test_oracle_mutants.py); every planted mistake must fail at least one pin.

What pins what:
  * closed forms: a context of one token returns that token's V row; equal
    scores return the mean of the V rows; scores 0 and ln 3 weight two rows
    1/4 and 3/4;
  * a library routine: torch's CPU scaled_dot_product_attention in float64
    (with its own GQA expansion and causal mask) on the *unpaged* K/V, i.e.
    the token-major arrays before they were scattered into the pool;
  * brute force: scalar Python over tiny shapes, walking each position through
    the block table one token at a time;
  * invariants: block permutation, poison in unused slots, split identity;
  * the pages' printed KV-size figures (tests/golden/kv_cache_bytes.json).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from paged_kv_decode_reshape_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# helpers (input plumbing only)
# ---------------------------------------------------------------------------

def oracle_pools(orc, step, include_new=True, dtype=np.float64):
    pk = orc.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim, dtype)
    pv = orc.new_pool(step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim, dtype)
    orc.append(pk, pv, step.cached_key.f32, step.cached_value.f32, step.cached_slots)
    if include_new:
        orc.append(pk, pv, step.new_key.f32, step.new_value.f32, step.new_slots)
    return pk, pv


def contiguous_kv(step, seq):
    """Sequence ``seq``'s K/V in position order, straight from the token-major
    inputs (cached run then new run), without going through any pool."""
    ctx = step.context_lens.astype(np.int64)
    n_new = np.zeros(len(ctx), np.int64)
    n_new[step.decode_seqs] = 1
    if step.cu_q_lens is not None:
        n_new[step.prefill_seqs] = np.diff(step.cu_q_lens)
    n_new = np.minimum(n_new, ctx)
    n_cached = ctx - n_new
    c0 = int(n_cached[:seq].sum())
    n0 = int(n_new[:seq].sum())
    k = np.concatenate([step.cached_key.f32[c0:c0 + n_cached[seq]],
                        step.new_key.f32[n0:n0 + n_new[seq]]])
    v = np.concatenate([step.cached_value.f32[c0:c0 + n_cached[seq]],
                        step.new_value.f32[n0:n0 + n_new[seq]]])
    return k.astype(np.float64), v.astype(np.float64)


def torch_sdpa(q, k, v, scale, causal_offset=None):
    """torch CPU float64 SDPA. q [T, Hq, D]; k, v [n, Hkv, D].

    causal_offset=None: no mask. Otherwise query row r may see keys
    0..causal_offset + r.
    """
    qt = torch.from_numpy(np.ascontiguousarray(q, np.float64)).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float64)).permute(1, 0, 2).unsqueeze(0)
    vt = torch.from_numpy(np.ascontiguousarray(v, np.float64)).permute(1, 0, 2).unsqueeze(0)
    mask = None
    if causal_offset is not None:
        t, n = q.shape[0], k.shape[0]
        mask = torch.arange(n)[None, :] <= (causal_offset + torch.arange(t))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.contiguous(), kt.contiguous(), vt.contiguous(), attn_mask=mask, scale=scale,
        enable_gqa=True)
    return o.squeeze(0).permute(1, 0, 2).numpy()


def small_step(seed=7, dtype="f32", hq=4, hkv=2, d=16, ctx=(1, 5, 16, 17, 40), q_lens=None):
    return W.custom(f"pin{seed}", seed=seed, dtype=dtype, hq=hq, hkv=hkv, d=d,
                    ctx=list(ctx), q_lens=q_lens)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_context_one_returns_v_row(orc):
    """ctx = 1: the single weight is exp(0)/exp(0) = 1, so the output is the V row."""
    step = small_step(seed=11, ctx=(1, 1, 1), hq=6, hkv=3, d=8)
    pk, pv = oracle_pools(orc, step)
    bt, cl = step.decode_inputs()
    out = orc.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale)
    g = step.num_q_heads // step.num_kv_heads
    for b in range(len(cl)):
        for i in range(step.num_q_heads):
            assert np.array_equal(out[b, i], step.new_value.f32[b, i // g].astype(np.float64))


def pin_uniform_scores_give_mean(orc):
    """q = 0 makes every score equal, so the output is the mean of the V rows."""
    step = small_step(seed=12, ctx=(3, 16, 33, 50), hq=4, hkv=1, d=8)
    pk, pv = oracle_pools(orc, step)
    bt, cl = step.decode_inputs()
    q = np.zeros_like(step.decode_query.f32)
    out = orc.paged_decode(q, pk, pv, bt, cl, step.scale)
    for b in range(len(cl)):
        _, v = contiguous_kv(step, b)
        for i in range(step.num_q_heads):
            np.testing.assert_allclose(out[b, i], v[:, 0].mean(axis=0), rtol=0, atol=1e-13)


def pin_two_token_closed_form(orc):
    """Scores 0 and ln 3 give weights 1/4 and 3/4: out = (v0 + 3 v1) / 4."""
    pk = orc.new_pool(4, 16, 1, 2)
    pv = orc.new_pool(4, 16, 1, 2)
    key = np.array([[[0.0, 5.0]], [[1.0, -2.0]]])
    val = np.array([[[4.0, -8.0]], [[8.0, 4.0]]])
    orc.append(pk, pv, key, val, np.array([2 * 16 + 0, 2 * 16 + 1]))
    q = np.array([[[math.log(3.0), 0.0]]])
    out = orc.paged_decode(q, pk, pv, np.array([[2]]), np.array([2]), 1.0)
    np.testing.assert_allclose(out[0, 0], [7.0, 1.0], rtol=0, atol=1e-14)


def pin_matches_torch_sdpa_decode(orc):
    """Paged decode equals torch float64 SDPA on the unpaged token-major K/V."""
    step = small_step(seed=13, ctx=(1, 2, 15, 16, 17, 31, 64, 100), hq=8, hkv=2, d=32)
    pk, pv = oracle_pools(orc, step)
    bt, cl = step.decode_inputs()
    out = orc.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale)
    for b in range(len(cl)):
        k, v = contiguous_kv(step, b)
        ref = torch_sdpa(step.decode_query.f32[b:b + 1], k, v, step.scale)[0]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def pin_matches_torch_sdpa_prefill(orc):
    """A prefill chunk on top of cached tokens equals causally masked SDPA, and a
    chunk with nothing cached before it equals plain causal attention."""
    step = small_step(seed=14, ctx=(37, 21, 64, 5), q_lens=(9, 21, 16, 0), hq=4, hkv=2, d=16)
    pk, pv = oracle_pools(orc, step)
    bt, cl = step.prefill_inputs()
    out = orc.paged_prefill_chunk(step.prefill_query.f32, step.cu_q_lens, pk, pv, bt, cl,
                                  step.scale)
    for j, s in enumerate(step.prefill_seqs):
        lo, hi = step.cu_q_lens[j], step.cu_q_lens[j + 1]
        k, v = contiguous_kv(step, s)
        ref = torch_sdpa(step.prefill_query.f32[lo:hi], k, v, step.scale,
                         causal_offset=len(k) - (hi - lo))
        np.testing.assert_allclose(out[lo:hi], ref, rtol=0, atol=1e-12)
        if hi - lo == len(k):   # nothing cached before the chunk
            qt = torch.from_numpy(step.prefill_query.f32[lo:hi].astype(np.float64))
            kt = torch.from_numpy(k).repeat_interleave(step.num_q_heads // step.num_kv_heads, 1)
            vt = torch.from_numpy(v).repeat_interleave(step.num_q_heads // step.num_kv_heads, 1)
            ref2 = torch.nn.functional.scaled_dot_product_attention(
                qt.permute(1, 0, 2).contiguous(), kt.permute(1, 0, 2).contiguous(),
                vt.permute(1, 0, 2).contiguous(), is_causal=True, scale=step.scale)
            np.testing.assert_allclose(out[lo:hi], ref2.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def pin_prefill_row_equals_decode(orc):
    """Chunk row r equals a decode query at context ctx - T + r + 1 over the same pool."""
    step = small_step(seed=15, ctx=(50,), q_lens=(20,), hq=4, hkv=1, d=8)
    pk, pv = oracle_pools(orc, step)
    bt, cl = step.prefill_inputs()
    out = orc.paged_prefill_chunk(step.prefill_query.f32, step.cu_q_lens, pk, pv, bt, cl,
                                  step.scale)
    t = int(step.cu_q_lens[1])
    for r in range(t):
        dec = orc.paged_decode(step.prefill_query.f32[r:r + 1], pk, pv, bt,
                               np.array([cl[0] - t + r + 1]), step.scale)
        np.testing.assert_array_equal(out[r], dec[0])


def _brute_decode(q, pool_k, pool_v, table, ctx, scale):
    bs, hkv, d = pool_k.shape[1], pool_k.shape[2], pool_k.shape[3]
    hq = len(q)
    out = [[0.0] * d for _ in range(hq)]
    if ctx == 0:
        return out
    for i in range(hq):
        h = (i * hkv) // hq
        where = [(int(table[t // bs]), t % bs) for t in range(ctx)]
        scores = []
        for blk, off in where:
            acc = 0.0
            for j in range(d):
                acc += float(q[i][j]) * float(pool_k[blk, off, h, j])
            scores.append(scale * acc)
        top = max(scores)
        w = [math.exp(x - top) for x in scores]
        tot = math.fsum(w)
        for j in range(d):
            out[i][j] = math.fsum(w[t] * float(pool_v[blk, off, h, j])
                                  for t, (blk, off) in enumerate(where)) / tot
    return out


def pin_brute_force_tiny(orc):
    """Scalar Python loops on tiny shapes agree with the vectorized oracle."""
    for seed, hq, hkv, ctx in ((21, 2, 1, (1, 7, 16, 17, 40)), (22, 6, 2, (3, 33)),
                               (23, 3, 3, (0, 18))):
        step = small_step(seed=seed, hq=hq, hkv=hkv, d=8, ctx=ctx)
        pk, pv = oracle_pools(orc, step)
        bt, cl = step.decode_inputs()
        out = orc.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale)
        for b in range(len(cl)):
            ref = _brute_decode(step.decode_query.f32[b], pk, pv, bt[b], int(cl[b]), step.scale)
            np.testing.assert_allclose(out[b], np.array(ref), rtol=0, atol=1e-12)


def pin_block_permutation_invariance(orc):
    """Moving physical blocks (and rewriting the tables) leaves the result bit-identical."""
    step = small_step(seed=16, ctx=(5, 16, 47, 90), hq=4, hkv=2, d=16)
    pk, pv = oracle_pools(orc, step)
    bt, cl = step.decode_inputs()
    out = orc.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale)
    perm = np.random.default_rng(5).permutation(step.num_blocks)    # new id of block i
    pk2, pv2 = np.empty_like(pk), np.empty_like(pv)
    pk2[perm], pv2[perm] = pk, pv
    out2 = orc.paged_decode(step.decode_query.f32, pk2, pv2, perm[bt], cl, step.scale)
    assert np.array_equal(out, out2)


def pin_poison_not_read(orc):
    """Unused slots of last blocks and unused table entries hold NaN; no output is NaN,
    and a context of zero gives zeros."""
    step = small_step(seed=17, ctx=(0, 1, 15, 17, 33), hq=4, hkv=2, d=16)
    pk, pv = oracle_pools(orc, step)
    assert np.isnan(pk[step.poison_block]).all()
    bt, cl = step.decode_inputs()
    out = orc.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale)
    assert np.isfinite(out).all()
    assert np.array_equal(out[0], np.zeros_like(out[0]))


def pin_large_scores_stay_finite(orc):
    """Scores in the hundreds overflow exp() unless the row maximum is subtracted;
    compare with scipy's softmax."""
    import scipy.special
    rng = np.random.default_rng(3)
    k = rng.standard_normal((40, 1, 8)) * 30.0
    v = rng.standard_normal((40, 1, 8))
    q = rng.standard_normal((2, 8)) * 30.0
    out = orc.attend(q, k, v, 1.0)
    for i in range(2):
        ref = scipy.special.softmax(k[:, 0] @ q[i]) @ v[:, 0]
        np.testing.assert_allclose(out[i], ref, rtol=0, atol=1e-12)


def pin_split_identity(orc):
    """Any cut of the KV axis, empty pieces included, recombines to the unsplit result."""
    rng = np.random.default_rng(4)
    for n in (1, 2, 17, 100):
        k = rng.standard_normal((n, 2, 16))
        k[rng.random(n) < 0.1] *= 8.0
        v = rng.standard_normal((n, 2, 16))
        q = rng.standard_normal((4, 16))
        ref = orc.attend(q, k, v, 0.25)
        for _ in range(5):
            cuts = np.sort(rng.integers(0, n + 1, size=rng.integers(0, 6)))
            bounds = [0, *cuts.tolist(), n]
            np.testing.assert_allclose(orc.attend_split(q, k, v, 0.25, bounds), ref,
                                       rtol=0, atol=1e-12)


def pin_append_semantics(orc):
    """Append writes exactly the listed slots (bit-exact) and skips negative slots."""
    pk = orc.new_pool(6, 16, 2, 4)
    pv = orc.new_pool(6, 16, 2, 4)
    rng = np.random.default_rng(1)
    key = rng.standard_normal((4, 2, 4))
    val = rng.standard_normal((4, 2, 4))
    slots = np.array([5 * 16 + 15, -1, 0, 3 * 16 + 7])
    orc.append(pk, pv, key, val, slots)
    assert np.array_equal(pk[5, 15], key[0]) and np.array_equal(pv[5, 15], val[0])
    assert np.array_equal(pk[0, 0], key[2]) and np.array_equal(pv[3, 7], val[3])
    assert np.isnan(pk).reshape(-1, 2, 4).all(axis=(1, 2)).sum() == 6 * 16 - 3


def pin_kv_bytes_golden(orc):
    """The pages' printed KV sizes."""
    with open(os.path.join(GOLDEN, "kv_cache_bytes.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        got = orc.kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["dtype_bytes"],
                                 c["seq_len"], c["batch"])
        assert got == c["bytes"], c["what"]
    for c in gold["blocks"]:
        assert orc.blocks_for(c["ctx"], c["block_size"]) == c["blocks"], c["what"]


def pin_last_block_waste_bound(orc):
    """Only the last block is partial: waste is at most block_size - 1 tokens."""
    for bs in (1, 16, 32):
        for ctx in range(0, 200):
            nb = orc.blocks_for(ctx, bs)
            assert 0 <= nb * bs - ctx <= bs - 1


def pin_copy_on_write_fork(orc):
    """Two sequences share a 40-token prompt (blocks 3, 7 full and block 5
    holding 8 tokens); at the fork the partly filled block 5 is copied into
    block 9 for the second sequence, and each appends its own 6 tokens. Each
    sequence's gathered cache must equal an unshared cache built for it alone,
    and the shared prompt's source blocks must still hold the prompt."""
    rng = np.random.default_rng(21)
    bs, hkv, d = 16, 2, 8
    prompt_k, prompt_v = rng.standard_normal((2, 40, hkv, d))
    tails = rng.standard_normal((2, 2, 6, hkv, d))            # [seq][k/v][token]
    pk = orc.new_pool(12, bs, hkv, d)
    pv = orc.new_pool(12, bs, hkv, d)
    shared = [3, 7, 5]
    slots = np.array([shared[p // bs] * bs + p % bs for p in range(40)])
    orc.append(pk, pv, prompt_k, prompt_v, slots)
    orc.copy_blocks(pk, pv, [[5, 9]])
    tables = [np.array([3, 7, 5]), np.array([3, 7, 9])]
    for sq in range(2):
        pos = np.arange(40, 46)
        orc.append(pk, pv, tails[sq, 0], tails[sq, 1], tables[sq][pos // bs] * bs + pos % bs)
    for sq in range(2):
        want_k = np.concatenate([prompt_k, tails[sq, 0]])
        want_v = np.concatenate([prompt_v, tails[sq, 1]])
        assert np.array_equal(orc.gather(pk, tables[sq], 46), want_k)
        assert np.array_equal(orc.gather(pv, tables[sq], 46), want_v)
    assert np.array_equal(orc.gather(pk, np.array([3, 7]), 32), prompt_k[:32])


def pin_block_size_32_matches_sdpa(orc):
    """With 32-token blocks the oracle's decode and chunk attention equal
    torch float64 SDPA on the unpaged K/V, exactly as with 16-token blocks."""
    for bs in (32, 16):
        step = W.custom(f"pin32_{bs}", seed=23, dtype="f32", hq=6, hkv=2, d=16,
                        ctx=[1, 2, 31, 32, 33, 64, 65, 150], block_size=bs)
        pk, pv = oracle_pools(orc, step)
        assert pk.shape[1] == bs
        bt, cl = step.decode_inputs()
        out = orc.paged_decode(step.decode_query.f32, pk, pv, bt, cl, step.scale)
        for b in range(len(cl)):
            k, v = contiguous_kv(step, b)
            ref = torch_sdpa(step.decode_query.f32[b:b + 1], k, v, step.scale)[0]
            np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)
    step = W.custom("pin32_chunk", seed=24, dtype="f32", hq=4, hkv=1, d=16, ctx=[33, 70, 64],
                    q_lens=[33, 5, 32], block_size=32)
    pk, pv = oracle_pools(orc, step)
    bt, cl = step.prefill_inputs()
    out = orc.paged_prefill_chunk(step.prefill_query.f32, step.cu_q_lens, pk, pv, bt, cl, step.scale)
    for i, s in enumerate(step.prefill_seqs):
        k, v = contiguous_kv(step, int(s))
        lo, hi = int(step.cu_q_lens[i]), int(step.cu_q_lens[i + 1])
        ref = torch_sdpa(step.prefill_query.f32[lo:hi], k, v, step.scale, causal_offset=len(k) - (hi - lo))
        np.testing.assert_allclose(out[lo:hi], ref, rtol=0, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
