"""Invariants of the seeded input generators (CPU only)."""
import numpy as np

from paged_kv_decode_reshape_amd import workloads as W


def _check_step(step):
    bs = step.block_size
    ctx = step.context_lens
    used = []
    for s, c in enumerate(ctx):
        nb = W.blocks_needed(c, bs)
        row = step.block_tables[s]
        assert (row[nb:] == step.poison_block).all()
        used.extend(row[:nb].tolist())
    used = np.array(used)
    assert len(np.unique(used)) == len(used), "a physical block is owned twice"
    assert (used >= 0).all() and (used < step.num_blocks).all()
    assert step.poison_block not in set(used.tolist())
    slots = np.concatenate([step.cached_slots, step.new_slots])
    slots = slots[slots >= 0]
    assert len(np.unique(slots)) == len(slots), "duplicate slot"
    assert (slots // bs != step.poison_block).all()
    assert len(slots) == int(ctx.sum())
    assert step.decode_query.shape[1:] == (step.num_q_heads, step.head_dim)


def test_tiny_fp32_shape():
    step = W.tiny_fp32()
    assert step.dtype == "f32" and step.num_blocks == 64
    assert step.context_lens.tolist() == [1, 17, 64, 200]
    assert (step.num_q_heads, step.num_kv_heads, step.head_dim) == (4, 1, 64)
    _check_step(step)


def test_qwen_grid_points():
    assert len(W.QWEN_GRID) == 13
    step = W.qwen_layer(4, 128)
    assert (step.num_q_heads, step.num_kv_heads, step.head_dim) == (12, 2, 128)
    need = sum(W.blocks_needed(c) for c in step.context_lens)
    assert step.num_blocks == int(np.ceil(1.25 * need)) + 1
    _check_step(step)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 0.0], np.float32)
    got = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5, 0.0]


def test_churn_fragments_pool():
    rng = np.random.Generator(np.random.PCG64(3))
    ctx = W.lognormal_lengths(rng, 256)
    assert 16 <= ctx.min() and ctx.max() <= 8192
    assert 450 <= np.median(ctx) <= 750
    tables, nblocks, poison = W._churn_tables(rng, ctx, 16)
    frac = W.adjacency_fraction(tables, ctx)
    assert frac < 0.4
    used = np.concatenate([tables[s, :W.blocks_needed(c)] for s, c in enumerate(ctx)])
    assert len(np.unique(used)) == len(used) and poison not in set(used.tolist())


def test_custom_with_prefill_and_empty():
    step = W.custom("t", seed=1, dtype="bf16", hq=8, hkv=2, d=64, ctx=[0, 5, 40, 33],
                    q_lens=[0, 0, 12, 33])
    _check_step(step)
    assert step.cu_q_lens.tolist() == [0, 12, 45]
    assert step.decode_seqs.tolist() == [0, 1]


def _check_shared_step(step):
    """Sharing groups: members' tables agree on the whole prefix blocks, no
    block outside them is listed twice, every slot is written once, and a
    member's copy of a partly filled prefix block holds the prefix values."""
    bs = step.block_size
    gs, pl = step.info["group_starts"], step.info["prefix_lens"]
    assert gs[0] == 0 and gs[-1] == len(step.context_lens) and (np.diff(gs) >= 0).all()
    owners = {}
    for k in range(len(pl)):
        n_sh = int(pl[k]) // bs
        rows = step.block_tables[gs[k]:gs[k + 1]]
        assert (rows[:, :n_sh] == rows[0, :n_sh]).all(), "members disagree on a shared block"
        for i, s in enumerate(range(gs[k], gs[k + 1])):
            c = int(step.context_lens[s])
            assert c >= pl[k]
            nb = W.blocks_needed(c, bs)
            assert (step.block_tables[s, nb:] == step.poison_block).all()
            for j, blk in enumerate(step.block_tables[s, :nb].tolist()):
                key = (k, j) if j < n_sh else (k, s, j)
                assert owners.setdefault(blk, key) == key, "a physical block is owned twice"
    slots = np.concatenate([step.cached_slots, step.new_slots])
    assert len(np.unique(slots)) == len(slots), "duplicate slot"
    # whole shared blocks are written once, every member writes the rest of
    # its context (a partly filled prefix block is copied per member);
    # unique_tokens counts each logical prefix token once
    stored = sum(int(pl[k]) // bs * bs + sum(int(c) - int(pl[k]) // bs * bs
                                              for c in step.context_lens[gs[k]:gs[k + 1]])
                 for k in range(len(pl)))
    assert len(slots) == stored
    assert step.info["unique_tokens"] == sum(int(pl[k]) + sum(int(c) - int(pl[k])
                                                              for c in step.context_lens[gs[k]:gs[k + 1]])
                                             for k in range(len(pl)))
    # the values stored at each member's logical prefix positions agree
    pos_val = {}
    for vals, sl in ((step.cached_key.bits, step.cached_slots), (step.new_key.bits, step.new_slots)):
        for x, slot in zip(vals, sl.tolist()):
            pos_val[slot] = x
    for k in range(len(pl)):
        members = range(gs[k], gs[k + 1])
        for p in range(int(pl[k])):
            ref = None
            for s in members:
                slot = int(step.block_tables[s, p // bs]) * bs + p % bs
                if ref is None:
                    ref = pos_val[slot]
                assert np.array_equal(pos_val[slot], ref), f"prefix position {p} differs in group {k}"


def test_shared_prefix_generator():
    groups = [(40, [41, 60, 100]), (0, [5]), (256, [256]), (33, [34, 35, 90]), (0, [0])]
    for bs in (16, 32):
        step = W.shared_prefix(f"sh{bs}", seed=5, dtype="bf16", hq=8, hkv=2, d=64, groups=groups,
                               block_size=bs)
        assert step.block_size == bs
        _check_shared_step(step)


def test_parallel_sampling_shape():
    step = W.parallel_sampling(prompts=4, samples=8, prompt_len=2000, max_new=64)
    assert len(step.context_lens) == 32 and (step.info["prefix_lens"] == 2000).all()
    assert ((step.context_lens > 2000) & (step.context_lens <= 2064)).all()
    _check_shared_step(step)


def test_block32_churn_step():
    step = W.llama8b_continuous(block_size=32)
    assert step.block_size == 32 and step.name.endswith("_bs32")
    _check_step(step)
