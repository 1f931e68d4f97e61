"""Seeded synthetic inputs for one continuous-batching attention step.

This module builds the *inputs* of a step and nothing else: context lengths,
block tables over a shared physical pool, slot mappings, and the K/V/Q values.
It holds none of the attention arithmetic. Both the GPU library's tests and the
CPU oracle are fed from here, so neither side depends on the other.

Problem statement followed (pages by title, section):
  * "LLM 7 - Efficient LLM Serving", section 3 "Paging the Cache": each
    sequence's logical KV is cut into fixed-size blocks; a block table maps
    logical blocks to physical blocks anywhere in the pool; only a sequence's
    last block can be partly filled.
  * "The Serving Playbook", section "Paged KV cache": blocks of 16 tokens, and
    "CUDA graphs and the CPU you forgot about": slot mappings preallocated next
    to the block tables.
  * "The Serving Playbook", "vLLM up close", "Prefix caching as a side effect of
    the allocator": freed blocks go to the tail of a free list (used by the
    alloc/free churn that fragments the pool).
  * "The Serving Playbook", "Continuous batching": ragged queries addressed by
    cumulative-length offsets.

Conventions (the library header documents the same contract):
  * context_lens[b] counts the tokens in the pool for sequence b *after* this
    step's append (so a decode query attends to its own new token).
  * slot = physical_block * block_size + offset_in_block; a negative slot means
    "skip this token".
  * Unused block-table entries point at a dedicated poison block, and every
    pool slot that is never written holds NaN, so a kernel that reads past a
    sequence's length produces NaN.

Values are drawn as float32 N(0, 1) and rounded to the storage dtype
(round-to-nearest-even for bf16); ``*_f32`` arrays hold those stored values
exactly, which is what the oracle consumes.
"""
from __future__ import annotations

import collections
import concurrent.futures
import dataclasses
import math
import os

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------
# dtype helpers (input preparation only)
# --------------------------------------------------------------------------

def _round_chunk(src: np.ndarray, dst: np.ndarray) -> None:
    u = src.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    dst[...] = t


def _parallel_chunks(n: int, fn, chunk: int = 1 << 22) -> None:
    starts = range(0, n, chunk)
    if n <= chunk:
        fn(0, n)
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda a: fn(a, min(n, a + chunk)), starts))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction, so no NaN handling is needed.
    """
    src = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(src.shape, dtype=np.uint16)
    fs, fo = src.reshape(-1), out.reshape(-1)
    _parallel_chunks(fs.size, lambda a, b: _round_chunk(fs[a:b], fo[a:b]))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Values:
    """A tensor of stored values: ``bits`` is what the device holds (uint16 for
    bf16, float32 for f32); ``f32`` is the exact float32 value of each element."""

    def __init__(self, dtype: str, bits: np.ndarray):
        self.dtype = dtype
        self.bits = bits

    @property
    def f32(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.bits
        return bf16_bits_to_f32(self.bits)

    @property
    def shape(self):
        return self.bits.shape

    @property
    def itemsize(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def make_values(x: np.ndarray, dtype: str) -> Values:
    if dtype == "bf16":
        return Values("bf16", f32_to_bf16_bits(x))
    if dtype == "f32":
        return Values("f32", np.ascontiguousarray(x, dtype=np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


# --------------------------------------------------------------------------
# Step description
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Step:
    """All inputs of one attention step over a paged pool (one layer).

    cached_*: tokens already in the pool before the step (token-major
      [n, Hkv, D]); new_*: the step's appended tokens. Both carry slots.
    Decode sequences are listed in ``decode_seqs``; prefill-chunk sequences in
    ``prefill_seqs`` with query rows packed by ``cu_q_lens``.
    """
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    poison_block: int
    context_lens: np.ndarray      # int32 [S] (all sequences of the pool)
    block_tables: np.ndarray      # int32 [S, max_blocks]
    cached_key: Values
    cached_value: Values
    cached_slots: np.ndarray      # int64 [n_cached]
    new_key: Values
    new_value: Values
    new_slots: np.ndarray         # int64 [n_new]
    decode_seqs: np.ndarray       # int32 indices into context_lens / block_tables
    decode_query: Values          # [len(decode_seqs), Hq, D]
    prefill_seqs: np.ndarray      # int32 indices
    prefill_query: Values | None  # [total_q, Hq, D]
    cu_q_lens: np.ndarray | None  # int32 [len(prefill_seqs)+1]
    scale: float
    partition_size: int = 0       # decode split size; 0 = library's choice
    info: dict = dataclasses.field(default_factory=dict)

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def decode_inputs(self):
        """Block tables / lengths restricted to the decode sequences (contiguous)."""
        idx = self.decode_seqs
        return (np.ascontiguousarray(self.block_tables[idx]),
                np.ascontiguousarray(self.context_lens[idx]))

    def prefill_inputs(self):
        idx = self.prefill_seqs
        return (np.ascontiguousarray(self.block_tables[idx]),
                np.ascontiguousarray(self.context_lens[idx]))


def blocks_needed(ctx: int, bs: int = BLOCK_SIZE) -> int:
    return -(-int(ctx) // bs)


def _slots_for(block_table_row: np.ndarray, positions: np.ndarray, bs: int) -> np.ndarray:
    positions = np.asarray(positions, dtype=np.int64)
    return block_table_row[positions // bs].astype(np.int64) * bs + positions % bs


def _assemble(name, rng, dtype, hq, hkv, d, bs, num_blocks, poison_block, ctx,
              tables, n_new_per_seq, decode_seqs, prefill_seqs,
              boost_k_fraction=0.0, boost=8.0, partition_size=0, info=None) -> Step:
    """Draw values and slots once block tables and lengths are fixed.

    n_new_per_seq[s] = number of this step's tokens of sequence s (1 for a
    decode, the chunk length for a prefill chunk); they occupy the last
    positions [ctx - n_new, ctx).
    """
    ctx = np.asarray(ctx, dtype=np.int32)
    nseq = len(ctx)
    cached_slots, new_slots = [], []
    for s in range(nseq):
        n_new = int(n_new_per_seq[s])
        c = int(ctx[s])
        cached_slots.append(_slots_for(tables[s], np.arange(0, c - n_new), bs))
        new_slots.append(_slots_for(tables[s], np.arange(c - n_new, c), bs))
    cached_slots = np.concatenate(cached_slots) if nseq else np.zeros(0, np.int64)
    new_slots = np.concatenate(new_slots) if nseq else np.zeros(0, np.int64)
    nc, nn = len(cached_slots), len(new_slots)

    ck = _normal(rng, (nc, hkv, d))
    cv = _normal(rng, (nc, hkv, d))
    nk = _normal(rng, (nn, hkv, d))
    nv = _normal(rng, (nn, hkv, d))
    if boost_k_fraction > 0.0:
        # Scale a fraction of (token, kv-head) key rows, before rounding; the
        # factor is a power of two so the scaled value is still exact.
        total_rows = (nc + nn) * hkv
        n_boost = int(math.floor(boost_k_fraction * total_rows))
        pick = rng.choice(total_rows, size=n_boost, replace=False)
        for arr, lo, n in ((ck, 0, nc * hkv), (nk, nc * hkv, nn * hkv)):
            sel = pick[(pick >= lo) & (pick < lo + n)] - lo
            flat = arr.reshape(-1, d)
            flat[sel] *= np.float32(boost)
        info = dict(info or {}, boosted_k_rows=n_boost)

    dq = _normal(rng, (len(decode_seqs), hq, d))
    if len(prefill_seqs):
        qlens = np.asarray([n_new_per_seq[s] for s in prefill_seqs], dtype=np.int32)
        cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        pq = make_values(_normal(rng, (int(cu[-1]), hq, d)), dtype)
    else:
        cu, pq = None, None

    return Step(
        name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=bs, num_blocks=int(num_blocks), poison_block=int(poison_block),
        context_lens=ctx, block_tables=np.ascontiguousarray(tables, dtype=np.int32),
        cached_key=make_values(ck, dtype), cached_value=make_values(cv, dtype),
        cached_slots=cached_slots, new_key=make_values(nk, dtype),
        new_value=make_values(nv, dtype), new_slots=new_slots,
        decode_seqs=np.asarray(decode_seqs, dtype=np.int32),
        decode_query=make_values(dq, dtype),
        prefill_seqs=np.asarray(prefill_seqs, dtype=np.int32),
        prefill_query=pq, cu_q_lens=cu, scale=1.0 / math.sqrt(d),
        partition_size=partition_size, info=dict(info or {}))


def _scattered_tables(rng, ctx, bs, num_blocks, max_blocks, poison_block):
    """Hand out blocks of a seeded permutation of the pool in sequence order."""
    order = rng.permutation(num_blocks)
    order = order[order != poison_block]
    tables = np.full((len(ctx), max_blocks), poison_block, dtype=np.int32)
    pos = 0
    for s, c in enumerate(ctx):
        nb = blocks_needed(c, bs)
        tables[s, :nb] = order[pos:pos + nb]
        pos += nb
    return tables


def adjacency_fraction(tables: np.ndarray, ctx: np.ndarray, bs: int = BLOCK_SIZE) -> float:
    """Fraction of logically adjacent block pairs that are also physically adjacent."""
    adj = tot = 0
    for s, c in enumerate(ctx):
        nb = blocks_needed(c, bs)
        if nb > 1:
            row = tables[s, :nb].astype(np.int64)
            adj += int(np.sum(row[1:] == row[:-1] + 1))
            tot += nb - 1
    return adj / tot if tot else 0.0


def _pool_size(ctx, bs, factor=1.25):
    need = sum(blocks_needed(c, bs) for c in ctx)
    # one extra block is reserved as the poison block
    return int(math.ceil(factor * need)) + 1


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

def _rng(config: int, rep: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * config + rep))


def tiny_fp32(rep: int = 0) -> Step:
    """Tiny fp32 decode: B=4, lengths {1,17,64,200}, Hq=4, Hkv=1, D=64, 64-block pool."""
    rng = _rng(1, rep)
    ctx = np.array([1, 17, 64, 200], dtype=np.int32)
    num_blocks, bs = 64, BLOCK_SIZE
    max_blocks = blocks_needed(ctx.max(), bs)
    perm = rng.permutation(num_blocks)
    poison = int(perm[-1])
    tables = np.full((4, max_blocks), poison, dtype=np.int32)
    pos = 0
    for s, c in enumerate(ctx):
        nb = blocks_needed(c, bs)
        tables[s, :nb] = perm[pos:pos + nb]
        pos += nb
    return _assemble("tiny_fp32", rng, "f32", 4, 1, 64, bs, num_blocks, poison, ctx,
                     tables, np.ones(4, np.int64), np.arange(4), [])


QWEN_GRID = [(b, c) for c in (128, 512, 2048) for b in (1, 4, 16, 64, 128)
             if not (c == 2048 and b > 16)]


def qwen_layer(batch: int, context: int, rep: int = 0) -> Step:
    """Qwen2.5-1.5B-shaped layer decode: Hq=12, Hkv=2, D=128, bf16, uniform context."""
    rng = _rng(2, rep * 100000 + batch * 10 + context)
    ctx = np.full(batch, context, dtype=np.int32)
    bs = BLOCK_SIZE
    num_blocks = _pool_size(ctx, bs)
    poison = num_blocks - 1
    max_blocks = blocks_needed(context, bs)
    tables = _scattered_tables(rng, ctx, bs, num_blocks, max_blocks, poison)
    return _assemble(f"qwen_b{batch}_c{context}", rng, "bf16", 12, 2, 128, bs, num_blocks,
                     poison, ctx, tables, np.ones(batch, np.int64), np.arange(batch), [])


def lognormal_lengths(rng, n, median=600.0, sigma=1.0, lo=16, hi=8192) -> np.ndarray:
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def _churn_tables(rng, ctx, bs, rounds=4, median=600.0, sigma=1.0, lo=16, hi=8192):
    """Block tables after a seeded alloc/free churn over a free list.

    The pool holds 1.25x the final need (+1 poison block). A sequence takes
    its prompt's blocks from the head of the free list when admitted, then
    grows one block at a time as it decodes; the growth of all running
    sequences is interleaved in a seeded random order, which is what scatters
    a sequence's blocks. Warm-up rounds admit random-length sequences while
    they fit, grow them, and retire a random half (blocks go back to the tail
    of the free list). Then the remaining warm-up sequences retire, in random
    order, and the real sequences are admitted and grown the same way.
    """
    num_blocks = _pool_size(ctx, bs)
    poison = num_blocks - 1
    free = collections.deque(range(num_blocks - 1))

    def admit_and_grow(targets):
        owned = []
        for nb in targets:
            prompt = max(1, int(nb * rng.uniform(0.2, 1.0)))
            owned.append([free.popleft() for _ in range(prompt)])
        pending = np.repeat(np.arange(len(targets)),
                            [t - len(o) for t, o in zip(targets, owned)])
        rng.shuffle(pending)
        for i in pending:
            owned[i].append(free.popleft())
        return owned

    live = []
    for _ in range(rounds):
        targets, budget = [], len(free)
        while True:
            nb = blocks_needed(int(lognormal_lengths(rng, 1, median, sigma, lo, hi)[0]), bs)
            if nb > budget:
                break
            targets.append(nb)
            budget -= nb
        live += admit_and_grow(targets)
        keep = rng.random(len(live)) >= 0.5
        for blk in (b for b, k in zip(live, keep) if not k):
            free.extend(blk)
        live = [b for b, k in zip(live, keep) if k]
    for i in rng.permutation(len(live)):
        free.extend(live[i])
    owned = admit_and_grow([blocks_needed(c, bs) for c in ctx])
    max_blocks = blocks_needed(int(np.max(ctx)), bs)
    tables = np.full((len(ctx), max_blocks), poison, dtype=np.int32)
    for s, blk in enumerate(owned):
        tables[s, :len(blk)] = blk
    return tables, num_blocks, poison


def llama8b_continuous(rep: int = 0, batch: int = 256, block_size: int = BLOCK_SIZE) -> Step:
    """Llama-8B-shaped layer, B=256 continuous batching, lognormal lengths, churned pool."""
    rng = _rng(3, rep)
    bs = block_size
    ctx = lognormal_lengths(rng, batch)
    tables, num_blocks, poison = _churn_tables(rng, ctx, bs)
    info = {"adjacent_block_fraction": adjacency_fraction(tables, ctx, bs),
            "total_tokens": int(ctx.sum())}
    name = "llama8b_b256_lognormal" + ("" if bs == BLOCK_SIZE else f"_bs{bs}")
    return _assemble(name, rng, "bf16", 32, 8, 128, bs, num_blocks,
                     poison, ctx, tables, np.ones(batch, np.int64), np.arange(batch), [],
                     info=info)


def long_context(rep: int = 0, batch: int = 8, context: int = 32768) -> Step:
    """Long-context split-K decode: B=8 x 32768, Hq=64, Hkv=8, bf16, 512-token partitions,
    1% of key rows scaled by 8."""
    rng = _rng(4, rep)
    bs = BLOCK_SIZE
    ctx = np.full(batch, context, dtype=np.int32)
    num_blocks = _pool_size(ctx, bs)
    poison = num_blocks - 1
    tables = _scattered_tables(rng, ctx, bs, num_blocks, blocks_needed(context, bs), poison)
    return _assemble(f"long_b{batch}_c{context}", rng, "bf16", 64, 8, 128, bs, num_blocks,
                     poison, ctx, tables, np.ones(batch, np.int64), np.arange(batch), [],
                     boost_k_fraction=0.01, boost=8.0, partition_size=512)


def mixed_chunked_prefill(rep: int = 0, chunk: int = 512, cached: int = 2048,
                          n_decode: int = 128, lo: int = 128, hi: int = 4096) -> Step:
    """Mixed step: one 512-token prefill chunk on 2048 cached tokens plus 128 decodes
    with lengths uniform in [128, 4096]; Hq=32, Hkv=8, bf16, one scattered pool."""
    rng = _rng(5, rep)
    bs = BLOCK_SIZE
    dec_ctx = rng.integers(lo, hi, size=n_decode, endpoint=True).astype(np.int32)
    ctx = np.concatenate([[cached + chunk], dec_ctx]).astype(np.int32)
    num_blocks = _pool_size(ctx, bs)
    poison = num_blocks - 1
    tables = _scattered_tables(rng, ctx, bs, num_blocks, blocks_needed(ctx.max(), bs), poison)
    n_new = np.concatenate([[chunk], np.ones(n_decode, np.int64)])
    return _assemble("mixed_chunk512_on2048_plus128", rng, "bf16", 32, 8, 128, bs,
                     num_blocks, poison, ctx, tables, n_new,
                     decode_seqs=np.arange(1, n_decode + 1), prefill_seqs=[0])


def custom(name, *, seed, dtype, hq, hkv, d, ctx, q_lens=None, pool_factor=1.25,
           boost_k_fraction=0.0, partition_size=0, block_size=BLOCK_SIZE) -> Step:
    """General seeded step for tests: per-sequence lengths ``ctx`` and, optionally,
    prefill chunk lengths ``q_lens`` (0 = the sequence decodes one token)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = block_size
    ctx = np.asarray(ctx, dtype=np.int32)
    q_lens = np.zeros(len(ctx), np.int64) if q_lens is None else np.asarray(q_lens, np.int64)
    num_blocks = max(_pool_size(ctx, bs, pool_factor), 2)
    poison = num_blocks - 1
    max_blocks = max(1, blocks_needed(int(ctx.max()) if len(ctx) else 1, bs))
    tables = _scattered_tables(rng, ctx, bs, num_blocks, max_blocks, poison)
    # a sequence of length 0 has nothing to append
    n_new = np.minimum(np.where(q_lens > 0, q_lens, 1), ctx)
    decode = [s for s in range(len(ctx)) if q_lens[s] == 0]
    prefill = [s for s in range(len(ctx)) if q_lens[s] > 0]
    return _assemble(name, rng, dtype, hq, hkv, d, bs, num_blocks, poison, ctx, tables,
                     n_new, decode, prefill, boost_k_fraction=boost_k_fraction,
                     partition_size=partition_size)


def shared_prefix(name, *, seed, dtype, hq, hkv, d, groups, pool_factor=1.25, block_size=BLOCK_SIZE) -> Step:
    """Decode step whose sequences share prefixes in groups.

    ``groups`` is a list of (prefix_len, [context lengths of the members]).
    The whole blocks of a group's prefix are allocated once and appear in every
    member's block table; a partly filled last prefix block is copied into a
    block of each member's own (the copy-on-write at divergence), holding the
    same values. Each member's tokens past the prefix are its own, the last
    one appended this step. Members are consecutive sequences; ``info`` holds
    ``group_starts`` and ``prefix_lens``. Values of a shared position are
    drawn once.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = block_size
    ctx = np.asarray([c for _, members in groups for c in members], dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum([len(m) for _, m in groups])]).astype(np.int32)
    plens = np.asarray([p for p, _ in groups], dtype=np.int32)
    nseq = len(ctx)
    need = sum(blocks_needed(p, bs) // 1 - (p % bs != 0) for p, _ in groups) + sum(
        blocks_needed(c, bs) - (p // bs) for p, m in groups for c in m)
    num_blocks = max(int(math.ceil(pool_factor * need)) + 1, 2)
    poison = num_blocks - 1
    order = [int(x) for x in rng.permutation(num_blocks) if x != poison]
    max_blocks = max(1, blocks_needed(int(ctx.max()) if nseq else 1, bs))
    tables = np.full((nseq, max_blocks), poison, dtype=np.int32)
    ck, cv, cslots, nk, nv, nslots = [], [], [], [], [], []
    pos = 0
    for k, (plen, members) in enumerate(groups):
        assert all(c >= plen for c in members), "a member's context must hold the prefix"
        n_sh = plen // bs                                  # whole shared blocks
        shared = order[pos:pos + n_sh]
        pos += n_sh
        pk, pv = _normal(rng, (plen, hkv, d)), _normal(rng, (plen, hkv, d))
        s0 = int(starts[k])
        for i, c in enumerate(members):
            s = s0 + i
            own = blocks_needed(c, bs) - n_sh
            tables[s, :n_sh] = shared
            tables[s, n_sh:n_sh + own] = order[pos:pos + own]
            pos += own
            if c == 0:
                continue
            assert c - 1 >= n_sh * bs or len(members) == 1, "the new token must land in an own block"
            lo = 0 if i == 0 else n_sh * bs                # shared blocks are written by member 0
            cached = np.arange(lo, c - 1)
            cslots.append(_slots_for(tables[s], cached, bs))
            in_prefix = cached[cached < plen]
            own_pos = cached[cached >= plen]
            ok, ov = _normal(rng, (len(own_pos), hkv, d)), _normal(rng, (len(own_pos), hkv, d))
            ck.append(np.concatenate([pk[in_prefix], ok]))
            cv.append(np.concatenate([pv[in_prefix], ov]))
            nslots.append(_slots_for(tables[s], np.asarray([c - 1]), bs))
            if c - 1 < plen:
                nk.append(pk[c - 1:c])
                nv.append(pv[c - 1:c])
            else:
                nk.append(_normal(rng, (1, hkv, d)))
                nv.append(_normal(rng, (1, hkv, d)))

    def cat(parts, shape):
        return np.concatenate(parts) if parts else np.zeros(shape, np.float32)

    dq = _normal(rng, (nseq, hq, d))
    return Step(
        name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=bs, num_blocks=num_blocks, poison_block=poison,
        context_lens=ctx, block_tables=tables,
        cached_key=make_values(cat(ck, (0, hkv, d)), dtype),
        cached_value=make_values(cat(cv, (0, hkv, d)), dtype),
        cached_slots=np.concatenate(cslots) if cslots else np.zeros(0, np.int64),
        new_key=make_values(cat(nk, (0, hkv, d)), dtype),
        new_value=make_values(cat(nv, (0, hkv, d)), dtype),
        new_slots=np.concatenate(nslots) if nslots else np.zeros(0, np.int64),
        decode_seqs=np.arange(nseq, dtype=np.int32), decode_query=make_values(dq, dtype),
        prefill_seqs=np.zeros(0, np.int32), prefill_query=None, cu_q_lens=None,
        scale=1.0 / math.sqrt(d),
        info=dict(group_starts=starts, prefix_lens=plens,
                  shared_tokens=int(sum(p * len(m) for p, m in groups)),
                  unique_tokens=int(sum(p + sum(c - p for c in m) for p, m in groups))))


def parallel_sampling(rep: int = 0, prompts: int = 32, samples: int = 8, prompt_len: int = 2000,
                      max_new: int = 512) -> Step:
    """Llama-8B-shaped decode (Hq=32, Hkv=8, D=128, bf16) of ``prompts`` prompts
    of ``prompt_len`` tokens, each sampled ``samples`` times in parallel: every
    sample shares its prompt's blocks and has generated a uniform 1..max_new
    tokens of its own (256 sequences by default)."""
    rng = _rng(6, rep)
    groups = [(prompt_len, [prompt_len + int(x) for x in rng.integers(1, max_new, size=samples, endpoint=True)])
              for _ in range(prompts)]
    return shared_prefix(f"llama8b_parallel_sampling_{prompts}x{samples}_prompt{prompt_len}",
                         seed=6000 + rep, dtype="bf16", hq=32, hkv=8, d=128, groups=groups)


CONFIGS = {
    1: "tiny_fp32",
    2: "qwen_layer",
    3: "llama8b_continuous",
    4: "long_context",
    5: "mixed_chunked_prefill",
}
