"""CPU oracle for paged-KV attention in one continuous-batching step.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never imports, links
or calls it, and the two share no code: this file is written from the
definitions on the pages, not from the kernels.

Everything here is plain numpy, computed in float64 from the exact stored
input values (bf16 or fp32 values widened without rounding). It is slow and
meant to be read against the pages:

  * Scaled dot-product attention and the row softmax with the maximum
    subtracted: "LLM 7 - Efficient LLM Serving", section 2 "FlashAttention",
    subsections "Attention Is Simple Algebra with Expensive Data Movement" and
    "Online Softmax Makes Tiling Possible". The page's formulas were lost in
    extraction; the prose fixes them as softmax(scale * q K^T) V with the row
    maximum subtracted before exponentiating.
  * Online-softmax summaries (running maximum, normalizer, normalized output)
    and their pairwise combination: same page, "Online Softmax Makes Tiling
    Possible"; used here for the split of one decode row along the KV axis
    ("The Serving Playbook", section "Kernel fusion, briefly", the
    Flash-Decoding bullet, and section "The block table lives in the hottest
    kernel in the system": partial softmax per piece, then a second pass that
    rescales the partials into the answer).
  * Paging: a block table maps a sequence's logical blocks to physical blocks
    of a shared pool; only the last block may be partial ("LLM 7 - Efficient
    LLM Serving", section 3, "Paging the Cache"; "The Serving Playbook",
    section "Paged KV cache").
  * Append before attend: the step's new keys/values are written to their
    slots, then the step's queries attend over the cache including them
    ("LLM 7 - Efficient LLM Serving", section 3, "What the Cache Stores";
    slot mappings: "The Serving Playbook", "CUDA graphs and the CPU you forgot
    about").
  * Grouped-query attention: query heads in contiguous groups share one KV
    head ("Inference Engineering, Part 2: What Actually Runs the Model",
    section "The KV cache").
  * Prefill chunk: the chunk attends causally to everything already cached
    plus itself ("The Serving Playbook", sections "Chunked prefill" and
    "Prefill and decode want different machines").
  * KV size: 2 x layers x kv_heads x head_dim x dtype_bytes x seq_len x batch
    ("Inference Engineering, Part 2", section "The KV cache").

Pool layout used by the oracle (its own, not the library's):
  pool[num_blocks, block_size, num_kv_heads, head_dim].
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# KV size ("Inference Engineering, Part 2", section "The KV cache")
# ---------------------------------------------------------------------------

def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int,
                   seq_len: int = 1, batch: int = 1) -> int:
    """Bytes of K plus V for ``batch`` sequences of ``seq_len`` tokens.

    Derivation: a cached token keeps, in every layer and for every KV head,
    one key vector and one value vector of head_dim elements. Its bytes are
    the number of stored vectors times the bytes of one vector; a batch holds
    seq_len * batch such tokens.
    """
    vectors_per_token = 2 * layers * kv_heads            # a key and a value per (layer, KV head)
    bytes_per_vector = head_dim * dtype_bytes
    return vectors_per_token * bytes_per_vector * seq_len * batch


def blocks_for(ctx: int, block_size: int) -> int:
    """Blocks a sequence of ``ctx`` tokens occupies: only the last may be partial
    ("LLM 7 - Efficient LLM Serving", section 3, "Paging the Cache")."""
    return (int(ctx) + block_size - 1) // block_size


# ---------------------------------------------------------------------------
# Pool, append ("reshape_and_cache") and gather
# ---------------------------------------------------------------------------

def new_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
             dtype=np.float64) -> np.ndarray:
    """A pool whose unwritten slots are NaN, so reading one poisons the result."""
    return np.full((num_blocks, block_size, num_kv_heads, head_dim), np.nan, dtype=dtype)


def append(pool_k: np.ndarray, pool_v: np.ndarray, key: np.ndarray, value: np.ndarray,
           slot_mapping: np.ndarray) -> None:
    """Write token t's key/value rows (all KV heads) into slot ``slot_mapping[t]``.

    slot = physical_block * block_size + offset; a negative slot is skipped.
    key, value: [num_tokens, num_kv_heads, head_dim].
    """
    bs = pool_k.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    blk, off = slots[keep] // bs, slots[keep] % bs
    pool_k[blk, off] = np.asarray(key)[keep]
    pool_v[blk, off] = np.asarray(value)[keep]


def copy_blocks(pool_k: np.ndarray, pool_v: np.ndarray, pairs) -> None:
    """Copy-on-write ("LLM 7 - Efficient LLM Serving", 3., "Sharing and
    Preemption"; "The Serving Playbook", "Sharing is a reference count"): for
    each (source, destination) pair, the destination block becomes a copy of
    the source block, all slots and KV heads, in K and in V."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        pool_k[dst] = pool_k[src]
        pool_v[dst] = pool_v[src]


def gather(pool: np.ndarray, block_table_row: np.ndarray, ctx: int) -> np.ndarray:
    """Logical positions 0..ctx-1 of one sequence as a contiguous [ctx, Hkv, D] array.

    Logical block j of the sequence lives in physical block block_table_row[j].
    """
    bs = pool.shape[1]
    nb = blocks_for(ctx, bs)
    ids = np.asarray(block_table_row[:nb], dtype=np.int64)
    blocks = pool[ids]                                    # [nb, bs, Hkv, D]
    return blocks.reshape(nb * bs, pool.shape[2], pool.shape[3])[:ctx]


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _softmax_row(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum exp(s - max s), in float64."""
    e = np.exp(s - s.max())
    return e / e.sum()


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One query position, all query heads, over n keys.

    q: [Hq, D]; k, v: [n, Hkv, D]. Query head i uses KV head i // (Hq // Hkv).
    With n = 0 the output is defined as zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    if k.shape[0] == 0:
        return out
    for i in range(hq):
        h = i // group
        s = scale * (k[:, h, :] @ q[i])                   # [n]
        out[i] = _softmax_row(s) @ v[:, h, :]
    return out


def paged_decode(query: np.ndarray, pool_k: np.ndarray, pool_v: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 seqs=None) -> np.ndarray:
    """Decode attention: sequence b's single query attends to its first
    context_lens[b] cached positions (this step's token included).

    query: [B, Hq, D]. Returns float64 [B, Hq, D] (rows not in ``seqs`` stay 0).
    """
    query = np.asarray(query)
    out = np.zeros(query.shape, dtype=np.float64)
    for b in (range(query.shape[0]) if seqs is None else seqs):
        ctx = int(context_lens[b])
        k = gather(pool_k, block_tables[b], ctx)
        v = gather(pool_v, block_tables[b], ctx)
        out[b] = attend(query[b], k, v, scale)
    return out


def paged_prefill_chunk(query: np.ndarray, cu_q_lens: np.ndarray, pool_k: np.ndarray,
                        pool_v: np.ndarray, block_tables: np.ndarray,
                        context_lens: np.ndarray, scale: float, rows=None) -> np.ndarray:
    """Causal attention of a prefill chunk over the paged cache.

    Sequence s owns query rows cu_q_lens[s]..cu_q_lens[s+1]-1 (T rows). Its
    chunk's keys/values are already appended, so the cache holds ctx =
    context_lens[s] tokens and chunk row r sits at absolute position
    ctx - T + r; it attends to positions 0..ctx - T + r inclusive.

    query: [total_q, Hq, D]. Returns float64 [total_q, Hq, D]. ``rows``
    optionally restricts the computation to the listed global query rows.
    """
    query = np.asarray(query)
    out = np.zeros(query.shape, dtype=np.float64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for s in range(len(cu_q_lens) - 1):
        lo, hi = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        t = hi - lo
        if t == 0:
            continue
        ctx = int(context_lens[s])
        k = gather(pool_k, block_tables[s], ctx)
        v = gather(pool_v, block_tables[s], ctx)
        for r in range(t):
            if wanted is not None and lo + r not in wanted:
                continue
            visible = ctx - t + r + 1
            out[lo + r] = attend(query[lo + r], k[:visible], v[:visible], scale)
    return out


# ---------------------------------------------------------------------------
# Online softmax split along the KV axis (the method's own reduction)
# ---------------------------------------------------------------------------

def softmax_summary(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Summary of one piece of a single head's row: (m, l, o).

    m = max score, l = sum exp(s - m), o = sum exp(s - m) v / l (normalized).
    An empty piece is (-inf, 0, zeros). q: [D]; k, v: [n, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(v.shape[1], dtype=np.float64)
    s = scale * (k @ q)
    m = float(s.max())
    e = np.exp(s - m)
    l = float(e.sum())
    return m, l, (e @ v) / l


def combine(a, b):
    """Merge two summaries: the larger maximum wins and each side's normalizer and
    output are rescaled by exp(its max - combined max) before adding."""
    m1, l1, o1 = a
    m2, l2, o2 = b
    if l1 == 0.0:
        return b
    if l2 == 0.0:
        return a
    m = max(m1, m2)
    w1 = np.exp(m1 - m) * l1
    w2 = np.exp(m2 - m) * l2
    l = w1 + w2
    return m, l, (w1 * o1 + w2 * o2) / l


def attend_split(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 bounds) -> np.ndarray:
    """Single-query GQA attention computed piecewise over the KV axis.

    ``bounds`` = increasing cut points 0 = c0 <= c1 <= ... <= cP = n; piece p
    covers keys [c_p, c_{p+1}). Pieces are summarized independently and then
    folded left to right with ``combine``. Returns [Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    for i in range(hq):
        h = i // group
        acc = (-np.inf, 0.0, np.zeros(d, dtype=np.float64))
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            acc = combine(acc, softmax_summary(q[i], k[lo:hi, h], v[lo:hi, h], scale))
        out[i] = acc[2]
    return out
