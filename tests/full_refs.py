"""Full-size oracle references for the GPU parity tests (test plumbing).

The large workloads (the B=256 lognormal Llama-8B layer, the mixed
chunked-prefill step, the parallel-sampling step) take tens of seconds to
generate and to run through the oracle. Each step and each reference is
built once per test process and shared by every test that compares against
it. Every reference covers every output row: nothing here samples.

References come only from ``oracle`` (fp64, the exact stored values); an
e4m3 pool's reference is the oracle's attention over the value each code
stands for (the oracle's own encoder, decoded, times the layer's scale).
"""
from __future__ import annotations

import functools

import numpy as np

import oracle
from oracle import fp8 as f8
from paged_kv_decode_reshape_amd import workloads as W


@functools.lru_cache(maxsize=None)
def step(kind: str) -> W.Step:
    """kind: 'llama8b' (B=256 lognormal, 16-token blocks), 'llama8b_bs32',
    'mixed' (512-token chunk on 2048 cached + 128 decodes), 'parallel'
    (32 prompts x 8 samples sharing prompt blocks)."""
    if kind == "llama8b":
        return W.llama8b_continuous()
    if kind == "llama8b_bs32":
        return W.llama8b_continuous(block_size=32)
    if kind == "mixed":
        return W.mixed_chunked_prefill()
    if kind == "parallel":
        return W.parallel_sampling()
    raise KeyError(kind)


def _pools(s: W.Step, k_scale=None, v_scale=None):
    """The oracle's pools after the step's appends (cached tokens, then the
    step's own). With scales: the values an e4m3 pool holds for them."""
    pk = oracle.new_pool(s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim)
    pv = oracle.new_pool(s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim)
    for key, value, slots in ((s.cached_key, s.cached_value, s.cached_slots),
                              (s.new_key, s.new_value, s.new_slots)):
        k, v = key.f32, value.f32
        if k_scale is not None:
            k, v = f8.quantize_dequantize(k, k_scale), f8.quantize_dequantize(v, v_scale)
        oracle.append(pk, pv, k, v, slots)
    return pk, pv


def refs(kind: str, k_scale=None, v_scale=None):
    """(decode reference [B, Hq, D] or None, prefill reference [total_q, Hq, D] or None),
    every row, float64."""
    return _refs(kind, None if k_scale is None else float(k_scale), None if v_scale is None else float(v_scale))


@functools.lru_cache(maxsize=None)
def _refs(kind, k_scale, v_scale):
    s = step(kind)
    pk, pv = _pools(s, k_scale, v_scale)
    dec = pre = None
    if len(s.decode_seqs):
        bt, cl = s.decode_inputs()
        dec = oracle.paged_decode(s.decode_query.f32, pk, pv, bt, cl, s.scale)
    if s.cu_q_lens is not None:
        bt, cl = s.prefill_inputs()
        pre = oracle.paged_prefill_chunk(s.prefill_query.f32, s.cu_q_lens, pk, pv, bt, cl, s.scale)
    del pk, pv
    return dec, pre


def decode_ref(kind: str, k_scale=None, v_scale=None) -> np.ndarray:
    return refs(kind, k_scale, v_scale)[0]


def prefill_ref(kind: str, k_scale=None, v_scale=None) -> np.ndarray:
    return refs(kind, k_scale, v_scale)[1]
