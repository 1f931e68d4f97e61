"""Drive the C-ABI library on the GPU from a generated step (test plumbing).

torch provides device memory and the stream; every computation is a call into
libpkv. ``decode_pool`` reads a device pool back and rearranges it into the
oracle's [num_blocks, block_size, num_kv_heads, head_dim] order, following
the layout the library header documents (an independent reading of that
text, not library code).
"""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_decode_reshape_amd as pkv
from paged_kv_decode_reshape_amd import workloads as W

DEV = "cuda:0"
PKV_DT = {"bf16": pkv.BF16, "f32": pkv.F32, "fp8": pkv.FP8_E4M3}
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
POISON_BITS = {"bf16": 0xFFFF, "f32": 0xFFFFFFFF, "fp8": 0xFF}   # NaN patterns for never-written slots
POOL_BYTES = {"bf16": 2, "f32": 4, "fp8": 1}
X = {"bf16": 8, "f32": 4, "fp8": 16}     # elements per 16-byte K vector


def to_device(values: W.Values) -> torch.Tensor:
    if values.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(values.bits).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(values.bits))
    return t.to(DEV)


def int_tensor(a, dtype=torch.int32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)


def to_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def raw_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.detach().cpu().numpy()
    return t.detach().view(torch.int32).cpu().numpy().view(np.uint32)


def workspace(ws, need: int):
    """A fresh zero-filled decode workspace of ``need`` bytes, or the given one
    (which must be large enough): (tensor, bytes passed to the call)."""
    if ws is None:
        return torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV), need
    assert ws.numel() >= need, (ws.numel(), need)
    return ws, ws.numel()


COUNTER_BYTES = 4096 * 4    # completion counters at the start of every decode workspace


class DevicePool:
    """K/V pools in HBM (one pair per layer), wrapped in a library pool handle.

    ``kv="fp8"`` makes an e4m3 pool for a bf16 step, with per-layer scales
    ``k_scales`` / ``v_scales`` (lists, one per layer)."""

    def __init__(self, step: W.Step, num_layers: int = 1, kv: str | None = None,
                 k_scales=None, v_scales=None):
        self.step = step
        s = step
        self.kv = s.dtype if kv is None else kv
        assert self.kv == s.dtype or (self.kv == "fp8" and s.dtype == "bf16")
        self.elems = s.num_blocks * s.num_kv_heads * s.block_size * s.head_dim
        kb, vb = pkv.kv_pool_bytes(s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim,
                                   PKV_DT[self.kv])
        assert kb == vb == self.elems * POOL_BYTES[self.kv]
        self.k = [self._poisoned() for _ in range(num_layers)]
        self.v = [self._poisoned() for _ in range(num_layers)]
        self.handle = pkv.kv_pool_create(num_layers, s.num_blocks, s.block_size, s.num_kv_heads,
                                         s.head_dim, PKV_DT[self.kv], self.k, self.v)
        if k_scales is not None:
            pkv.kv_pool_set_fp8_scales(self.handle, k_scales, v_scales)

    def _poisoned(self) -> torch.Tensor:
        if self.kv == "fp8":
            return torch.full((self.elems,), 0xFF, dtype=torch.uint8, device=DEV)
        if self.kv == "bf16":
            t = torch.full((self.elems,), -1, dtype=torch.int16, device=DEV)
            return t.view(torch.bfloat16)
        t = torch.full((self.elems,), -1, dtype=torch.int32, device=DEV)
        return t.view(torch.float32)

    def close(self):
        if self.handle:
            pkv.kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- appends ----
    def append(self, key: W.Values, value: W.Values, slots: np.ndarray, layer: int = 0):
        n = len(slots)
        if n == 0:
            return
        kd, vd = to_device(key), to_device(value)
        sd = int_tensor(slots, torch.int64)
        pkv.reshape_and_cache(self.handle, layer, kd, vd, sd, n)

    def fill(self, include_new: bool = True, layer: int = 0):
        s = self.step
        self.append(s.cached_key, s.cached_value, s.cached_slots, layer)
        if include_new:
            self.append(s.new_key, s.new_value, s.new_slots, layer)

    # ---- attention ----
    def decode(self, partition_size: int | None = None, query=None, tables=None, lens=None,
               scale=None, layer: int = 0, ws=None):
        s = self.step
        bt, cl = s.decode_inputs()
        bt = bt if tables is None else tables
        cl = cl if lens is None else lens
        q = to_device(s.decode_query) if query is None else query
        nseq = len(cl)
        out = torch.empty((nseq, s.num_q_heads, s.head_dim), dtype=TORCH_DT[s.dtype], device=DEV)
        part = s.partition_size if partition_size is None else partition_size
        wsb = pkv.paged_attention_decode_workspace_bytes(self.handle, nseq, s.num_q_heads,
                                                         bt.shape[1], part)
        ws, wsb = workspace(ws, wsb)
        pkv.paged_attention_decode(self.handle, layer, out, q, int_tensor(bt), int_tensor(cl),
                                   nseq, s.num_q_heads, bt.shape[1],
                                   s.scale if scale is None else scale, part, ws, wsb)
        return out

    def decode_multi(self, q_per_seq: int, partition_size: int | None = None, layer: int = 0, ws=None):
        """Several query rows per sequence: the step's prefill chunks, all of
        length q_per_seq, through paged_attention_decode_multi."""
        s = self.step
        bt, cl = s.prefill_inputs()
        assert np.all(np.diff(s.cu_q_lens) == q_per_seq)
        q = to_device(s.prefill_query)
        nseq = len(cl)
        out = torch.empty((nseq * q_per_seq, s.num_q_heads, s.head_dim), dtype=TORCH_DT[s.dtype], device=DEV)
        part = s.partition_size if partition_size is None else partition_size
        wsb = pkv.paged_attention_decode_multi_workspace_bytes(self.handle, nseq, q_per_seq, s.num_q_heads,
                                                               bt.shape[1], part)
        ws, wsb = workspace(ws, wsb)
        pkv.paged_attention_decode_multi(self.handle, layer, out, q, q_per_seq, int_tensor(bt), int_tensor(cl),
                                         nseq, s.num_q_heads, bt.shape[1], s.scale, part, ws, wsb)
        return out

    def decode_shared(self, partition_size: int = 0, groups=None, prefix_lens=None, layer: int = 0, ws=None):
        """Decode through paged_attention_decode_shared with the step's sharing
        groups (``info['group_starts']``, ``info['prefix_lens']``) unless given."""
        s = self.step
        bt, cl = s.decode_inputs()
        gs = s.info["group_starts"] if groups is None else np.asarray(groups, np.int32)
        pl = s.info["prefix_lens"] if prefix_lens is None else np.asarray(prefix_lens, np.int32)
        q = to_device(s.decode_query)
        nseq = len(cl)
        out = torch.empty((nseq, s.num_q_heads, s.head_dim), dtype=TORCH_DT[s.dtype], device=DEV)
        wsb = pkv.paged_attention_decode_shared_workspace_bytes(self.handle, nseq, s.num_q_heads,
                                                                bt.shape[1], partition_size)
        ws, wsb = workspace(ws, wsb)
        ng = len(gs) - 1
        max_group = int(np.max(np.diff(gs))) if ng else 1
        pkv.paged_attention_decode_shared(self.handle, layer, out, q, int_tensor(bt), int_tensor(cl),
                                          int_tensor(gs), int_tensor(pl), nseq, ng, max_group,
                                          s.num_q_heads, bt.shape[1], s.scale, partition_size, ws, wsb)
        return out

    def prefill(self, layer: int = 0):
        s = self.step
        bt, cl = s.prefill_inputs()
        q = to_device(s.prefill_query)
        total = int(s.cu_q_lens[-1])
        out = torch.empty((total, s.num_q_heads, s.head_dim), dtype=TORCH_DT[s.dtype], device=DEV)
        max_q = int(np.max(np.diff(s.cu_q_lens)))
        pkv.paged_attention_prefill_chunk(self.handle, layer, out, q, int_tensor(s.cu_q_lens),
                                          int_tensor(bt), int_tensor(cl), len(cl), total, max_q,
                                          s.num_q_heads, bt.shape[1], s.scale)
        return out

    # ---- read back ----
    def decode_pool(self, layer: int = 0):
        """(K, V) as [num_blocks, block_size, Hkv, D] raw bit arrays."""
        s = self.step
        x = X[self.kv]
        nb, hkv, d, bs = s.num_blocks, s.num_kv_heads, s.head_dim, s.block_size
        k = raw_bits(self.k[layer]).reshape(nb, hkv, d // x, bs, x)
        k = k.transpose(0, 3, 1, 2, 4).reshape(nb, bs, hkv, d)
        v = raw_bits(self.v[layer]).reshape(nb, hkv, bs, d).transpose(0, 2, 1, 3)
        return np.ascontiguousarray(k), np.ascontiguousarray(v)


def bf16_tol(ref: np.ndarray):
    return 2e-3 + 1e-2 * np.abs(ref)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """The parity bar: bf16 |err| <= 2e-3 + 1e-2|ref|; fp32 |err| <= 1e-5."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = bf16_tol(ref) if dtype == "bf16" else np.full(ref.shape, 1e-5)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at "
                             f"{i}: got {got[i]!r} ref {ref[i]!r} err {err[i]:.3g} tol {tol[i]:.3g}")
    return float(err.max())
