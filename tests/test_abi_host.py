"""The C-ABI library loads without a GPU, exports every symbol the header
declares, and rejects invalid arguments before touching the device (CPU)."""
import os
import re

import pytest

import paged_kv_decode_reshape_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(pkv.library_path()),
                                reason="libpkv.so not built (run __graft_entry__.build())")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = header_functions()
    for n in ("kv_pool_create", "reshape_and_cache", "paged_attention_decode",
              "paged_attention_prefill_chunk"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound():
    lib = pkv.load()
    names = header_functions()
    assert set(names) == set(pkv.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def _status(fn, *args):
    with pytest.raises(pkv.PkvError) as e:
        fn(*args)
    return e.value.status, str(e.value)


def test_pool_bytes_and_geometry_checks():
    assert pkv.kv_pool_bytes(10, 16, 8, 128, pkv.BF16) == (10 * 8 * 16 * 128 * 2,) * 2
    assert pkv.kv_pool_bytes(3, 16, 1, 64, pkv.F32) == (3 * 16 * 64 * 4,) * 2
    # block_size 32: bf16 and e4m3 pools only
    assert pkv.kv_pool_bytes(10, 32, 8, 128, pkv.BF16) == (10 * 8 * 32 * 128 * 2,) * 2
    assert pkv.kv_pool_bytes(10, 32, 8, 64, pkv.FP8_E4M3) == (10 * 8 * 32 * 64,) * 2
    assert _status(pkv.kv_pool_bytes, 10, 32, 8, 128, pkv.F32)[0] == -2
    assert _status(pkv.kv_pool_bytes, 10, 64, 8, 128, pkv.BF16)[0] == -2
    assert _status(pkv.kv_pool_bytes, 10, 8, 8, 128, pkv.BF16)[0] == -2
    assert _status(pkv.kv_pool_bytes, 10, 16, 8, 96, pkv.BF16)[0] == -2    # head_dim 96
    assert _status(pkv.kv_pool_bytes, 0, 16, 8, 128, pkv.BF16)[0] == -1
    assert _status(pkv.kv_pool_bytes, 10, 16, 8, 128, 7)[0] == -1


def test_pool_create_validates_pointers():
    assert _status(pkv.kv_pool_create, 1, 4, 16, 1, 64, pkv.F32, [0], [256])[0] == -1
    assert _status(pkv.kv_pool_create, 1, 4, 16, 1, 64, pkv.F32, [8], [256])[0] == -1   # misaligned
    h = pkv.kv_pool_create(2, 4, 16, 1, 64, pkv.F32, [256, 512], [768, 1024])
    try:
        assert h
        # layer out of range, bad head counts, bad partition size: all rejected on the host
        st, msg = _status(pkv.paged_attention_decode, h, 2, 16, 16, 16, 16, 1, 4, 1, 1.0)
        assert st == -1 and "layer" in msg
        assert _status(pkv.paged_attention_decode, h, 0, 16, 16, 16, 16, 1, 9, 1, 1.0)[0] == -2
        assert _status(pkv.paged_attention_decode, h, 0, 16, 16, 16, 16, 1, 4, 1, 1.0, 100)[0] == -1
        assert _status(pkv.paged_attention_decode, h, 0, 16, 16, 16, 16, 1, 4, 1,
                       float("nan"))[0] == -1
        for bad_scale in (0.0, -0.125, float("inf"), 3e38):      # 3e38 * log2(e) overflows
            st, msg = _status(pkv.paged_attention_decode, h, 0, 16, 16, 16, 16, 1, 4, 1, bad_scale)
            assert st == -1 and "scale" in msg
            assert _status(pkv.paged_attention_prefill_chunk, h, 0, 16, 16, 16, 16, 16, 1, 4, 4, 4, 1,
                           bad_scale)[0] in (-1, -2)
        assert _status(pkv.reshape_and_cache, h, 0, 16, 16, 16, -1)[0] == -1
        assert _status(pkv.reshape_and_cache, h, 0, 8, 16, 16, 1)[0] == -1        # misaligned key
        # prefill runs on bf16 MFMA only
        assert _status(pkv.paged_attention_prefill_chunk, h, 0, 16, 16, 16, 16, 16, 1, 4, 4, 4, 1,
                       1.0)[0] == -2
        # zero-sized calls are no-ops that succeed without touching the device
        pkv.reshape_and_cache(h, 0, 16, 16, 16, 0)
        pkv.paged_attention_decode(h, 0, 16, 16, 16, 16, 0, 4, 1, 1.0)
    finally:
        pkv.kv_pool_destroy(h)


def test_workspace_sizing_and_check():
    h = pkv.kv_pool_create(1, 4096, 16, 8, 128, pkv.BF16, [256], [512])
    try:
        # max context 2048 tokens, 512-token partitions -> 4 partitions per sequence
        nb = pkv.paged_attention_decode_workspace_bytes(h, 3, 32, 128, 512)
        rows = 3 * 32 * 4
        counters = 4096 * 4          # completion counters at the start of every non-empty workspace
        assert nb == counters + ((rows * 8 + 15) // 16) * 16 + rows * 128 * 4
        assert pkv.paged_attention_decode_workspace_bytes(h, 3, 32, 128, -1) == 0
        assert pkv.paged_attention_decode_workspace_bytes(h, 3, 32, 32, 512) == 0   # fits one partition
        st, msg = _status(pkv.paged_attention_decode, h, 0, 256, 256, 256, 256, 3, 32, 128, 0.1,
                          512, 256, nb - 16)
        assert st == -4 and "too small" in msg
        assert _status(pkv.paged_attention_decode, h, 0, 256, 256, 256, 256, 3, 32, 128, 0.1,
                       512, None, nb)[0] == -4
    finally:
        pkv.kv_pool_destroy(h)


def test_fp8_pool_bytes_and_scales():
    assert pkv.kv_pool_bytes(10, 16, 8, 128, pkv.FP8_E4M3) == (10 * 8 * 16 * 128,) * 2
    h = pkv.kv_pool_create(2, 4, 16, 1, 64, pkv.FP8_E4M3, [256, 512], [768, 1024])
    try:
        pkv.kv_pool_set_fp8_scales(h, [0.5, 2.0], [1.0, 0.01])
        assert _status(pkv.kv_pool_set_fp8_scales, h, [1.0], [1.0])[0] == -1            # count
        for bad in (0.0, -1.0, float("inf"), float("nan"), 1e-39):                      # 1e-39: 1/x overflows
            st, msg = _status(pkv.kv_pool_set_fp8_scales, h, [1.0, bad], [1.0, 1.0])
            assert st == -1 and "layer 1" in msg
            assert _status(pkv.kv_pool_set_fp8_scales, h, [1.0, 1.0], [bad, 1.0])[0] == -1
        # an e4m3 pool takes prefill chunks (bf16 MFMA on widened codes): only the
        # NULL query below is rejected, not the dtype
        st, msg = _status(pkv.paged_attention_prefill_chunk, h, 0, 16, None, 16, 16, 16, 1, 4, 4,
                          4, 1, 1.0)
        assert st == -1 and "NULL" in msg
    finally:
        pkv.kv_pool_destroy(h)
    hb = pkv.kv_pool_create(1, 4, 16, 1, 64, pkv.BF16, [256], [512])
    try:
        assert _status(pkv.kv_pool_set_fp8_scales, hb, [1.0], [1.0])[0] == -1         # not an e4m3 pool
    finally:
        pkv.kv_pool_destroy(hb)


def test_multi_query_decode_checks():
    h = pkv.kv_pool_create(1, 4096, 16, 8, 128, pkv.BF16, [256], [512])
    hf = pkv.kv_pool_create(1, 64, 16, 8, 128, pkv.F32, [256], [512])
    try:
        # workspace: summary rows scale with the query rows per sequence
        one = pkv.paged_attention_decode_multi_workspace_bytes(h, 3, 1, 32, 128, 512)
        assert one == pkv.paged_attention_decode_workspace_bytes(h, 3, 32, 128, 512)
        rows = 3 * 32 * 4 * 4
        assert pkv.paged_attention_decode_multi_workspace_bytes(h, 3, 4, 32, 128, 512) == \
            4096 * 4 + ((rows * 8 + 15) // 16) * 16 + rows * 128 * 4
        assert _status(pkv.paged_attention_decode_multi_workspace_bytes, h, 3, 0, 32, 128, 512)[0] == -1
        # more rows x heads per KV head than the 16 matrix-core columns: run as
        # equal-length prefill chunks, which need no workspace
        assert pkv.paged_attention_decode_multi_workspace_bytes(h, 3, 5, 32, 128, 0) == 0
        assert pkv.paged_attention_decode_multi_workspace_bytes(h, 3, 16, 32, 128, 512) == 0
        assert _status(pkv.paged_attention_decode_multi, h, 0, 16, 16, 0, 16, 16, 1, 32, 4, 1.0)[0] == -1
        # fp32 pools take one query row per sequence only
        st, msg = _status(pkv.paged_attention_decode_multi, hf, 0, 16, 16, 2, 16, 16, 1, 32, 4, 1.0)
        assert st == -2 and "bf16" in msg
        pkv.paged_attention_decode_multi(h, 0, 16, 16, 4, 16, 16, 0, 32, 4, 1.0)   # no sequences: no-op
    finally:
        pkv.kv_pool_destroy(h)
        pkv.kv_pool_destroy(hf)


def test_copy_blocks_checks():
    h = pkv.kv_pool_create(2, 8, 16, 2, 64, pkv.BF16, [256, 512], [768, 1024])
    try:
        pkv.copy_blocks(h, 16, 0)                                  # no pairs: no-op
        assert _status(pkv.copy_blocks, h, 16, -1)[0] == -1
        assert _status(pkv.copy_blocks, h, None, 2)[0] == -1
        assert _status(pkv.copy_blocks, h, 18, 2)[0] == -1         # misaligned pairs
    finally:
        pkv.kv_pool_destroy(h)


def test_shared_prefix_decode_checks():
    h = pkv.kv_pool_create(1, 4096, 16, 8, 128, pkv.BF16, [256], [512])
    hf = pkv.kv_pool_create(1, 64, 16, 8, 128, pkv.F32, [256], [512])
    try:
        # workspace: completion counters, summaries of every (sequence, head,
        # 512-token piece), one int32 per sequence, then the balanced split's
        # slots (two per wave, G heads each) and descriptors; at most one wave
        # per window
        rows = 3 * 32 * 4                                         # 128 blocks = 2048 tokens = 4 pieces
        waves = 3 * 8 * 2048 // 64
        r16 = lambda x: (x + 15) // 16 * 16
        want = (4096 * 4 + r16(rows * 8) + rows * 128 * 4 + 16 + r16(waves * 2 * 4 * 8) +
                waves * 2 * 4 * 128 * 4 + waves * 2 * 32)
        assert pkv.paged_attention_decode_shared_workspace_bytes(h, 3, 32, 128, 0) == want
        assert pkv.paged_attention_decode_shared_workspace_bytes(h, 3, 32, 128, 512) == want
        assert pkv.paged_attention_decode_shared_workspace_bytes(h, 3, 32, 128, 256) > want
        assert _status(pkv.paged_attention_decode_shared_workspace_bytes, h, 3, 32, 128, -1)[0] == -1
        assert _status(pkv.paged_attention_decode_shared_workspace_bytes, h, 3, 32, 128, 100)[0] == -1
        args = (0, 16, 16, 16, 16, 16, 16)   # layer, out, query, tables, lens, group_starts, prefix_lens
        # groups and their largest size must be within [1, num_seqs]
        assert _status(pkv.paged_attention_decode_shared, h, *args, 4, 0, 1, 32, 128, 1.0)[0] == -1
        assert _status(pkv.paged_attention_decode_shared, h, *args, 4, 5, 1, 32, 128, 1.0)[0] == -1
        assert _status(pkv.paged_attention_decode_shared, h, *args, 4, 2, 0, 32, 128, 1.0)[0] == -1
        # the workspace is required
        assert _status(pkv.paged_attention_decode_shared, h, *args, 4, 2, 2, 32, 128, 1.0)[0] == -4
        # null group arrays are rejected
        st, msg = _status(pkv.paged_attention_decode_shared, h, 0, 16, 16, 16, 16, None, 16, 4, 2, 2, 32, 128,
                          1.0)
        assert st == -1 and "group_starts" in msg
        # fp32 pools: the shared products run on the matrix cores
        st, msg = _status(pkv.paged_attention_decode_shared, hf, *args, 4, 2, 2, 32, 128, 1.0)
        assert st == -2 and "bf16" in msg
        pkv.paged_attention_decode_shared(h, *args, 0, 0, 0, 32, 128, 1.0)   # no sequences: no-op
    finally:
        pkv.kv_pool_destroy(h)
        pkv.kv_pool_destroy(hf)


def test_fused_append_decode_checks():
    h = pkv.kv_pool_create(1, 64, 16, 8, 128, pkv.BF16, [256], [512])
    hf = pkv.kv_pool_create(1, 64, 16, 8, 128, pkv.F32, [256], [512])
    try:
        args = (0, 16, 16)                       # layer, out, query
        # key and value are required, 16-byte aligned
        assert _status(pkv.paged_attention_decode_append, h, *args, None, 16, 16, 16, 4, 32, 4, 1.0)[0] == -1
        assert _status(pkv.paged_attention_decode_append, h, *args, 16, 24, 16, 16, 4, 32, 4, 1.0)[0] == -1
        # fp32 pools run the lane-per-token decode, which has no fused append
        st, msg = _status(pkv.paged_attention_decode_append, hf, *args, 16, 16, 16, 16, 4, 32, 4, 1.0, -1)
        assert st == -2 and "bf16" in msg
        # the usual decode checks apply (heads not a multiple of KV heads)
        assert _status(pkv.paged_attention_decode_append, h, *args, 16, 16, 16, 16, 4, 30, 4, 1.0)[0] == -1
        pkv.paged_attention_decode_append(h, *args, 16, 16, 16, 16, 0, 32, 4, 1.0)   # no sequences: no-op
    finally:
        pkv.kv_pool_destroy(h)
        pkv.kv_pool_destroy(hf)


def test_enum_arguments_outside_their_range_are_rejected():
    # values outside pkv_dtype / pkv_kernel_kind are read as integers and rejected
    assert _status(pkv.kv_pool_create, 1, 4, 16, 1, 64, 5, [256], [512])[0] == -1
    assert _status(pkv.kv_pool_create, 1, 4, 16, 1, 64, -3, [256], [512])[0] == -1
    for kind in (-1, 6, 1 << 20):
        assert _status(pkv.pkv_timing_read, kind)[0] == -1
        assert _status(pkv.pkv_timing_read_launches, kind, 4)[0] == -1


def test_debug_read_errors_in_the_release_library():
    if os.environ.get("PKV_LIBRARY_PATH"):
        pytest.skip("a substitute library is loaded")
    st, msg = _status(pkv.pkv_debug_read_errors)
    assert st == -2 and "PKV_DEBUG" in msg


def test_gather_checksum_validates_on_the_host():
    h = pkv.kv_pool_create(1, 4, 16, 1, 64, pkv.F32, [256], [768])
    try:
        # checksum, block_tables, context_lens, workspace: fake device addresses
        args = (16, 32, 48)
        assert _status(pkv.paged_kv_gather_checksum, h, 1, *args, 1, 1, 64, 64)[0] == -1      # layer
        assert _status(pkv.paged_kv_gather_checksum, h, 0, *args, -1, 1, 64, 64)[0] == -1     # num_seqs
        assert _status(pkv.paged_kv_gather_checksum, h, 0, *args, 8193, 1, 64, 1 << 20)[0] == -2
        assert _status(pkv.paged_kv_gather_checksum, h, 0, *args, 1, 0, 64, 64)[0] == -1      # max blocks
        assert _status(pkv.paged_kv_gather_checksum, h, 0, *args, 4, 1, 64, 16)[0] == -4      # workspace
        assert _status(pkv.paged_kv_gather_checksum, h, 0, *args, 4, 1, None, 64)[0] == -1
        assert _status(pkv.paged_kv_gather_checksum, h, 0, 18, 32, 48, 4, 1, 64, 64)[0] == -1  # misaligned
        pkv.paged_kv_gather_checksum(h, 0, *args, 0, 1, 64, 64)   # no sequences: a no-op
    finally:
        pkv.kv_pool_destroy(h)
