"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
every one of them fails at least one pin. This shows the pins are sharp enough
to catch a dropped term, a wrong index or a transposed operand."""
import os
import types

import pytest

import oracle as real_oracle
from oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(real_oracle.__file__), "paged_attention.py")

MUTANTS = {
    "gqa_modulo_grouping": ("h = i // group\n        s = scale", "h = i % hkv\n        s = scale"),
    "scale_dropped": ("s = scale * (k[:, h, :] @ q[i])", "s = (k[:, h, :] @ q[i])"),
    "no_max_subtraction": ("e = np.exp(s - s.max())", "e = np.exp(s)"),
    "normalizer_dropped": ("return e / e.sum()", "return e"),
    "gather_one_extra_token": ("[:ctx]\n", "[:ctx + 1]\n"),
    "gather_one_token_short": ("[:ctx]\n", "[:max(ctx - 1, 1)]\n"),
    "causal_excludes_diagonal": ("visible = ctx - t + r + 1", "visible = ctx - t + r"),
    "causal_from_chunk_start": ("visible = ctx - t + r + 1", "visible = r + 1"),
    "slot_offset_swapped": ("blk, off = slots[keep] // bs, slots[keep] % bs",
                            "blk, off = slots[keep] % bs, slots[keep] // bs"),
    "v_uses_k": ("out[i] = _softmax_row(s) @ v[:, h, :]", "out[i] = _softmax_row(s) @ k[:, h, :]"),
    "combine_no_rescale": ("w1 = np.exp(m1 - m) * l1", "w1 = l1"),
    "combine_wrong_sign": ("w2 = np.exp(m2 - m) * l2", "w2 = np.exp(m - m2) * l2"),
    "kv_bytes_no_factor_two": ("vectors_per_token = 2 * layers * kv_heads", "vectors_per_token = layers * kv_heads"),
    "kv_bytes_dtype_dropped": ("bytes_per_vector = head_dim * dtype_bytes", "bytes_per_vector = head_dim"),
    "blocks_floor": ("return (int(ctx) + block_size - 1) // block_size", "return int(ctx) // block_size"),
    "negative_slots_written": ("keep = slots >= 0", "keep = slots >= -1"),
    "copy_reversed": ("pool_k[dst] = pool_k[src]\n        pool_v[dst] = pool_v[src]",
                      "pool_k[src] = pool_k[dst]\n        pool_v[src] = pool_v[dst]"),
    "copy_k_only": ("pool_v[dst] = pool_v[src]", "pass"),
}


def _mutant(old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
