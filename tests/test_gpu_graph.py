"""A whole layer-step captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed gives the eager step's outputs bit for bit.

The library only enqueues kernels on the caller's stream and never allocates,
synchronizes or clears memory with a memset, so a step can be captured. Each
replay is checked against the eager result, with eager work and
synchronizations between replays.
"""
import numpy as np
import pytest

from paged_kv_decode_reshape_amd import workloads as W
import paged_kv_decode_reshape_amd as pkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_harness import DEV, DevicePool, int_tensor, to_device


def _step_fn(pool, step, kv, ws, outs, tq):
    s = step
    k_new, v_new = to_device(s.new_key), to_device(s.new_value)
    slots = int_tensor(s.new_slots, torch.int64)
    if tq == 1:
        bt, cl = s.decode_inputs()
        q = to_device(s.decode_query)
    else:
        bt, cl = s.prefill_inputs()
        q = to_device(s.prefill_query)
    bt_d, cl_d = int_tensor(bt), int_tensor(cl)
    nseq = len(cl)

    def run():
        st = torch.cuda.current_stream()
        pkv.reshape_and_cache(pool.handle, 0, k_new, v_new, slots, len(s.new_slots), st)
        pkv.paged_attention_decode_multi(pool.handle, 0, outs, q, tq, bt_d, cl_d, nseq, s.num_q_heads,
                                         bt.shape[1], s.scale, 0, ws, ws.numel(), st)
    return run, nseq


@pytest.mark.parametrize("kv,tq", [("bf16", 1), ("fp8", 1), ("bf16", 4)])
def test_captured_step_matches_eager(kv, tq):
    rng = np.random.default_rng(3)
    ctx = W.lognormal_lengths(rng, 48).astype(int).tolist()
    q_lens = [tq] * len(ctx) if tq > 1 else None
    step = W.custom(f"graph_{kv}_{tq}", seed=900 + tq, dtype="bf16", hq=32, hkv=8, d=128, ctx=ctx, q_lens=q_lens)
    pool = DevicePool(step, kv=None if kv == "bf16" else "fp8",
                      k_scales=None if kv == "bf16" else [1 / 80], v_scales=None if kv == "bf16" else [1 / 80])
    pool.append(step.cached_key, step.cached_value, step.cached_slots)
    bt, cl = (step.decode_inputs() if tq == 1 else step.prefill_inputs())
    nseq = len(cl)
    wsb = pkv.paged_attention_decode_multi_workspace_bytes(pool.handle, nseq, tq, step.num_q_heads,
                                                           bt.shape[1], 0)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=DEV)
    out_eager = torch.empty((nseq * tq, step.num_q_heads, step.head_dim), dtype=torch.bfloat16, device=DEV)
    out_graph = torch.empty_like(out_eager)
    run_eager, _ = _step_fn(pool, step, kv, ws, out_eager, tq)
    run_graph, _ = _step_fn(pool, step, kv, ws, out_graph, tq)
    run_eager()
    torch.cuda.synchronize()
    ref = out_eager.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_graph()                         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_graph()
    for i in range(4):
        out_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_graph.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        run_eager()                         # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out_eager.view(torch.int16), ref.view(torch.int16))


def _replay_check(run_eager, run_graph, out_eager, out_graph):
    run_eager()
    torch.cuda.synchronize()
    ref = out_eager.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_graph()                         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_graph()
    for i in range(4):
        out_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_graph.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        run_eager()                         # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out_eager.view(torch.int16), ref.view(torch.int16))


def test_captured_shared_prefix_decode_matches_eager():
    """paged_attention_decode_shared captured with its append: the groups and
    prefix lengths are device buffers, so replays equal the eager step."""
    groups = [(300, [301, 320, 400, 900]), (0, [50]), (1000, [1001 + 13 * i for i in range(9)])]
    step = W.shared_prefix("graph_shared", seed=931, dtype="bf16", hq=32, hkv=8, d=128, groups=groups)
    pool = DevicePool(step)
    pool.append(step.cached_key, step.cached_value, step.cached_slots)
    bt, cl = step.decode_inputs()
    nseq = len(cl)
    gs, pl = int_tensor(step.info["group_starts"]), int_tensor(step.info["prefix_lens"])
    max_group = int(np.max(np.diff(step.info["group_starts"])))
    wsb = pkv.paged_attention_decode_shared_workspace_bytes(pool.handle, nseq, step.num_q_heads, bt.shape[1], 0)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=DEV)
    k_new, v_new = to_device(step.new_key), to_device(step.new_value)
    slots = int_tensor(step.new_slots, torch.int64)
    q, bt_d, cl_d = to_device(step.decode_query), int_tensor(bt), int_tensor(cl)
    outs = [torch.empty((nseq, step.num_q_heads, step.head_dim), dtype=torch.bfloat16, device=DEV) for _ in range(2)]

    def make(out):
        def run():
            st = torch.cuda.current_stream()
            pkv.reshape_and_cache(pool.handle, 0, k_new, v_new, slots, len(step.new_slots), st)
            pkv.paged_attention_decode_shared(pool.handle, 0, out, q, bt_d, cl_d, gs, pl, nseq, len(groups), max_group,
                                              step.num_q_heads, bt.shape[1], step.scale, 0, ws, wsb, st)
        return run
    _replay_check(make(outs[0]), make(outs[1]), outs[0], outs[1])


def test_captured_block32_step_matches_eager():
    rng = np.random.default_rng(4)
    ctx = W.lognormal_lengths(rng, 48).astype(int).tolist()
    step = W.custom("graph_bs32", seed=932, dtype="bf16", hq=32, hkv=8, d=128, ctx=ctx, block_size=32)
    pool = DevicePool(step)
    pool.append(step.cached_key, step.cached_value, step.cached_slots)
    bt, cl = step.decode_inputs()
    nseq = len(cl)
    wsb = pkv.paged_attention_decode_multi_workspace_bytes(pool.handle, nseq, 1, step.num_q_heads, bt.shape[1], 0)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=DEV)
    outs = [torch.empty((nseq, step.num_q_heads, step.head_dim), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    run_eager, _ = _step_fn(pool, step, "bf16", ws, outs[0], 1)
    run_graph, _ = _step_fn(pool, step, "bf16", ws, outs[1], 1)
    _replay_check(run_eager, run_graph, outs[0], outs[1])
