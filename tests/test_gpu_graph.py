"""A decode step (slot scatter, then paged decode and its merge) captured in
a HIP graph and replayed: every replay gives the eager call's output bit for
bit, with eager work and synchronisation between replays. The library's
calls enqueue only kernels when the caller brings the workspace (no
allocation, no memset), which is what makes them capturable."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DevBatch, assert_attention_close, bits_of, note, oracle_step
from oracle_pins import small_batch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv,d,q_len", [(32, 8, 128, 1), (8, 8, 64, 1), (16, 4, 128, 3)])
def test_graph_replay_matches_eager(hq, hkv, d, q_len):
    import paged_kv_cache_433_amd as pa
    from paged_kv_cache_433_amd import workloads as W

    lens = [q_len, 17, 100, 513, 1000, 2049, 40]
    if q_len == 1:
        b = small_batch(950 + hq + d, lens, hq, hkv, d, spare=7)
    else:
        nb = int(sum((n + 15) // 16 for n in lens)) + 7
        b = W.make_batch("graph", 950 + hq + d, lens, hq, hkv, d, nb, q_len=q_len)
    db = DevBatch(b)
    S, mb = b.num_seqs, b.block_tables.shape[1]
    if q_len == 1:
        ws_bytes = pa.decode_workspace_bytes(db.k_cache, S, hq, mb)
    else:
        ws_bytes = pa.decode_multi_workspace_bytes(db.k_cache, S, q_len, hq, mb)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=db.k_cache.device)
    out = torch.empty_like(db.q)

    def step():
        db.scatter()
        if q_len == 1:
            pa.decode(db.q, db.k_cache, db.v_cache, db.block_tables, db.context_lens, float(b.scale),
                      out=out, workspace=ws)
        else:
            pa.decode_multi(db.q, db.k_cache, db.v_cache, db.block_tables, db.context_lens, float(b.scale),
                            out=out, workspace=ws)

    note(f"graph eager hq={hq} hkv={hkv} d={d} q_len={q_len}")
    step()
    torch.cuda.synchronize()
    eager = bits_of(out)
    if q_len == 1:
        assert_attention_close(eager, oracle_step(b)[2], "graph eager")
    else:
        hk, hv = b.k_cache.copy(), b.v_cache.copy()
        oracle.reshape_and_cache(hk, hv, b.new_k, b.new_v, b.slot_mapping)
        assert_attention_close(eager, oracle.decode_multi(b.q, hk, hv, b.block_tables, b.context_lens, b.scale),
                               "graph eager multi")

    note(f"graph capture hq={hq} hkv={hkv} d={d} q_len={q_len}")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device=out.device)
    for r in range(3):
        out.zero_()                     # the replay must rewrite every output
        scratch.add_(1.0)               # eager work between replays
        torch.cuda.synchronize()
        note(f"graph replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), eager), f"replay {r} differs from the eager call"


def test_graph_replay_fused_step():
    """pa_decode_step captured with its workspace: every replay rewrites the
    output and the new tokens' slots exactly as the eager call does."""
    import paged_kv_cache_433_amd as pa

    b = small_batch(960, [1, 17, 100, 513, 1000, 2049, 40], 32, 8, 128, spare=7)
    db = DevBatch(b)
    S, hq, mb = b.num_seqs, b.num_q_heads, b.block_tables.shape[1]
    ws = torch.empty(max(pa.decode_workspace_bytes(db.k_cache, S, hq, mb + 1), 16), dtype=torch.uint8,
                     device=db.k_cache.device)
    from paged_kv_cache_433_amd import _lib
    import ctypes
    need = _lib.lib().pa_decode_step_workspace_bytes(ctypes.byref(pa.ops._cache_desc(db.k_cache, db.v_cache)),
                                                     S, hq, mb)
    assert ws.numel() >= need
    out = torch.empty_like(db.q)

    def step():
        pa.decode_step(db.q, db.new_k, db.new_v, db.k_cache, db.v_cache, db.block_tables, db.context_lens,
                       float(b.scale), out=out, workspace=ws)

    note("graph eager fused step")
    step()
    torch.cuda.synchronize()
    eager, k_after = bits_of(out), bits_of(db.k_cache)
    kc, vc, ref, _ = oracle_step(b)
    assert np.array_equal(k_after, kc)
    assert_attention_close(eager, ref, "graph eager fused step")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        db.k_cache.copy_(torch.from_numpy(b.k_cache.view(np.int16)).view(torch.bfloat16).to(out.device))
        torch.cuda.synchronize()
        note(f"graph replay fused step {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), eager), f"replay {r} differs from the eager call"
        assert np.array_equal(bits_of(db.k_cache), k_after), f"replay {r}: k_cache differs"


def test_graph_replay_sharing_aware_layers():
    """A step of a model with two layers on one sharing plan, captured in a
    graph: the plan (pa_share_plan), then a planned decode per layer, plus
    the one-call tree form. Every replay equals the eager calls bit for bit;
    the outputs are cleared (to NaN) between replays, so each replay must
    rewrite them, empty segments included."""
    import paged_kv_cache_433_amd as pa
    from gpu_util import to_dev, to_dev_bf16
    from paged_kv_cache_433_amd import workloads as W

    nb = 3 + 12 * 2 * 5 + 9 + 64
    b = W.make_tree_batch("graph", 970, [64, 130, 20], [5, 6, 3], 2, 40, 32, 8, 128, nb)
    b = W.permuted(b, W.tree_order(b.block_tables, b.context_lens))
    ctx = b.context_lens.copy()
    ctx[3] = 0                                            # an empty sequence: its rows must be rewritten too
    sprev = W.declared_chain(b.block_tables, ctx)
    dev = torch.device("cuda:0")
    tables, lens, sp = to_dev(b.block_tables), to_dev(ctx), to_dev(sprev)
    rng = np.random.default_rng(971)
    layers = [(to_dev_bf16(W.normal_bf16(rng, b.q.shape)), to_dev_bf16(W.normal_bf16(rng, b.k_cache.shape)),
               to_dev_bf16(W.normal_bf16(rng, b.v_cache.shape))) for _ in range(2)]
    S, hq, mb = b.num_seqs, b.num_q_heads, b.max_blocks_per_seq
    kd = layers[0][1]
    plan = torch.empty(pa.ops._lib.lib().pa_share_plan_bytes(ctypes_desc(pa, kd), S, hq, mb), dtype=torch.uint8,
                       device=dev)
    wsp = torch.empty(pa.ops._lib.lib().pa_decode_shared_planned_workspace_bytes(ctypes_desc(pa, kd), S, hq, mb),
                      dtype=torch.uint8, device=dev)
    wst = torch.empty(pa.ops._lib.lib().pa_decode_shared_tree_workspace_bytes(ctypes_desc(pa, kd), S, hq, mb),
                      dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(layers[0][0]) for _ in range(3)]

    def step():
        pa.share_plan(kd, lens, hq, mb, shared_prev=sp, plan=plan)
        for (q, k, v), out in zip(layers, outs):
            pa.decode_shared_planned(q, k, v, tables, plan, float(b.scale), out=out, workspace=wsp)
        q, k, v = layers[1]
        pa.decode_shared_tree(q, k, v, tables, lens, sp, float(b.scale), out=outs[2], workspace=wst)

    note("graph eager sharing-aware layers")
    step()
    torch.cuda.synchronize()
    eager = [bits_of(o) for o in outs]
    assert np.array_equal(eager[1], eager[2])             # planned layer 2 == the one-call form
    assert np.all(eager[0][3] == 0)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        plan.fill_(0)                                    # the replay must rebuild the plan too
        torch.cuda.synchronize()
        note(f"graph replay sharing-aware layers {r}")
        graph.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(bits_of(o), eager[i]), f"replay {r}, output {i} differs from the eager call"


def ctypes_desc(pa, k):
    import ctypes
    return ctypes.byref(pa.ops._cache_desc(k, k))
