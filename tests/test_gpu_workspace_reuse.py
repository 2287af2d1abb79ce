"""GPU: calls that reuse one workspace. A sequence cut between workgroups
leaves partial records and a per-workgroup merge record in the workspace; a
call must neither read what an earlier call left there nor depend on the
workspace's initial contents. Calls whose context lengths (and
so cut points) differ alternate on one workspace that starts as random bytes;
every output equals, bit for bit, the same call's output on a workspace of
its own, and sampled sequences match the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_433_amd as pa
from gpu_util import DEV, DevBatch, assert_attention_close, bits_of, note, oracle_step, to_dev, to_dev_bf16
from paged_kv_cache_433_amd import workloads as W

pytestmark = pytest.mark.gpu


def random_bytes(n, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(0, 256, (max(n, 1),), dtype=torch.uint8, generator=g).to(DEV)


def alternate(calls, nbytes, rounds=3):
    """Runs each call on a random workspace of its own, then all of them in
    turn on one shared random workspace, ``rounds`` times, and checks that
    every shared-workspace output equals the call's own-workspace output."""
    alone = [bits_of(call(random_bytes(nbytes, 100 + i))) for i, call in enumerate(calls)]
    ws = random_bytes(nbytes, 99)
    for r in range(rounds):
        for i, call in enumerate(calls):
            got = bits_of(call(ws))
            assert np.array_equal(got, alone[i]), f"call {i}, round {r}: differs on a reused workspace"
    return alone


def test_decode_alternating_lengths_on_one_workspace():
    rng = np.random.default_rng(41)
    S, mb = 96, 200
    batches = []
    for seed in (0, 1, 2):
        lens = rng.integers(1, mb * 16, size=S, endpoint=True)
        lens[seed::7] = rng.integers(1, 40, size=len(lens[seed::7]))     # short ones move the cuts
        nb = int(sum((n + 15) // 16 for n in lens)) + 5
        batches.append(W.make_batch("reuse", 820 + seed, lens, 32, 8, 128, nb, max_blocks_per_seq=mb))
    devs = []
    for b in batches:
        d = DevBatch(b)
        d.scatter()
        devs.append(d)
    nbytes = pa.decode_workspace_bytes(devs[0].k_cache, S, 32, mb)
    assert nbytes > 0
    note("workspace reuse: decode, three length sets alternating")
    alone = alternate([lambda ws, d=d: d.decode(workspace=ws) for d in devs], nbytes)
    for b, out in zip(batches, alone):
        idx = np.arange(0, S, 11)
        _, _, ref, idx = oracle_step(b, idx)
        assert_attention_close(out[idx], ref, "decode on own workspace")


def test_decode_multi_alternating_lengths_on_one_workspace():
    rng = np.random.default_rng(42)
    S, mb, ql = 40, 64, 3
    devs, batches = [], []
    for seed in (0, 1):
        lens = rng.integers(ql, mb * 16, size=S, endpoint=True)
        nb = int(sum((n + 15) // 16 for n in lens)) + 5
        b = W.make_batch("reuse-multi", 830 + seed, lens, 16, 4, 128, nb, max_blocks_per_seq=mb, q_len=ql)
        d = DevBatch(b)
        d.scatter()
        devs.append(d)
        batches.append(b)
    nbytes = pa.decode_multi_workspace_bytes(devs[0].k_cache, S, ql, 16, mb)
    assert nbytes > 0
    note("workspace reuse: decode_multi q_len 3, two length sets alternating")
    calls = [lambda ws, d=d: pa.decode_multi(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                             float(d.b.scale), workspace=ws) for d in devs]
    alone = alternate(calls, nbytes)
    for b, out in zip(batches, alone):
        kc, vc = b.k_cache.copy(), b.v_cache.copy()
        oracle.reshape_and_cache(kc, vc, b.new_k, b.new_v, b.slot_mapping)
        idx = np.arange(0, S, 7)
        ref = oracle.decode_multi(b.q[idx], kc, vc, b.block_tables[idx], b.context_lens[idx], b.scale)
        assert_attention_close(out[idx], ref, "decode_multi on own workspace")


def test_decode_shared_alternating_groups_on_one_workspace():
    S = 48
    cases = []
    for seed, sizes, plens in ((0, [4, 9, 3, 32], [100, 512, 16, 300]), (1, [16, 2, 30], [64, 900, 37]),
                               (2, [1] * 48, [0] * 48)):
        rng = np.random.default_rng(850 + seed)
        privs = rng.integers(0, 90, size=S, endpoint=True)
        if sum(plens) == 0:
            privs = np.maximum(privs, 1)
        nb = sum((p + 15) // 16 for p in plens) + int(sum((x + 16) // 16 for x in privs)) + S + 9
        b, starts, shared = W.make_shared_batch("reuse-shared", 850 + seed, sizes, plens, privs, 32, 8, 128, nb)
        cases.append((b, starts, shared))
    mb = max(b.block_tables.shape[1] for b, _, _ in cases)
    devs = []
    for b, starts, shared in cases:
        tab = np.full((S, mb), b.num_blocks, dtype=np.int32)
        tab[:, : b.block_tables.shape[1]] = b.block_tables
        b.block_tables = tab
        devs.append((to_dev_bf16(b.q), to_dev_bf16(b.k_cache), to_dev_bf16(b.v_cache), to_dev(tab),
                     to_dev(b.context_lens), to_dev(np.asarray(starts, dtype=np.int32)),
                     to_dev(np.asarray(shared, dtype=np.int32)), float(b.scale)))
    nbytes = max(pa.decode_shared_workspace_bytes(d[1], S, 32, mb, len(c[2])) for d, c in zip(devs, cases))
    note("workspace reuse: decode_shared, three group layouts alternating")
    calls = [lambda ws, d=d: pa.decode_shared(*d[:7], d[7], workspace=ws) for d in devs]
    alone = alternate(calls, nbytes)
    for (b, starts, shared), out in zip(cases, alone):
        ref = oracle.decode_shared(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, starts, shared,
                                   b.scale)
        assert_attention_close(out, ref, "decode_shared on own workspace")
