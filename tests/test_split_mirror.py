"""The decode launches' bookkeeping, checked on the CPU through a model of
the kernels' integer logic (tests/split_mirror.py): for the GPU tests'
shapes and work splits, the full-size workloads, and seeded random cases,
every workgroup writes its merge record, every index the merge kernel
dereferences is in range and names a record of the same segment written by
the same call, and every output row is written exactly once."""

import numpy as np
import pytest

import split_mirror as M
from paged_kv_cache_433_amd import workloads as W

EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 100, 511, 512, 513, 1000, 1024, 1031]
SPLITS = [None, 1, 2, 3, 5, 7, 37, 64, 2000, 5000]


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 2), (32, 8), (16, 1), (12, 4), (7, 7), (40, 8), (96, 12),
                                    (64, 32)])
def test_edge_lengths(hq, hkv):
    mb = max((n + 15) // 16 for n in EDGE_LENS)
    for wgs in SPLITS:
        M.check_plain(EDGE_LENS, hq, hkv, mb, override=wgs)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_block_sizes(bs):
    mb = max((n + bs - 1) // bs for n in EDGE_LENS)
    for wgs in SPLITS:
        M.check_plain(EDGE_LENS, 32, 8, mb, block_size=bs, override=wgs)


def test_many_sequences_with_empty_ones():
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 90, size=700)
    lens[[0, 1, 2, 64, 65, 300, 511, 512, 513, 697, 698, 699]] = 0
    for hkv in (1, 8):
        for wgs in (None, 1, 37, 2000):
            M.check_plain(lens, 4 * hkv, hkv, 6, override=wgs)


def test_all_empty_and_lengths_past_the_table():
    for wgs in (None, 1, 3):
        M.check_plain([0, 0, 0], 8, 8, 4, override=wgs)
        # lengths past what a table row addresses are clamped to it
        M.check_plain([10_000, -5, 64, 65], 8, 2, 4, override=wgs)


@pytest.mark.parametrize("name", ["llama2_7b", "llama3_8b_gqa", "long_splitk", "long_splitk_max",
                                  "llama3_8b_gqa_tp8", "tiny_mha", "many_short", "many_short_tp8"])
def test_full_size_workloads(name):
    hq, hkv, _, _, mb, seed = W.CONFIG_SHAPES[name]
    lens = np.asarray(W.config_lens(name, seed))
    sp = M.check_plain(lens, hq, hkv, mb)
    assert sp.E == sp.W


@pytest.mark.parametrize("q_len,hq,hkv", [(4, 32, 8), (9, 32, 8), (64, 32, 8), (8, 64, 8), (100, 2, 1),
                                          (20, 12, 4)])
def test_multi_token_splits(q_len, hq, hkv):
    lens = [max(n, q_len) for n in EDGE_LENS]
    mb = max((n + 15) // 16 for n in lens)
    for wgs in SPLITS:
        M.check_plain(lens, hq, hkv, mb, override=wgs, q_len=q_len)
    hq_, hkv_, _, _, mb, seed = W.CONFIG_SHAPES["llama3_8b_gqa"]
    M.check_plain(np.maximum(W.config_lens("llama3_8b_gqa", seed), q_len), hq_, hkv_, mb, q_len=q_len)


def test_fused_step_splits():
    """pa_decode_step: every sequence has one more chunk (its newest
    position), so segments and cuts move."""
    for hq, hkv in [(8, 8), (32, 8), (16, 1), (96, 12)]:
        mb = max((n + 15) // 16 for n in EDGE_LENS)
        for wgs in SPLITS:
            M.check_plain(EDGE_LENS, hq, hkv, mb, override=wgs, step=True)
    for name in ("llama3_8b_gqa", "llama2_7b", "long_splitk", "llama3_8b_gqa_tp8", "many_short", "many_short_tp8"):
        hq, hkv, _, _, mb, seed = W.CONFIG_SHAPES[name]
        M.check_plain(np.asarray(W.config_lens(name, seed)), hq, hkv, mb, step=True)
    rng = np.random.default_rng(99)
    for case in range(100):
        lens = rng.integers(0, 300, size=int(rng.integers(1, 40)))
        M.check_plain(lens, 8, 2, 20, block_size=int(rng.choice([8, 16, 32])),
                      override=None if case % 2 else int(rng.integers(1, 200)), step=True)


def test_seeded_random_plain_cases():
    rng = np.random.default_rng(2024)
    for case in range(300):
        S = int(rng.integers(1, 60))
        hkv = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 32]))
        hq = hkv * int(rng.choice([1, 2, 4, 8, 16]))
        bs = int(rng.choice([8, 16, 32]))
        mb = int(rng.integers(1, 40))
        lens = rng.integers(-2, mb * bs + 3, size=S)
        lens[rng.random(S) < 0.2] = 0
        wgs = None if case % 3 == 0 else int(rng.integers(1, 400))
        M.check_plain(lens, hq, hkv, mb, block_size=bs, override=wgs)


def shared_case(seed, sizes, plens, hq, hkv, max_private=70, bs=16):
    """Lengths and declarations of the GPU tests' shared batches: members
    fork a prompt and append private tokens; the declaration is every whole
    block of the prompt plus any private blocks the members still share."""
    rng = np.random.default_rng(seed)
    privs = rng.integers(0, max_private, size=int(sum(sizes)), endpoint=True)
    privs[::5] = 0
    lens, i = [], 0
    for m, p in zip(sizes, plens):
        for _ in range(m):
            lens.append(p + int(privs[i]))
            i += 1
    starts = np.cumsum([0] + list(sizes))
    shared = np.array([p // bs for p in plens])
    return np.array(lens), starts, shared


SHARED_SHAPES = [(32, 8), (8, 8), (16, 4), (4, 1), (48, 4), (16, 1)]


@pytest.mark.parametrize("hq,hkv", SHARED_SHAPES)
def test_shared_shapes_and_splits(hq, hkv):
    lens, starts, shared = shared_case(600 + hq, [4, 9, 1, 3, 40], [100, 512, 16, 37, 64], hq, hkv)
    mb = (int(lens.max()) + 15) // 16
    for wgs in (None, 1, 3, 7, 64, 5000):
        M.check_shared(lens, starts, shared, hq, hkv, mb, override=wgs)
        M.check_shared(lens, starts, shared + 3, hq, hkv, mb, override=wgs)
        M.check_shared(lens, starts, np.array([-1, 2, 100, 0, 1]), hq, hkv, mb, override=wgs)


def test_shared_invalid_lists_empty_members_and_ungrouped_tail():
    lens, starts, shared = shared_case(613, [3, 4, 2], [64, 130, 20], 32, 8)
    mb = (int(lens.max()) + 15) // 16
    for wgs in (None, 1, 3, 7):
        for bad in ([0, 8, 4, 9], [0, 4, 8, 13], [-1, 4, 8, 9]):
            M.check_shared(lens, bad, shared, 32, 8, mb, override=wgs)
        M.check_shared(lens, [0], [], 32, 8, mb, override=wgs)
        l2 = lens.copy()
        l2[4] = 0
        M.check_shared(l2, starts[:-1], shared[:-1], 32, 8, mb, override=wgs)
        M.check_shared(np.zeros(9, dtype=int), starts, shared, 32, 8, mb, override=wgs)


@pytest.mark.parametrize("bs", [8, 32])
def test_shared_block_sizes(bs):
    for hq, hkv in [(32, 8), (8, 8), (16, 1)]:
        lens, starts, shared = shared_case(900 + bs + hq, [4, 9, 1, 3, 5], [24, 100, 8, 40, 64], hq, hkv,
                                           max_private=50, bs=bs)
        mb = (int(lens.max()) + bs - 1) // bs
        for wgs in (None, 1, 3):
            M.check_shared(lens, starts, shared, hq, hkv, mb, block_size=bs, override=wgs)
            M.check_shared(lens, starts, shared + 3, hq, hkv, mb, block_size=bs, override=wgs)


def test_shared_beam_workload_shape():
    """64 prompts x 4 beams, 1024-token prompts, U{0..200} private tokens."""
    rng = np.random.default_rng(5)
    lens = 1024 + rng.integers(0, 201, size=256)
    starts = np.arange(0, 257, 4)
    shared = np.full(64, 64)
    for wgs in (None, 1, 255, 1000):
        M.check_shared(lens, starts, shared, 32, 8, 80, override=wgs)


def test_seeded_random_shared_cases():
    rng = np.random.default_rng(77)
    for case in range(200):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        bs = int(rng.choice([8, 16, 32]))
        G = int(rng.integers(0, 6))
        sizes = rng.integers(1, 12, size=G)
        tail = int(rng.integers(0, 5))
        S = int(sizes.sum()) + tail
        if S == 0:
            continue
        mb = int(rng.integers(1, 30))
        lens = rng.integers(0, mb * bs + 1, size=S)
        starts = np.cumsum([0] + list(sizes))
        shared = rng.integers(-2, mb + 3, size=G)
        wgs = None if case % 3 == 0 else int(rng.integers(1, 300))
        M.check_shared(lens, starts, shared, hkv * g, hkv, mb, block_size=bs, override=wgs)


def test_mirror_catches_a_missing_merge_record():
    """The model fails when a workgroup past the last one with units leaves
    its merge record unwritten (the bookkeeping slip that once let the merge
    read uninitialised workspace): planted here on the CPU, in a copy of the
    split's records."""
    sp = M.check_plain([40, 3], 8, 8, 4, override=20)
    assert sp.E < sp.W
    bad = M.Split(W=sp.W, U=sp.U, E=sp.E, desc=list(sp.desc), records=dict(sp.records))
    bad.desc[-1] = (123456, 999)  # what uninitialised workspace could hold
    with pytest.raises(AssertionError):
        M.merge(bad, M.plain_segments([40, 3], 64), 2, 2)


# ---------------------------------------------------------------------------
# chain form (pa_decode_shared_tree) and the stream each segment walks
# ---------------------------------------------------------------------------

def tree_case(seed, roots, beams, rounds, bs, max_append=40):
    from paged_kv_cache_433_amd import workloads as W
    rng = np.random.default_rng(seed)
    root_lens = [int(x) for x in rng.integers(0, 120, size=roots)]
    nb = sum((p + bs - 1) // bs for p in root_lens) + sum(beams) * rounds * ((max_append + bs - 1) // bs + 2) + 9
    return W.make_tree_batch("tree", seed, root_lens, beams, rounds, max_append, 8, 1, 64, nb, block_size=bs)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (16, 4), (48, 4), (16, 1)])
def test_tree_plans_read_each_members_own_blocks(bs, hq, hkv):
    """Trees of shared prefixes (beam-search histories), in depth-first and
    in batch order, with the declarations read back from the tables: every
    member sees each chunk of its context once, through a table row that
    names its own blocks, and every output row is written once."""
    from paged_kv_cache_433_amd import workloads as W
    for seed, roots, beams, rounds in [(1, 3, [4, 9, 3], 3), (2, 2, [40, 1], 2), (3, 4, [2, 5, 8, 1], 4)]:
        b = tree_case(seed + bs + hq, roots, beams, rounds, bs)
        for order in (np.arange(b.num_seqs), W.tree_order(b.block_tables, b.context_lens, bs)):
            bp = W.permuted(b, order)
            d = W.declared_chain(bp.block_tables, bp.context_lens, bs)
            for wgs in (None, 1, 3, 7):
                M.check_shared(bp.context_lens, [0], [], hq, hkv, bp.max_blocks_per_seq, block_size=bs,
                               override=wgs, shared_prev=d, tables=bp.block_tables)


def test_tree_order_reads_less():
    """Depth-first order never reads more chunks than batch order, and both
    read fewer than no sharing when the tree shares anything."""
    from paged_kv_cache_433_amd import workloads as W
    b = tree_case(11, 4, [4, 4, 4, 4], 4, 16)
    chunks = []
    for order in (np.arange(b.num_seqs), W.tree_order(b.block_tables, b.context_lens)):
        bp = W.permuted(b, order)
        d = W.declared_chain(bp.block_tables, bp.context_lens)
        items, _, _ = M.share_plan(bp.context_lens, [0], [], bp.max_blocks_per_seq, 16, 8, d)
        chunks.append(sum(it["L"] for it in items))
    plain = int(((b.context_lens + 15) // 16).sum())
    assert chunks[1] <= chunks[0] < plain


def test_group_form_reads_each_members_own_blocks():
    """The group form through the same stream model, with tables: true
    declarations, 8-, 16- and 32-token blocks, groups wider than one item."""
    from paged_kv_cache_433_amd import workloads as W
    for bs in (8, 16, 32):
        for hq, hkv in [(32, 8), (16, 1), (8, 8)]:
            rng = np.random.default_rng(40 + bs + hq)
            sizes, plens = [4, 9, 1, 3, 40], [24, 100, 8, 40, 64]
            privs = rng.integers(0, 50, size=int(sum(sizes)), endpoint=True)
            privs[::5] = 0
            nb = sum((p + bs - 1) // bs for p in plens) + int(sum((x + bs) // bs for x in privs)) + 9
            b, starts, shared = W.make_shared_batch("g", 40 + bs, sizes, plens, privs, 8, 1, 64, nb, block_size=bs)
            for wgs in (None, 1, 5):
                M.check_shared(b.context_lens, starts, shared, hq, hkv, b.max_blocks_per_seq, block_size=bs,
                               override=wgs, tables=b.block_tables)


def test_seeded_random_tree_declarations():
    """Random lengths and arbitrary declarations (negative, past the
    contexts, past the table): the plan and the streams stay consistent and
    every output row is written once."""
    rng = np.random.default_rng(78)
    for case in range(200):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        bs = int(rng.choice([8, 16, 32]))
        S = int(rng.integers(1, 60))
        mb = int(rng.integers(1, 30))
        lens = rng.integers(0, mb * bs + 1, size=S)
        if case % 4 == 0:
            lens[rng.integers(0, S)] = 0
        decl = rng.integers(-3, mb + 4, size=S)
        wgs = None if case % 3 == 0 else int(rng.integers(1, 300))
        M.check_shared(lens, [0], [], hkv * g, hkv, mb, block_size=bs, override=wgs, shared_prev=decl)


def test_stream_check_catches_a_wrong_visibility_end(monkeypatch):
    """The stream model fails when a chunk is shown to one member too many
    (planted on the CPU, in the model's seg_at)."""
    from paged_kv_cache_433_amd import workloads as W
    b = tree_case(5, 2, [4, 4], 2, 16)
    bp = W.permuted(b, W.tree_order(b.block_tables, b.context_lens))
    d = W.declared_chain(bp.block_tables, bp.context_lens)
    good = M.seg_at

    def wide(item, lanes, j, b_, nj):
        c = good(item, lanes, j, b_, nj)
        return (c[0], min(c[1] + 1, item["ntok"] - 1), *c[2:])

    monkeypatch.setattr(M, "seg_at", wide)
    with pytest.raises(AssertionError):
        M.check_shared(bp.context_lens, [0], [], 32, 8, bp.max_blocks_per_seq, shared_prev=d,
                       tables=bp.block_tables)


def test_prologue_search_matches_the_definition():
    """The many-sequence prologue (contiguous ranges per thread, a scan over
    threads, one thread walking its range) finds, for every workgroup, the
    sequence whose units hold its first unit, with that sequence's first
    chunk, as the plain definition does; and every workgroup past the units
    is told so."""
    rng = np.random.default_rng(91)
    for case in range(120):
        S = int(rng.integers(2, 700))
        nthr = int(rng.choice([64, 128, 256]))
        if S <= nthr:
            S = nthr + int(rng.integers(1, 300))
        cap = int(rng.choice([64, 512, 4096]))
        lens = rng.integers(0, cap + 40, size=S)
        lens[rng.random(S) < 0.2] = 0
        NG = int(rng.choice([1, 2, 4]))
        step = bool(case % 2)
        n = np.minimum(lens, cap)
        L = np.where(n > 0, (n - 1 + 15) // 16 + 1, 0) if step else (n + 15) // 16
        starts = np.concatenate([[0], np.cumsum(L)])
        U = int(starts[-1]) * NG
        W = int(rng.integers(1, 2 * max(U, 1) + 3))
        for w in sorted(set(int(x) for x in rng.integers(0, W, size=8)) | {0, W - 1}):
            got = M.prologue_search(lens, cap, nthr, NG, W, w, step)
            E = min(U, W)
            if w >= E:
                assert got is None
                continue
            lo = M.range_lo(w, U, E)
            s = int(np.searchsorted(starts * NG, lo, side="right")) - 1
            while L[s] == 0:  # the units of empty sequences are none: the holder is the next non-empty one
                s += 1
            assert got[:3] == (U, lo, M.range_lo(w + 1, U, E))
            assert got[3:] == (s, int(starts[s]), int(n[s])), (case, w, got, s)
