"""float64 / bit-exact reference for paged decode, slot scatter and CoW copy.

TEST INFRASTRUCTURE ONLY (see the package docstring). Arrays of bfloat16
values are carried as their raw 16-bit patterns in ``numpy.uint16`` arrays,
because numpy has no bfloat16 type; widening a pattern to float64 is exact.

Layouts (the same ones the GPU library documents):

* ``k_cache``, ``v_cache``: ``[num_blocks, block_size, num_kv_heads, head_size]``
* ``q``: ``[num_seqs, num_q_heads, head_size]``
* ``block_tables``: int32 ``[num_seqs, max_blocks_per_seq]``
* ``context_lens``: int32 ``[num_seqs]``; it counts every cached token of the
  sequence, the one written in this step included.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64.

    A bfloat16 number is the upper half of an IEEE float32, so shifting the
    pattern into the top 16 bits of a 32-bit word gives the float32 of equal
    value, and float32 widens to float64 without rounding.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_sequence(q_s, k_cache, v_cache, table_s, n, scale) -> np.ndarray:
    """Decode attention of one sequence, every query head, in float64.

    Follows the definition the pages give of a decode step ("Inside vLLM",
    section "Scheduler": one new token attends over all cached K/V vectors)
    with the cache located through the block table ("vLLM: Anatomy and
    Mechanisms", section "Block-Level Management"): logical position ``i``
    lives in physical block ``table_s[i // block_size]`` at offset
    ``i % block_size``.

    Query head ``h`` reads key/value head ``h // (num_q_heads // num_kv_heads)``
    (consecutive query heads share one K/V head). For each head::

        z_i = scale * sum_d q[h, d] * k_i[d]
        p_i = exp(z_i - max_j z_j) / sum_j exp(z_j - max_j z_j)
        out[h, :] = sum_i p_i * v_i[:]

    ``n == 0`` (no cached token) gives a zero output. Returns float64
    ``[num_q_heads, head_size]``.
    """
    q_s = np.asarray(q_s)
    num_q_heads, head_size = q_s.shape
    _, block_size, num_kv_heads, _ = k_cache.shape
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_q_heads, head_size), dtype=np.float64)
    n = int(n)
    if n == 0:
        return out
    positions = np.arange(n)
    physical = np.asarray(table_s)[positions // block_size].astype(np.int64)
    offsets = positions % block_size
    qf = bf16_bits_to_f64(q_s)
    scale64 = np.float64(np.float32(scale))
    for kv_head in range(num_kv_heads):
        keys = bf16_bits_to_f64(k_cache[physical, offsets, kv_head, :])    # [n, D]
        values = bf16_bits_to_f64(v_cache[physical, offsets, kv_head, :])  # [n, D]
        for h in range(kv_head * group, (kv_head + 1) * group):
            z = scale64 * (keys @ qf[h])                                  # [n]
            w = np.exp(z - z.max())
            p = w / w.sum()
            out[h] = p @ values
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale) -> np.ndarray:
    """Decode attention of a batch: ``decode_sequence`` for every sequence.

    Returns float64 ``[num_seqs, num_q_heads, head_size]``. Block-table entries
    past ``ceil(n / block_size)`` are never read, so they may hold anything.
    """
    q = np.asarray(q)
    num_seqs = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(num_seqs):
        out[s] = decode_sequence(q[s], k_cache, v_cache, block_tables[s],
                                 context_lens[s], scale)
    return out


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale) -> np.ndarray:
    """Attention of several new tokens per sequence over the paged cache.

    A step that runs ``q_len`` new tokens of a sequence at once (verifying
    speculative tokens in one forward pass: "vLLM: Anatomy and Mechanisms",
    section "Speculative Decoding"; a chunk of a prefill: section "Chunked
    Prefill") has all of them in the cache already, at positions
    ``n - q_len .. n - 1``. Attention is causal: new token ``j`` attends over
    positions ``0 .. n - q_len + j``, itself included, which is the decode
    step of a context of ``n - q_len + j + 1`` tokens. ``q``:
    ``[num_seqs, q_len, num_q_heads, head_size]`` bfloat16 bits; returns
    float64 of that shape. ``n == 0`` gives zeros; otherwise ``n >= q_len``.
    """
    q = np.asarray(q)
    num_seqs, q_len = q.shape[:2]
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(num_seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        assert n >= q_len, "the new tokens must be in the cache"
        for j in range(q_len):
            out[s, j] = decode_sequence(q[s, j], k_cache, v_cache, block_tables[s], n - q_len + j + 1, scale)
    return out


def decode_shared(q, k_cache, v_cache, block_tables, context_lens, group_starts, shared_blocks,
                  scale) -> np.ndarray:
    """Decode attention of a batch whose sequences share leading blocks.

    Several sequences can hold the same physical blocks at the start of their
    tables: the outputs of parallel sampling share the prompt's blocks, beams
    share their common history ("vLLM: Anatomy and Mechanisms", section
    "Memory Sharing via Copy-on-Write (CoW)"), and prompts with a common
    beginning reuse cached blocks (section "Prefix Caching"). A caller that
    knows this declares it: group ``g`` is the sequences
    ``group_starts[g] <= i < group_starts[g + 1]``, and their tables agree on
    the first ``shared_blocks[g]`` entries. ``group_starts`` has one entry
    more than ``shared_blocks``, never decreases, and stays within
    ``0..num_seqs``; a sequence in no group is on its own.

    Reading (the pages define the sharing, not a call that uses it): the
    declared prefix of group ``g`` counts only whole blocks that every member
    fills, ``e = min(shared_blocks[g], n_j // block_size for each member j)``
    (clamped to ``0..max_blocks_per_seq``), and every member reads those
    ``e`` blocks through the table of the group's first member, the rest
    through its own. When the declaration is true the tables agree there and
    the result is ``decode``'s. Returns float64 ``[num_seqs, num_q_heads,
    head_size]``.
    """
    block_size = k_cache.shape[1]
    starts = np.asarray(group_starts, dtype=np.int64)
    shared = np.asarray(shared_blocks, dtype=np.int64)
    num_seqs = np.asarray(q).shape[0]
    assert starts.ndim == 1 and len(starts) == len(shared) + 1
    assert np.all(np.diff(starts) >= 0) and starts[0] >= 0 and starts[-1] <= num_seqs
    tables = np.array(block_tables, copy=True)
    for g in range(len(shared)):
        lo, hi = int(starts[g]), int(starts[g + 1])
        if hi <= lo:
            continue
        full = min(int(context_lens[j]) // block_size for j in range(lo, hi))
        e = max(0, min(int(shared[g]), full, tables.shape[1]))
        for j in range(lo + 1, hi):
            tables[j, :e] = block_tables[lo, :e]
    return decode(q, k_cache, v_cache, tables, context_lens, scale)


def decode_shared_tree(q, k_cache, v_cache, block_tables, context_lens, shared_prev, scale) -> np.ndarray:
    """Decode attention of a batch whose sequences form trees of shared
    prefixes.

    After a step of beam search the beams that picked the same parent hold
    all of its full blocks, so the beams of a prompt form a tree of shared
    prefixes; cached prompt prefixes form one too ("vLLM: Anatomy and
    Mechanisms", sections "Memory Sharing via Copy-on-Write (CoW)" and
    "Prefix Caching"). A caller declares, for each sequence ``i > 0``, the
    leading table entries it has in common with sequence ``i - 1``
    (``shared_prev[i]``; ``shared_prev[0]`` is ignored).

    Reading (the pages define the sharing, not a call that uses it):
    sequence ``i`` shares ``e_i = min(shared_prev[i], n_i // block_size,
    n_{i-1} // block_size)`` blocks with ``i - 1`` (whole blocks both fill,
    never fewer than none) and reads them as ``i - 1`` reads them: its first
    ``e_i`` table entries are those of ``i - 1`` after ``i - 1``'s own
    substitution, so a chain of declarations resolves to the first sequence
    of the chain. When the declarations are true the tables agree there and
    the result is ``decode``'s. Returns float64 ``[num_seqs, num_q_heads,
    head_size]``.
    """
    block_size = k_cache.shape[1]
    n = [int(x) for x in context_lens]
    declared = np.asarray(shared_prev, dtype=np.int64)
    assert declared.shape == (len(n),)
    tables = np.array(block_tables, copy=True)
    for i in range(1, len(n)):
        e = max(0, min(int(declared[i]), n[i] // block_size, n[i - 1] // block_size))
        tables[i, :e] = tables[i - 1, :e]
    return decode(q, k_cache, v_cache, tables, context_lens, scale)


def reshape_and_cache(k_cache, v_cache, k, v, slot_mapping) -> None:
    """Scatter each new token's K and V into its physical slot, in place.

    A decode step first stores the newest token's K/V in the slot the block
    manager gave it, so that the attention that follows sees every earlier
    token cached ("Inside vLLM", section "Scheduler"; on-demand allocation in
    "vLLM: Anatomy and Mechanisms", section "Block-Level Management"). Slot
    ``s`` is offset ``s % block_size`` of physical block ``s // block_size``.
    A negative slot marks a padding token and is skipped. Slots must be
    distinct and inside the pool; the copy is bit-exact.
    """
    num_blocks, block_size = k_cache.shape[:2]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    assert np.all(live < num_blocks * block_size), "slot outside the block pool"
    assert len(np.unique(live)) == len(live), "two tokens mapped to one slot"
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        k_cache[blk, off] = k[t]
        v_cache[blk, off] = v[t]


def copy_blocks(k_cache, v_cache, src_dst_pairs) -> None:
    """Copy whole physical blocks, K and V, in place (copy-on-write).

    When sequences that share blocks diverge, only the block where they
    diverge is copied ("vLLM: Anatomy and Mechanisms", section "Memory Sharing
    via Copy-on-Write (CoW)"). For every pair ``(src, dst)`` block ``dst``
    becomes a bit copy of block ``src`` as it was before the call.
    Destinations must be distinct and never also a source (a copy-on-write
    destination is a fresh block from the free pool).
    """
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    if len(pairs) == 0:
        return
    src, dst = pairs[:, 0], pairs[:, 1]
    num_blocks = k_cache.shape[0]
    assert np.all((src >= 0) & (src < num_blocks) & (dst >= 0) & (dst < num_blocks))
    assert len(np.unique(dst)) == len(dst), "duplicate copy destination"
    assert not np.intersect1d(src, dst).size, "a destination is also a source"
    k_src = k_cache[src].copy()
    v_src = v_cache[src].copy()
    for i, d in enumerate(dst):
        k_cache[d] = k_src[i]
        v_cache[d] = v_src[i]


def swap_blocks(dev_k, dev_v, host_k, host_v, src_dst_pairs, direction) -> None:
    """Move whole blocks, K and V, between the device cache and a host cache.

    A preempted request's KV blocks are moved to CPU RAM and brought back
    when it is rescheduled ("vLLM: Anatomy and Mechanisms", section
    "Preemption and Recovery"; "vLLM Internals", section "The Block
    Manager"). ``direction`` "out": host block ``dst`` becomes a bit copy of
    device block ``src``; "in": device block ``dst`` becomes a bit copy of
    host block ``src``. The two sides are different arrays, so only the
    destinations must be distinct.
    """
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    if len(pairs) == 0:
        return
    if direction == "out":
        (fk, fv), (tk, tv) = (dev_k, dev_v), (host_k, host_v)
    elif direction == "in":
        (fk, fv), (tk, tv) = (host_k, host_v), (dev_k, dev_v)
    else:
        raise ValueError(direction)
    src, dst = pairs[:, 0], pairs[:, 1]
    assert np.all((src >= 0) & (src < fk.shape[0]) & (dst >= 0) & (dst < tk.shape[0]))
    assert len(np.unique(dst)) == len(dst), "duplicate swap destination"
    for s_, d_ in zip(src, dst):
        tk[d_] = fk[s_]
        tv[d_] = fv[s_]
