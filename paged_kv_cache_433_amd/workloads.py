"""Seeded synthetic decode batches and a small CPU block manager.

This module makes inputs; it holds none of the attention arithmetic. Tests,
``bench.py`` and the smoke check feed the same arrays to the GPU library and
to the float64 oracle.

bfloat16 data is carried as raw 16-bit patterns (``numpy.uint16``).

Block management follows the pages' description:

* "vLLM: Anatomy and Mechanisms of High-Throughput LLM Inference", section
  "Block-Level Management": a request's logical blocks map to physical blocks
  through a block table; a new physical block comes from a free block pool
  when the last logical block is full; the default block holds 16 tokens.
* the same page, section "Memory Sharing via Copy-on-Write (CoW)": beams
  share physical blocks, and only the block where they diverge is copied.
* "vLLM Internals", section "The Block Manager": the worked example of three
  requests with tables [B0,B1,B2], [B3,B4] and [B5..B8].
* "Inside vLLM: Anatomy of a High-Throughput LLM Inference System", section
  "Generate function": a finished request's blocks go back to the free queue.

The page's example says that R1 holds 48 tokens and that it is "at token 47".
This module reads "48 tokens cached" as positions 0..47, which fill three
blocks. So the token at position 48 opens logical block 3. The rule used is:
a token at position ``pos`` needs a fresh block iff ``pos % block_size == 0``.
"""

from __future__ import annotations

import collections
import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_SIZE = 16
BF16_QNAN = np.uint16(0x7FC0)          # poison for slots no table references
TABLE_PAD_OFFSET = 12345               # padded table entries hold num_blocks + this

# ----------------------------------------------------------------------------
# bfloat16 bit helpers (input preparation only)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits.

    Only finite inputs are expected (generated data); NaN maps to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """``N(0, 1)`` float32 draws rounded to bfloat16 bits."""
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def bytes_per_block(block_size: int, num_kv_heads: int, head_size: int, dtype_bytes: int = 2) -> int:
    """Bytes of one physical KV block of one layer, K and V together.

    The figure the page gives for sizing the cache ("Inside vLLM", section
    "LLM Engine constructor"): 2 (key and value) x block_size x num_kv_heads x
    head_size x bytes per element.
    """
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes


def _rng(seed: int, *stream: int) -> np.random.Generator:
    """Independent generator for one named stream of one seed."""
    return np.random.default_rng([seed, *stream])


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# the block manager
# ----------------------------------------------------------------------------


class BlockPool:
    """Free-block pool with reference counts.

    Blocks are handed out in the order of ``order`` (a shuffled pool when the
    caller passes a permutation) and come back to the tail of the queue when
    their count drops to zero.
    """

    def __init__(self, num_blocks: int, order=None):
        self.num_blocks = int(num_blocks)
        order = np.arange(num_blocks) if order is None else np.asarray(order)
        assert sorted(order.tolist()) == list(range(num_blocks))
        self.free = collections.deque(int(b) for b in order)
        self.ref = np.zeros(num_blocks, dtype=np.int64)

    def alloc(self) -> int:
        if not self.free:
            raise MemoryError("block pool exhausted")
        b = self.free.popleft()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def incref(self, b: int) -> None:
        assert self.ref[b] > 0
        self.ref[b] += 1

    def decref(self, b: int) -> None:
        assert self.ref[b] > 0
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(int(b))

    @property
    def num_free(self) -> int:
        return len(self.free)


@dataclasses.dataclass
class SeqBlocks:
    """A sequence's block table and number of cached tokens."""

    table: list
    length: int = 0

    def fork(self, pool: BlockPool) -> "SeqBlocks":
        for b in self.table:
            pool.incref(b)
        return SeqBlocks(list(self.table), self.length)

    def release(self, pool: BlockPool) -> None:
        for b in self.table:
            pool.decref(b)
        self.table = []
        self.length = 0


def append_token(pool: BlockPool, seq: SeqBlocks, block_size: int = BLOCK_SIZE):
    """Give the sequence's next token a slot; return ``(slot, cow_pair)``.

    A token at position ``pos`` opens a new block iff ``pos % block_size == 0``.
    Otherwise it goes into the last block. If that block is shared, it is
    first replaced by a private copy: ``cow_pair = (old, new)``.
    """
    pos = seq.length
    cow = None
    if pos % block_size == 0:
        seq.table.append(pool.alloc())
    else:
        last = seq.table[-1]
        if pool.ref[last] > 1:
            fresh = pool.alloc()
            pool.decref(last)
            seq.table[-1] = fresh
            cow = (last, fresh)
    seq.length += 1
    slot = seq.table[-1] * block_size + pos % block_size
    return slot, cow


def allocate_prefix(pool: BlockPool, n_tokens: int, block_size: int = BLOCK_SIZE) -> SeqBlocks:
    """Blocks for a sequence's first ``n_tokens`` tokens, in one go."""
    seq = SeqBlocks([])
    for _ in range((n_tokens + block_size - 1) // block_size):
        seq.table.append(pool.alloc())
    seq.length = n_tokens
    return seq


# ----------------------------------------------------------------------------
# decode batches
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class DecodeBatch:
    """One decode step's inputs, all as host arrays.

    The caches hold every token before the newest one. The newest token of
    each sequence (position ``context_lens[s] - 1``) is in ``new_k``/``new_v``
    and goes to ``slot_mapping[s]``, so the step is a scatter followed by a
    decode over ``context_lens``. Slots no table references, including the
    newest token's slot before the scatter, hold bfloat16 NaN. Table entries
    past a sequence's last block hold ``num_blocks + 12345``.

    With ``q_len`` > 1 (several new tokens per sequence: speculative-decode
    verification, a prefill chunk) the newest ``q_len`` tokens of every
    sequence are new: ``new_k``/``new_v``/``slot_mapping`` hold them sequence
    by sequence (``T = S * q_len``) and ``q`` is ``[S, q_len, Hq, D]``.
    """

    name: str
    seed: int
    num_blocks: int
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    scale: np.float32
    block_tables: np.ndarray   # int32 [S, MB]
    context_lens: np.ndarray   # int32 [S]
    q: np.ndarray              # uint16 [S, Hq, D]
    k_cache: np.ndarray        # uint16 [NB, bs, Hkv, D]
    v_cache: np.ndarray
    new_k: np.ndarray          # uint16 [T, Hkv, D]
    new_v: np.ndarray
    slot_mapping: np.ndarray   # int64 [T]
    cow_pairs: np.ndarray      # int64 [P, 2]
    q_len: int = 1

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


def _fill_sequence(k_cache, v_cache, table, k_bits, v_bits, block_size):
    """Put per-logical-position data ``[m, Hkv, D]`` into its physical slots."""
    m = k_bits.shape[0]
    for j in range((m + block_size - 1) // block_size):
        lo, hi = j * block_size, min(m, (j + 1) * block_size)
        k_cache[table[j], : hi - lo] = k_bits[lo:hi]
        v_cache[table[j], : hi - lo] = v_bits[lo:hi]


def make_batch(name, seed, lens, num_q_heads, num_kv_heads, head_size, num_blocks,
               max_blocks_per_seq=None, scale=None, block_size=BLOCK_SIZE, q_len=1) -> DecodeBatch:
    """A decode batch with the given context lengths (new tokens included).

    Draw order for ``seed``:
    * stream (seed, 0) shuffles the free pool;
    * stream (seed, 2) draws q (``[S, Hq, D]``, or ``[S, q_len, Hq, D]``);
    * stream (seed, 1, s) draws sequence s's K then V, per logical position.

    Blocks are popped from the shuffled pool in (sequence, logical block)
    order. Data therefore depends only on (seed, s, position), not on where a
    block lands.
    """
    lens = np.asarray(lens, dtype=np.int64)
    assert np.all(lens >= q_len) and q_len >= 1
    S = len(lens)
    nblk = (lens + block_size - 1) // block_size
    MB = int(max_blocks_per_seq or nblk.max())
    assert nblk.max() <= MB
    pool = BlockPool(num_blocks, _rng(seed, 0).permutation(num_blocks))
    seqs = [allocate_prefix(pool, int(n), block_size) for n in lens]
    tables = np.full((S, MB), num_blocks + TABLE_PAD_OFFSET, dtype=np.int32)
    for s, sq in enumerate(seqs):
        tables[s, : len(sq.table)] = sq.table
    shape = (num_blocks, block_size, num_kv_heads, head_size)
    k_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
    v_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
    new_k = np.empty((S * q_len, num_kv_heads, head_size), dtype=np.uint16)
    new_v = np.empty_like(new_k)
    slots = np.empty(S * q_len, dtype=np.int64)

    def one(s):
        n = int(lens[s])
        r = _rng(seed, 1, s)
        kb = normal_bf16(r, (n, num_kv_heads, head_size))
        vb = normal_bf16(r, (n, num_kv_heads, head_size))
        old = n - q_len
        _fill_sequence(k_cache, v_cache, seqs[s].table, kb[:old], vb[:old], block_size)
        for j in range(q_len):
            pos = old + j
            new_k[s * q_len + j], new_v[s * q_len + j] = kb[pos], vb[pos]
            slots[s * q_len + j] = seqs[s].table[pos // block_size] * block_size + pos % block_size

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(S)))
    q_shape = (S, num_q_heads, head_size) if q_len == 1 else (S, q_len, num_q_heads, head_size)
    q = normal_bf16(_rng(seed, 2), q_shape)
    if scale is None:
        scale = 1.0 / math.sqrt(head_size)
    return DecodeBatch(name, seed, num_blocks, block_size, num_q_heads, num_kv_heads,
                       head_size, np.float32(scale), tables, lens.astype(np.int32), q,
                       k_cache, v_cache, new_k, new_v, slots,
                       np.zeros((0, 2), dtype=np.int64), q_len)


def sequence_kv(batch: DecodeBatch, s: int):
    """Regenerate sequence ``s``'s logical K/V bits ``[n, Hkv, D]``.

    The draws are the same ones ``make_batch`` made. Tests use this to build
    the dense, contiguous K/V without reading the paged cache.
    """
    n = int(batch.context_lens[s])
    r = _rng(batch.seed, 1, s)
    kb = normal_bf16(r, (n, batch.num_kv_heads, batch.head_size))
    vb = normal_bf16(r, (n, batch.num_kv_heads, batch.head_size))
    return kb, vb


# ----------------------------------------------------------------------------
# groups of sequences that share leading blocks
# ----------------------------------------------------------------------------


def consecutive_groups(num_seqs: int, group_size: int) -> np.ndarray:
    """``group_starts`` for groups of ``group_size`` consecutive sequences (the
    last one may be shorter): int32 ``[ceil(num_seqs / group_size) + 1]``."""
    return np.array(list(range(0, num_seqs, group_size)) + [num_seqs], dtype=np.int32)


def declared_sharing(block_tables, context_lens, group_starts, block_size=BLOCK_SIZE) -> np.ndarray:
    """Leading blocks each group's members hold in common: int32 ``[G]``.

    A block manager knows this from its reference counts; here it is read
    back from the tables: the run of equal leading entries, counting only
    blocks every member of the group fills.
    """
    out = []
    for lo, hi in zip(group_starts[:-1], group_starts[1:]):
        lo, hi = int(lo), int(hi)
        if hi <= lo:
            out.append(0)
            continue
        full = min(int(context_lens[j]) // block_size for j in range(lo, hi))
        rows = np.asarray(block_tables)[lo:hi, :full]
        same = np.all(rows == rows[0], axis=0)
        out.append(full if same.all() else int(np.argmin(same)))
    return np.array(out, dtype=np.int32)


def make_shared_batch(name, seed, group_sizes, prefix_lens, private_lens, num_q_heads, num_kv_heads,
                      head_size, num_blocks, block_size=BLOCK_SIZE):
    """A decode batch whose sequences come in groups that share a prompt.

    Group g's ``group_sizes[g]`` members fork one prompt of ``prefix_lens[g]``
    tokens; then member i (counted over the whole batch) appends its own
    ``private_lens[i]`` tokens, and a shared partial last block is copied
    before the first append into it (copy-on-write). Every token is cached
    already: ``new_k``/``new_v``/``slot_mapping`` are empty.

    Draw order for ``seed``: stream (seed, 0) shuffles the pool, (seed, 1, g)
    draws group g's prompt K then V, (seed, 4, i) member i's private K then
    V, (seed, 2) q. Returns ``(batch, group_starts, shared_blocks)``, the
    sharing read back from the tables by ``declared_sharing``.
    """
    S = int(sum(group_sizes))
    assert len(prefix_lens) == len(group_sizes) and len(private_lens) == S
    pool = BlockPool(num_blocks, _rng(seed, 0).permutation(num_blocks))
    shape = (num_blocks, block_size, num_kv_heads, head_size)
    k_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
    v_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
    seqs = []
    for g, (m, plen) in enumerate(zip(group_sizes, prefix_lens)):
        prompt = allocate_prefix(pool, int(plen), block_size)
        r = _rng(seed, 1, g)
        kb = normal_bf16(r, (int(plen), num_kv_heads, head_size))
        vb = normal_bf16(r, (int(plen), num_kv_heads, head_size))
        _fill_sequence(k_cache, v_cache, prompt.table, kb, vb, block_size)
        for b in range(int(m)):
            seqs.append(prompt.fork(pool) if b < m - 1 else prompt)
        if m == 0:
            prompt.release(pool)
    for i, sq in enumerate(seqs):
        m = int(private_lens[i])
        r = _rng(seed, 4, i)
        kb = normal_bf16(r, (m, num_kv_heads, head_size))
        vb = normal_bf16(r, (m, num_kv_heads, head_size))
        for t in range(m):
            slot, cow = append_token(pool, sq, block_size)
            if cow is not None:
                k_cache[cow[1]] = k_cache[cow[0]]
                v_cache[cow[1]] = v_cache[cow[0]]
            blk, off = divmod(slot, block_size)
            k_cache[blk, off] = kb[t]
            v_cache[blk, off] = vb[t]
    lens = np.array([sq.length for sq in seqs], dtype=np.int32)
    MB = max(1, max(len(sq.table) for sq in seqs))
    tables = np.full((S, MB), num_blocks + TABLE_PAD_OFFSET, dtype=np.int32)
    for s, sq in enumerate(seqs):
        tables[s, : len(sq.table)] = sq.table
    q = normal_bf16(_rng(seed, 2), (S, num_q_heads, head_size))
    empty = np.zeros((0, num_kv_heads, head_size), dtype=np.uint16)
    batch = DecodeBatch(name, seed, num_blocks, block_size, num_q_heads, num_kv_heads, head_size,
                        np.float32(1.0 / math.sqrt(head_size)), tables, lens, q, k_cache, v_cache,
                        empty, empty.copy(), np.zeros(0, dtype=np.int64), np.zeros((0, 2), dtype=np.int64))
    starts = np.cumsum([0] + list(group_sizes)).astype(np.int32)
    return batch, starts, declared_sharing(tables, lens, starts, block_size)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

CONFIG_NAMES = ("tiny_mha", "llama2_7b", "llama3_8b_gqa", "long_splitk", "beam_cow")


# ----------------------------------------------------------------------------
# sequences that form trees of shared prefixes
# ----------------------------------------------------------------------------


def _used_rows(block_tables, context_lens, block_size):
    t = np.asarray(block_tables)
    return [tuple(int(x) for x in t[s, :(int(n) + block_size - 1) // block_size])
            for s, n in enumerate(np.asarray(context_lens))]


def tree_order(block_tables, context_lens, block_size=BLOCK_SIZE) -> np.ndarray:
    """A depth-first order of the prefix tree the tables form: the sequences
    sorted by their used table entries, compared entry by entry (a row comes
    before its extensions), ties kept in batch order; int64 ``[S]``. In this
    order the sequences below any node of the tree are consecutive."""
    rows = _used_rows(block_tables, context_lens, block_size)
    return np.array(sorted(range(len(rows)), key=lambda s: rows[s]), dtype=np.int64)


def declared_chain(block_tables, context_lens, block_size=BLOCK_SIZE) -> np.ndarray:
    """``shared_prev`` of a batch: the leading used table entries each
    sequence has in common with the one before it (0 for the first); int32
    ``[S]``. A block manager knows this from its tree; here it is read back
    from the tables."""
    rows = _used_rows(block_tables, context_lens, block_size)
    out = np.zeros(len(rows), dtype=np.int32)
    for i in range(1, len(rows)):
        a, b = rows[i - 1], rows[i]
        k = 0
        while k < min(len(a), len(b)) and a[k] == b[k]:
            k += 1
        out[i] = k
    return out


def chain_sharing(context_lens, shared_prev, max_blocks_per_seq, block_size=BLOCK_SIZE) -> np.ndarray:
    """Blocks each sequence really shares with the one before it: the
    declaration clamped to ``0..max_blocks_per_seq`` and to the whole blocks
    both fill (int64 ``[S]``; 0 for the first)."""
    n = np.asarray(context_lens, dtype=np.int64)
    d = np.asarray(shared_prev, dtype=np.int64)
    out = np.zeros(len(n), dtype=np.int64)
    for i in range(1, len(n)):
        out[i] = max(0, min(int(d[i]), max_blocks_per_seq, int(n[i]) // block_size, int(n[i - 1]) // block_size))
    return out


def tree_algorithmic_bytes(context_lens, shared_prev, max_blocks_per_seq, num_q_heads, num_kv_heads, head_size,
                           block_size=BLOCK_SIZE, dtype_bytes=2) -> int:
    """Bytes a decode over trees of shared prefixes must move: K and V of
    each sequence's tokens past the blocks it shares with the one before it
    (so of every distinct block once, in a depth-first order), q in and out
    back, the table entries read, the context lengths and the
    declarations."""
    n = np.asarray(context_lens, dtype=np.int64)
    e = chain_sharing(n, shared_prev, max_blocks_per_seq, block_size)
    tokens = int(n.sum()) - int(e.sum()) * block_size
    row = 2 * num_kv_heads * head_size * dtype_bytes
    entries = int(((n + block_size - 1) // block_size).sum()) - int(e.sum())
    qo = len(n) * 2 * num_q_heads * head_size * dtype_bytes
    return tokens * row + qo + entries * 4 + 4 * len(n) + 4 * len(n)


def permuted(batch: DecodeBatch, order) -> DecodeBatch:
    """The batch with its sequences taken in ``order`` (same caches; new
    tokens, slots and queries follow their sequences)."""
    order = np.asarray(order, dtype=np.int64)
    assert batch.q_len == 1 and sorted(order.tolist()) == list(range(batch.num_seqs))
    live = len(batch.slot_mapping) == batch.num_seqs
    return dataclasses.replace(
        batch, block_tables=np.ascontiguousarray(batch.block_tables[order]),
        context_lens=np.ascontiguousarray(batch.context_lens[order]), q=np.ascontiguousarray(batch.q[order]),
        new_k=np.ascontiguousarray(batch.new_k[order]) if live else batch.new_k,
        new_v=np.ascontiguousarray(batch.new_v[order]) if live else batch.new_v,
        slot_mapping=np.ascontiguousarray(batch.slot_mapping[order]) if live else batch.slot_mapping)


def make_tree_batch(name, seed, root_lens, beams, rounds, max_append, num_q_heads, num_kv_heads, head_size,
                    num_blocks, block_size=BLOCK_SIZE):
    """A decode batch whose sequences form trees of shared prefixes, the way
    beam search leaves them.

    Root r is a prompt of ``root_lens[r]`` tokens held by ``beams[r]``
    sequences. Then, ``rounds`` times: every sequence appends
    ``U{0..max_append}`` tokens of its own (a shared partial last block is
    copied before the first append into it), and each root's sequences are
    replaced by forks of parents drawn uniformly among them. The batch lists
    the sequences root by root in the order of the last draw (not depth
    first). Every token is cached: ``new_k``/``new_v``/``slot_mapping`` are
    empty.

    Draw order for ``seed``: stream (seed, 0) shuffles the pool, (seed, 1, r)
    draws root r's K then V, (seed, 3, k) round k's append counts then
    parents, (seed, 4, k, i) K then V of sequence i's appends in round k,
    (seed, 2) q.
    """
    assert len(root_lens) == len(beams)
    pool = BlockPool(num_blocks, _rng(seed, 0).permutation(num_blocks))
    shape = (num_blocks, block_size, num_kv_heads, head_size)
    k_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
    v_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
    seqs, root_of = [], []
    for r, (plen, m) in enumerate(zip(root_lens, beams)):
        prompt = allocate_prefix(pool, int(plen), block_size)
        g = _rng(seed, 1, r)
        kb = normal_bf16(g, (int(plen), num_kv_heads, head_size))
        vb = normal_bf16(g, (int(plen), num_kv_heads, head_size))
        _fill_sequence(k_cache, v_cache, prompt.table, kb, vb, block_size)
        for b in range(int(m)):
            seqs.append(prompt.fork(pool) if b < m - 1 else prompt)
            root_of.append(r)
        if m == 0:
            prompt.release(pool)
    S = len(seqs)
    for k in range(rounds):
        g = _rng(seed, 3, k)
        counts = g.integers(0, max_append, size=S, endpoint=True)
        for i, sq in enumerate(seqs):
            c = int(counts[i])
            if c == 0:
                continue
            h = _rng(seed, 4, k, i)
            kb = normal_bf16(h, (c, num_kv_heads, head_size))
            vb = normal_bf16(h, (c, num_kv_heads, head_size))
            for t in range(c):
                slot, cow = append_token(pool, sq, block_size)
                if cow is not None:
                    k_cache[cow[1]] = k_cache[cow[0]]
                    v_cache[cow[1]] = v_cache[cow[0]]
                blk, off = divmod(slot, block_size)
                k_cache[blk, off] = kb[t]
                v_cache[blk, off] = vb[t]
        new, lo = [], 0
        for m in beams:
            parents = g.integers(0, max(int(m), 1), size=int(m))
            new.extend(seqs[lo + int(p)].fork(pool) for p in parents)
            lo += int(m)
        for sq in seqs:
            sq.release(pool)
        seqs = new
    lens = np.array([sq.length for sq in seqs], dtype=np.int32)
    MB = max(1, max((len(sq.table) for sq in seqs), default=1))
    tables = np.full((S, MB), num_blocks + TABLE_PAD_OFFSET, dtype=np.int32)
    for s, sq in enumerate(seqs):
        tables[s, : len(sq.table)] = sq.table
    q = normal_bf16(_rng(seed, 2), (S, num_q_heads, head_size))
    empty = np.zeros((0, num_kv_heads, head_size), dtype=np.uint16)
    return DecodeBatch(name, seed, num_blocks, block_size, num_q_heads, num_kv_heads, head_size,
                       np.float32(1.0 / math.sqrt(head_size)), tables, lens, q, k_cache, v_cache,
                       empty, empty.copy(), np.zeros(0, dtype=np.int64), np.zeros((0, 2), dtype=np.int64))


def lognormal_lens(rng, count, median, sigma, lo, hi):
    """``clip(round(exp(N(ln median, sigma))), lo, hi)``."""
    x = np.exp(rng.normal(math.log(median), sigma, size=count))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def config_lens(name: str, seed: int):
    """Context lengths of a named config (stream (seed, 3))."""
    r = _rng(seed, 3)
    if name == "tiny_mha":
        return np.array([1, 17, 33, 100])
    if name == "llama2_7b":
        return r.integers(128, 2048, size=64, endpoint=True)
    if name in ("llama3_8b_gqa", "llama3_8b_gqa_tp8"):
        return lognormal_lens(r, 256, 1024, 0.5, 16, 4096)
    if name == "long_splitk":
        return np.tile(np.array([32768, 65536, 98304, 131072]), 2)
    if name == "long_splitk_max":
        return np.full(8, 131072)
    if name in ("many_short", "many_short_tp8"):
        return lognormal_lens(r, 4096, 64, 0.5, 16, 256)
    raise KeyError(name)


CONFIG_SHAPES = {
    # name: (num_q_heads, num_kv_heads, head_size, num_blocks, max_blocks_per_seq, seed)
    "tiny_mha": (8, 8, 64, 64, 8, 1),
    "llama2_7b": (32, 32, 128, 16384, 128, 2),
    "llama3_8b_gqa": (32, 8, 128, 65536, 256, 3),
    "long_splitk": (64, 8, 128, 65536, 8192, 4),
    "long_splitk_max": (64, 8, 128, 65536, 8192, 4),
    # One GPU's share of the GQA layer under 8-way tensor parallelism: the
    # same sequences and lengths, 32/8 query heads on 8/8 KV heads.
    "llama3_8b_gqa_tp8": (4, 1, 128, 65536, 256, 3),
    # Many short requests in one batch (serving early in their decode):
    # 4096 sequences, lognormal lengths with median 64, the GQA layer's heads
    # and one GPU's share of them at 8-way tensor parallelism.
    "many_short": (32, 8, 128, 65536, 16, 6),
    "many_short_tp8": (4, 1, 128, 65536, 16, 6),
}


def make_config(name: str, seed: int | None = None, q_len: int = 1, block_size: int = BLOCK_SIZE) -> DecodeBatch:
    """Build one of the named decode configs (the CoW config has its own
    class); ``q_len`` > 1 makes the newest q_len tokens of each sequence new.
    Another ``block_size`` keeps the pool's token capacity and the tables'
    token reach (blocks and table width scaled by 16 / block_size)."""
    hq, hkv, d, nb, mb, default_seed = CONFIG_SHAPES[name]
    seed = default_seed if seed is None else seed
    nb = nb * BLOCK_SIZE // block_size
    mb = (mb * BLOCK_SIZE + block_size - 1) // block_size
    return make_batch(name, seed, config_lens(name, seed), hq, hkv, d, nb, mb, q_len=q_len, block_size=block_size)


def memory_utilization(context_lens, block_size=BLOCK_SIZE) -> float:
    """Share of the allocated slots that hold a token: each sequence owns
    ceil(n / block_size) whole blocks, so its last block is partly empty
    (internal fragmentation)."""
    n = np.asarray(context_lens, dtype=np.int64)
    slots = int(((n + block_size - 1) // block_size).sum()) * block_size
    return float(n.sum()) / slots if slots else 1.0


def algorithmic_bytes(context_lens, num_q_heads, num_kv_heads, head_size,
                      block_size=BLOCK_SIZE, dtype_bytes=2, q_len=1) -> int:
    """Bytes a decode step must move: K and V of every cached token, q in,
    out back (q_len rows of each per sequence), the used block-table entries
    and the context lengths."""
    n = np.asarray(context_lens, dtype=np.int64)
    kv = int(n.sum()) * 2 * num_kv_heads * head_size * dtype_bytes
    qo = len(n) * q_len * 2 * num_q_heads * head_size * dtype_bytes
    tables = int(((n + block_size - 1) // block_size).sum()) * 4
    return kv + qo + tables + 4 * len(n)


def algorithmic_flops(context_lens, num_q_heads, head_size, q_len=1) -> int:
    """Floating-point operations a step's attention must do: for every new
    token j of a sequence of n cached tokens, every query head, and every
    position it sees (n - q_len + j + 1 of them), a dot product with the key
    and a scaled add of the value, 2 * head_size flops each."""
    n = np.asarray(context_lens, dtype=np.int64)
    live = n > 0
    seen = q_len * n[live] - q_len * (q_len - 1) // 2  # sum over j of n - q_len + j + 1
    return int(seen.sum()) * num_q_heads * 4 * head_size


def effective_sharing(context_lens, group_starts, shared_blocks, max_blocks_per_seq,
                      block_size=BLOCK_SIZE) -> np.ndarray:
    """Shared blocks each group really gets: the declaration clamped to
    ``0..max_blocks_per_seq`` and to the whole blocks every member fills
    (int64 ``[G]``; nondecreasing ``group_starts`` within ``0..S`` assumed)."""
    out = []
    for g in range(len(shared_blocks)):
        lo, hi = int(group_starts[g]), int(group_starts[g + 1])
        if hi <= lo:
            out.append(0)
            continue
        full = min(int(context_lens[j]) // block_size for j in range(lo, hi))
        out.append(max(0, min(int(shared_blocks[g]), full, max_blocks_per_seq)))
    return np.array(out, dtype=np.int64)


def shared_algorithmic_bytes(context_lens, group_starts, shared_blocks, max_blocks_per_seq, num_q_heads,
                             num_kv_heads, head_size, block_size=BLOCK_SIZE, dtype_bytes=2) -> int:
    """Bytes a sharing-aware decode step must move: K and V of a group's
    shared blocks once and of each member's tokens past them once, q in and
    out back, the block-table entries read (shared ones once), the context
    lengths and the group description."""
    n = np.asarray(context_lens, dtype=np.int64)
    e = effective_sharing(n, group_starts, shared_blocks, max_blocks_per_seq, block_size)
    shared_of = np.zeros(len(n), dtype=np.int64)
    for g in range(len(e)):
        shared_of[int(group_starts[g]):int(group_starts[g + 1])] = e[g]
    tokens = int(e.sum()) * block_size + int((n - shared_of * block_size).sum())
    row = 2 * num_kv_heads * head_size * dtype_bytes
    entries = int(e.sum()) + int(((n + block_size - 1) // block_size - shared_of).sum())
    qo = len(n) * 2 * num_q_heads * head_size * dtype_bytes
    return tokens * row + qo + entries * 4 + 4 * len(n) + 4 * (2 * len(e) + 1)


def step_write_bytes(context_lens, num_kv_heads, head_size, dtype_bytes=2) -> int:
    """Bytes the fused step writes besides its output: the new K and V row of
    every sequence with a non-empty context (read as part of its context)."""
    live = int(np.count_nonzero(np.asarray(context_lens) > 0))
    return live * 2 * num_kv_heads * head_size * dtype_bytes


def scatter_bytes(num_tokens, num_kv_heads, head_size, dtype_bytes=2) -> int:
    """Bytes of the slot scatter: read new K/V, write them, read the slots."""
    return num_tokens * (2 * num_kv_heads * head_size * dtype_bytes * 2 + 8)


def copy_bytes(num_pairs, block_size, num_kv_heads, head_size, dtype_bytes=2) -> int:
    """Bytes of the copy-on-write: read and write K and V of every pair."""
    return num_pairs * (bytes_per_block(block_size, num_kv_heads, head_size, dtype_bytes) * 2 + 16)


# ----------------------------------------------------------------------------
# beam search with copy-on-write
# ----------------------------------------------------------------------------


class BeamSearchWorkload:
    """Prompts shared by beams, then fork / copy-on-write / append steps.

    ``num_prompts`` prompts of ``prompt_len`` tokens each, each shared by
    ``beams`` beams (refcount = beams), plus ``U{0..max_private}`` private
    tokens per beam. A step does the following:

    1. every new beam picks a parent uniformly among its prompt's beams and
       inherits its table (refcounts go up), then the old beams let go of
       theirs;
    2. beams append one token each, in ascending index. A partial last block
       that is still shared is copied first (copy-on-write), so the
       highest-index sharer keeps the original;
    3. the batch is the pairs to copy, the new tokens' slots and K/V, and the
       tables and lengths to decode over.

    ``k_cache``/``v_cache`` hold the state before the first step. Callers
    apply each step's copy and scatter themselves (GPU library or oracle).
    """

    def __init__(self, seed=5, num_prompts=64, beams=4, prompt_len=1024, max_private=200,
                 num_q_heads=32, num_kv_heads=8, head_size=128, num_blocks=16384,
                 block_size=BLOCK_SIZE):
        self.seed, self.beams, self.bs = seed, beams, block_size
        self.num_q_heads, self.num_kv_heads, self.head_size = num_q_heads, num_kv_heads, head_size
        self.num_blocks = num_blocks
        self.scale = np.float32(1.0 / math.sqrt(head_size))
        self.num_seqs = num_prompts * beams
        self.pool = BlockPool(num_blocks, _rng(seed, 0).permutation(num_blocks))
        shape = (num_blocks, block_size, num_kv_heads, head_size)
        self.k_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
        self.v_cache = np.full(shape, BF16_QNAN, dtype=np.uint16)
        priv = _rng(seed, 3).integers(0, max_private, size=self.num_seqs, endpoint=True)
        self.seqs = []
        for p in range(num_prompts):
            prompt = allocate_prefix(self.pool, prompt_len, block_size)
            r = _rng(seed, 1, p)
            kb = normal_bf16(r, (prompt_len, num_kv_heads, head_size))
            vb = normal_bf16(r, (prompt_len, num_kv_heads, head_size))
            _fill_sequence(self.k_cache, self.v_cache, prompt.table, kb, vb, block_size)
            for b in range(beams):
                sq = prompt.fork(self.pool) if b < beams - 1 else prompt
                self.seqs.append(sq)
        for i, sq in enumerate(self.seqs):
            m = int(priv[i])
            if m == 0:
                continue
            r = _rng(seed, 4, i)
            kb = normal_bf16(r, (m, num_kv_heads, head_size))
            vb = normal_bf16(r, (m, num_kv_heads, head_size))
            for t in range(m):
                slot, cow = append_token(self.pool, sq, block_size)
                if cow is not None:
                    src, dst = cow
                    self.k_cache[dst] = self.k_cache[src]
                    self.v_cache[dst] = self.v_cache[src]
                blk, off = divmod(slot, block_size)
                self.k_cache[blk, off] = kb[t]
                self.v_cache[blk, off] = vb[t]
        self.q_rng = _rng(seed, 2)
        self.step_index = 0

    def step(self) -> DecodeBatch:
        i = self.step_index
        self.step_index += 1
        r = _rng(self.seed, 5, i)
        parents = r.integers(0, self.beams, size=self.num_seqs)
        new = []
        for s in range(self.num_seqs):
            base = (s // self.beams) * self.beams
            new.append(self.seqs[base + int(parents[s])].fork(self.pool))
        for sq in self.seqs:
            sq.release(self.pool)
        self.seqs = new
        slots = np.empty(self.num_seqs, dtype=np.int64)
        pairs = []
        for s, sq in enumerate(self.seqs):
            slot, cow = append_token(self.pool, sq, self.bs)
            slots[s] = slot
            if cow is not None:
                pairs.append(cow)
        lens = np.array([sq.length for sq in self.seqs], dtype=np.int32)
        MB = max(len(sq.table) for sq in self.seqs)
        tables = np.full((self.num_seqs, MB), self.num_blocks + TABLE_PAD_OFFSET, dtype=np.int32)
        for s, sq in enumerate(self.seqs):
            tables[s, : len(sq.table)] = sq.table
        kv_shape = (self.num_seqs, self.num_kv_heads, self.head_size)
        new_k = normal_bf16(r, kv_shape)
        new_v = normal_bf16(r, kv_shape)
        q = normal_bf16(self.q_rng, (self.num_seqs, self.num_q_heads, self.head_size))
        return DecodeBatch("beam_cow", self.seed, self.num_blocks, self.bs, self.num_q_heads,
                           self.num_kv_heads, self.head_size, self.scale, tables, lens, q,
                           self.k_cache, self.v_cache, new_k, new_v, slots,
                           np.array(pairs, dtype=np.int64).reshape(-1, 2))

    def unique_blocks(self) -> int:
        return int(np.count_nonzero(self.pool.ref))
