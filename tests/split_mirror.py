"""CPU model of the decode launches' bookkeeping: the balanced work split,
the walk of each workgroup's range into pieces, the partial and merge
records the decode kernel writes, the sharing-aware plan, and the records
the merge kernel reads back.

It models the HIP kernels' integer logic (csrc/decode.hip: the prologue,
``next_piece``, ``finish_piece``, ``share_plan_kernel``, ``merge_kernel``)
and the host-side sizes (csrc/pa_api.cpp: ``decode_wgs``,
``heads_per_workgroup``), not attention: no arithmetic of the method is
here. The tests use it to show, without a GPU, that every workgroup writes
its merge record, that every record index the merge dereferences is in
range and was written for the same segment by this call, and that every
output row is written exactly once.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CHUNK = 16  # tokens per unit of work (one MFMA tile of rows)


def heads_per_workgroup(num_kv_heads: int) -> int:
    for h in (4, 3, 2):
        if num_kv_heads % h == 0:
            return h
    return 1


def decode_wgs(num_seqs: int, num_head_groups: int, heads_per_wg: int, max_chunks_per_seq: int,
               override: int | None = None, waves_per_cu: int = 4) -> int:
    w = 256 * max(waves_per_cu // heads_per_wg, 1)
    by_work = (num_seqs * num_head_groups * max_chunks_per_seq + 3) // 4
    w = min(w, by_work)
    if override is not None and override > 0:
        w = override
    return max(1, min(w, 1 << 20))


def chunks_per_row(max_blocks_per_seq: int, block_size: int) -> int:
    return (max_blocks_per_seq * block_size + CHUNK - 1) // CHUNK


@dataclass
class Segment:
    """What a segment stands for: kernel-side (item or sequence, head group),
    its unit count and the output rows it covers."""
    key: tuple
    L: int
    rows: tuple  # output row keys the segment produces (one per (q row, KV head))


@dataclass
class Split:
    W: int
    U: int
    E: int
    desc: list = field(default_factory=list)      # per workgroup: (x, y) as the kernel writes it
    records: dict = field(default_factory=dict)   # (w, slot) -> (segment key, offset, count)
    written: dict = field(default_factory=dict)   # output row key -> times written
    pieces: list = field(default_factory=list)    # per workgroup: [(key, off, cnt)]


def range_lo(w: int, U: int, E: int) -> int:
    return w * U // E


def owner_of(u: int, U: int, E: int) -> int:
    return ((u + 1) * E - 1) // U


def walk(segments: list, NG: int, W: int) -> Split:
    """The balanced split and the decode kernel's walk.

    ``segments`` lists (key, L, rows) in kernel order, one entry per
    sequence or item (head groups expand inside, head-group major). Returns
    the records each workgroup writes, as decode_kernel does.
    """
    U = sum(seg.L for seg in segments) * NG
    E = min(W, U)
    sp = Split(W=W, U=U, E=E)
    # unit -> (segment index, head group, offset)
    starts, acc = [], 0
    for seg in segments:
        starts.append(acc)
        acc += seg.L * NG
    for w in range(W):
        sp.pieces.append([])
        if w >= E:
            sp.desc.append((-1, -1))
            continue
        lo, hi = range_lo(w, U, E), range_lo(w + 1, U, E)
        # the segment holding `lo`: the one whose units contain it (empty ones never do)
        si = max(i for i, st in enumerate(starts) if st <= lo and segments[i].L > 0 and lo < st + segments[i].L * NG)
        seg_base = starts[si]
        L = segments[si].L
        hg, off = (lo - seg_base) // L, (lo - seg_base) % L
        u, first, desc = lo, True, (-1, -1)
        while u < hi:
            seg = segments[si]
            cnt = min(seg.L - off, hi - u)
            seg_start = seg_base + hg * seg.L
            key = (seg.key, hg)
            sp.pieces[w].append((key, off, cnt))
            whole = off == 0 and cnt == seg.L
            if whole:
                for r in seg.rows:
                    rk = (r, hg)
                    sp.written[rk] = sp.written.get(rk, 0) + 1
            else:
                slot = 0 if first else 1
                assert (w, slot) not in sp.records, f"workgroup {w} writes slot {slot} twice"
                sp.records[(w, slot)] = (key, off, cnt)
            if first:
                if not whole and off + cnt == seg.L:
                    w0 = owner_of(seg_start, U, E)
                    slot0 = 1 if range_lo(w0, U, E) < seg_start else 0
                    desc = (si * NG + hg, w0 * 2 + slot0)
                first = False
            u += cnt
            off += cnt
            if off == seg.L:
                off = 0
                hg += 1
                if hg == NG and u < hi:
                    hg = 0
                    seg_base += seg.L * NG
                    si += 1
                    while segments[si].L == 0:
                        si += 1
        sp.desc.append(desc)
    return sp


def merge(sp: Split, segments: list, NG: int, S_items: int) -> None:
    """The merge kernel's reads: checks every index before use the way the
    kernel does, and that what it reads is this segment's pieces, in order,
    covering the segment exactly."""
    for w1, (x, y) in enumerate(sp.desc):
        if x < 0:
            continue
        assert 0 <= x < S_items * NG, f"merge record of workgroup {w1}: segment {x} out of range"
        assert 0 <= y and (y >> 1) <= w1, f"merge record of workgroup {w1}: first piece {y} out of range"
        si, hg = divmod(x, NG)
        seg = segments[si]
        key = (seg.key, hg)
        w0 = y >> 1
        got = []
        for w in range(w0, w1 + 1):
            rec = (w0, y & 1) if w == w0 else (w, 0)
            assert rec in sp.records, f"merge of workgroup {w1} reads record {rec}, never written"
            k, off, cnt = sp.records[rec]
            assert k == key, f"merge of workgroup {w1} reads record {rec} of another segment"
            got.append((off, cnt))
        pos = 0
        for off, cnt in got:
            assert off == pos, f"merge of workgroup {w1}: pieces not contiguous"
            pos += cnt
        assert pos == seg.L, f"merge of workgroup {w1}: pieces cover {pos} of {seg.L} units"
        for r in seg.rows:
            rk = (r, hg)
            sp.written[rk] = sp.written.get(rk, 0) + 1


def plain_segments(lens, cap: int, step: bool = False) -> list:
    """Sequences as segments (pa_decode, pa_decode_multi): clamped lengths.
    With `step` (pa_decode_step) the newest position is a chunk of its own."""
    segs = []
    for s, n in enumerate(lens):
        n = min(max(int(n), 0), cap)
        L = ((n - 1 + CHUNK - 1) // CHUNK + 1 if n > 0 else 0) if step else (n + CHUNK - 1) // CHUNK
        segs.append(Segment(key=s, L=L, rows=(s,)))
    return segs


def check_plain(lens, num_q_heads, num_kv_heads, max_blocks_per_seq, block_size=16, override=None,
                q_len=1, step=False) -> Split:
    cols = q_len * (num_q_heads // num_kv_heads)
    if cols > 64:  # a workgroup per KV head, a wavefront per 32 columns, 8 wavefronts per CU
        hg, NG, wpc = (cols + 31) // 32, num_kv_heads, 8
    else:
        hg = heads_per_workgroup(num_kv_heads)
        NG = num_kv_heads // hg
        # one-wavefront workgroups on one tile with few segments: 3 per unit
        wpc = 3 if hg == 1 and cols <= 16 and len(lens) * NG <= 512 else 4
    cap = max_blocks_per_seq * block_size
    W = decode_wgs(len(lens), NG, hg, chunks_per_row(max_blocks_per_seq, block_size) + (1 if step else 0),
                   override, wpc)
    segs = plain_segments(lens, cap, step)
    sp = walk(segs, NG, W)
    if W > 1:
        merge(sp, segs, NG, len(lens))
    # every sequence row: once per head group, or zeroed when empty
    for s, seg in enumerate(segs):
        for g in range(NG):
            times = sp.written.get((s, g), 0)
            want = 0 if seg.L == 0 else 1
            assert times == want, f"output of sequence {s}, head group {g} written {times} times"
    return sp


def share_plan(lens, group_starts, shared_blocks, max_blocks_per_seq, block_size, members_per_item,
               shared_prev=None):
    """share_plan_kernel: items (segments) of a sharing-aware call, group
    form, or chain form when ``shared_prev`` is given. Returns (items, zeroed
    rows, member records) with each item as a dict of its fields and each
    member record as (clamped context length, chunks before its own)."""
    S = len(lens)
    C = members_per_item
    cap = max_blocks_per_seq * block_size
    n = [min(max(int(x), 0), cap) for x in lens]
    grp = [-1] * S
    if shared_prev is not None:
        gs, shb = [], []
        common = [0] * S
        for i in range(1, S):
            blocks = min(min(max(int(shared_prev[i]), 0), max_blocks_per_seq), min(n[i], n[i - 1]) // block_size)
            common[i] = blocks * block_size // CHUNK
        run = 0
        opens, own = [], []
        for i in range(S):
            if common[i] == 0:
                run = i
            op = (i - run) % C == 0
            opens.append(op)
            own.append(0 if op else common[i])
    else:
        gs = [int(x) for x in group_starts] if len(shared_blocks) else []
        G = len(shared_blocks)
        shb = [min(max(int(x), 0), max_blocks_per_seq) for x in shared_blocks]
        valid = True
        for g in range(G):
            lo, hi = gs[g], gs[g + 1]
            if lo > hi or (g == 0 and lo < 0) or (g == G - 1 and hi > S):
                valid = False
        if valid:
            marks = [-1] * S
            for g in range(G):
                if gs[g + 1] > gs[g]:
                    marks[gs[g]] = g
            run = -1
            for i in range(S):
                run = max(run, marks[i])
                grp[i] = run
        for i in range(S):
            g = grp[i]
            if g >= 0 and i >= gs[g + 1]:
                grp[i] = -1
        for i in range(S):
            g = grp[i]
            if g >= 0:
                shb[g] = min(shb[g], n[i] // block_size)
        opens = [grp[i] < 0 or (i - gs[grp[i]]) % C == 0 for i in range(S)]
        own = [0 if opens[i] else shb[grp[i]] * block_size // CHUNK for i in range(S)]
    csum, acc = [], 0
    for i in range(S):
        acc += (n[i] + CHUNK - 1) // CHUNK - own[i]
        csum.append(acc)
    items, zeroed = [], []
    for i in range(S):
        if not opens[i]:
            continue
        ntok = 1
        while ntok < C and i + ntok < S and not opens[i + ntok]:
            ntok += 1
        start = csum[i - 1] if i > 0 else 0
        blocks = csum[i + ntok - 1] - start
        g = grp[i]
        eb = shb[g] if g >= 0 else 0
        items.append(dict(row=gs[g] if g >= 0 else i, qrow=i, ntok=ntok, b0=eb * block_size // CHUNK, eb=eb,
                          L=blocks))
        if blocks == 0:
            zeroed.extend(range(i, i + ntok))
    return items, zeroed, list(zip(n, own))


def _chunks(n: int) -> int:
    return (n + CHUNK - 1) // CHUNK


def member_lanes(item, members):
    """member_info: lane j's (context length, chunks before its own) for
    member j of the item, the second clamped to the member's chunks."""
    out = []
    for j in range(item["ntok"]):
        n, y = members[item["qrow"] + j]
        n = max(n, 0)
        out.append((n, min(max(y, 0), _chunks(n))))
    return out


def seg_at(item, lanes, j, b, nj):
    """The kernel's cursor of member j's chunk b: (j, e, b, n, row)."""
    stop = [k for k in range(j + 1, item["ntok"]) if lanes[k][1] <= b]
    e = stop[0] - 1 if stop else item["ntok"] - 1
    return (j, e, b, nj, item["row"] if b < item["b0"] else item["qrow"] + j)


def seg_first(item, lanes, off):
    r, j, nj, yj = off, 0, 0, 0
    while j < item["ntok"]:
        nj, yj = lanes[j]
        lj = _chunks(nj) - yj
        if r < lj:
            break
        r -= lj
        j += 1
    if j == item["ntok"]:
        j -= 1
    return seg_at(item, lanes, j, yj + r, nj)


def seg_next(item, lanes, c):
    j, _, b, n, _ = c
    if b + 1 < _chunks(n):
        return seg_at(item, lanes, j, b + 1, n)
    for k in range(j + 1, item["ntok"]):
        nk, yk = lanes[k]
        if _chunks(nk) > yk:
            return seg_at(item, lanes, k, yk, nk)
    return c


def check_item_stream(item, members, tables=None, block_size=16):
    """Walks an item's stream the way the decode kernel does (seg_first at
    every offset, seg_next between) and checks what each member sees:
      * the stream has the item's L chunks, and seg_first at any offset
        agrees with seg_next from the start;
      * every member sees each chunk of its context exactly once, and with
        the reader's context length as the limit, it sees exactly its own
        positions of that chunk;
      * with ``tables`` (a true declaration), the cache blocks read for a
        member hold its own tokens: the reader's table row (the segment's
        row for the blocks of the group prefix) names the same physical
        blocks as the member's own row for those tokens.
    Returns the stream as a list of cursors."""
    lanes = member_lanes(item, members)
    L = item["L"]
    stream = []
    if L > 0:
        c = seg_first(item, lanes, 0)
        for off in range(L):
            assert seg_first(item, lanes, off) == c, f"seg_first({off}) disagrees with the walk"
            stream.append(c)
            c = seg_next(item, lanes, c)
    seen = {}
    for (j, e, b, nj, row) in stream:
        assert 0 <= j <= e < item["ntok"]
        for k in range(j, e + 1):
            nk = lanes[k][0]
            key = (k, b)
            assert key not in seen, f"member {k} sees chunk {b} twice"
            seen[key] = (j, row, nj)
            assert min(CHUNK, nj - b * CHUNK) == min(CHUNK, nk - b * CHUNK), \
                f"member {k}: chunk {b} limit {nj} differs from its own context {nk}"
    for k in range(item["ntok"]):
        got = sorted(b for (kk, b) in seen if kk == k)
        assert got == list(range(_chunks(lanes[k][0]))), f"member {k} sees chunks {got}"
    if tables is not None:
        t = np.asarray(tables)
        bs = block_size
        for (k, b), (j, row, nj) in seen.items():
            own_row = item["qrow"] + k
            for tok in range(b * CHUNK, min((b + 1) * CHUNK, lanes[k][0])):
                blk = tok // bs
                if bs < CHUNK:  # the chunk's first block may come through the segment's row
                    rr = item["row"] if (blk == 2 * b and blk < item["eb"]) else row
                else:
                    rr = row
                assert t[rr, blk] == t[own_row, blk], \
                    f"member {k} token {tok}: block {t[rr, blk]} read, its table has {t[own_row, blk]}"
    return stream


def check_shared(lens, group_starts, shared_blocks, num_q_heads, num_kv_heads, max_blocks_per_seq,
                 block_size=16, override=None, shared_prev=None, tables=None) -> Split:
    group = num_q_heads // num_kv_heads
    C = 32 // group
    hg = heads_per_workgroup(num_kv_heads)
    NG = num_kv_heads // hg
    W = decode_wgs(len(lens), NG, hg, chunks_per_row(max_blocks_per_seq, block_size), override)
    items, zeroed, members = share_plan(lens, group_starts, shared_blocks, max_blocks_per_seq, block_size, C,
                                        shared_prev)
    assert len(items) <= len(lens)
    segs = [Segment(key=v, L=it["L"], rows=tuple(range(it["qrow"], it["qrow"] + it["ntok"])))
            for v, it in enumerate(items)]
    for it in items:
        assert 0 <= it["qrow"] and it["qrow"] + it["ntok"] <= len(lens) and it["ntok"] * group <= 32
        check_item_stream(it, members, tables, block_size)
    sp = walk(segs, NG, W)
    if W > 1:
        merge(sp, segs, NG, len(items))
    for s in range(len(lens)):
        for g in range(NG):
            times = sp.written.get((s, g), 0) + (1 if s in zeroed else 0)
            assert times == 1, f"output of sequence {s}, head group {g} written {times} times"
    return sp


def prologue_search(lens, cap: int, nthr: int, NG: int, W: int, w: int, step: bool = False, tile: int = 16):
    """The decode prologue with more sequences than threads: thread t sums
    the units of its contiguous range of K = ceil(S / nthr) sequences, read
    in tiles; an exclusive scan over the threads gives each range's first
    chunk; the thread whose range holds `lo` walks it again to find the
    sequence. Returns (total units, lo, hi, found sequence, its first chunk,
    its length) or None for a workgroup past the last one with units."""
    S = len(lens)
    K = (S + nthr - 1) // nthr
    n_of = [min(max(int(x), 0), cap) for x in lens]

    def chunks(n):
        return ((n - 1 + CHUNK - 1) // CHUNK + 1 if n > 0 else 0) if step else (n + CHUNK - 1) // CHUNK

    mine = []
    for t in range(nthr):
        s0, s1 = min(t * K, S), min(t * K + K, S)
        acc = 0
        for s in range(s0, s1, tile):
            vals = [n_of[s + k] if s + k < S else 0 for k in range(tile)]  # the buffer range reads 0 past S
            for k in range(tile):
                if s + k < s1:
                    acc += chunks(vals[k])
        mine.append(acc)
    U = sum(mine) * NG
    E = min(U, W)
    if w >= E:
        return None
    lo, hi = range_lo(w, U, E), range_lo(w + 1, U, E)
    found = []
    excl = 0
    for t in range(nthr):
        s0, s1 = min(t * K, S), min(t * K + K, S)
        if mine[t] > 0 and excl * NG <= lo < (excl + mine[t]) * NG:
            acc = excl
            for s in range(s0, s1):
                L = chunks(n_of[s])
                if L > 0 and acc * NG <= lo < (acc + L) * NG:
                    found.append((s, acc, n_of[s]))
                    break
                acc += L
        excl += mine[t]
    assert len(found) == 1, f"{len(found)} threads found the sequence holding unit {lo}"
    return (U, lo, hi) + found[0]
