"""The log-sum-exp merge of partition partials equals one softmax.

The GPU path splits long contexts into partitions; each yields the running
maximum m_p (base 2), the sum l_p of 2^(z - m_p) and the unnormalised
output o_p; the merge rescales by 2^(m_p - M). This float64 model of that
rewrite checks the identity against the oracle's single softmax; it is not
an oracle itself."""

import numpy as np
import pytest

import oracle
from oracle_pins import small_batch, scattered, widen

LOG2E = 1.4426950408889634


def split_then_merge(q, keys, values, scale, part):
    n = keys.shape[0]
    ms, ls, os_ = [], [], []
    for lo in range(0, n, part):
        z = (keys[lo:lo + part] @ q) * scale * LOG2E
        m = z.max()
        w = np.exp2(z - m)
        ms.append(m)
        ls.append(w.sum())
        os_.append(w @ values[lo:lo + part])
    M = max(ms)
    r = [np.exp2(m - M) for m in ms]
    return sum(ri * o for ri, o in zip(r, os_)) / sum(ri * li for ri, li in zip(r, ls))


@pytest.mark.parametrize("part", [16, 32, 48, 512])
def test_lse_merge_equals_single_softmax(part):
    b = small_batch(41, [1, 15, 100, 700], 4, 2, 16)
    kc, vc = scattered(oracle, b)
    ref = oracle.decode(b.q, kc, vc, b.block_tables, b.context_lens, b.scale)
    for s, n in enumerate(b.context_lens):
        n = int(n)
        pos = np.arange(n)
        blk, off = b.block_tables[s][pos // 16], pos % 16
        for h in range(4):
            keys = widen(kc[blk, off, h // 2])
            vals = widen(vc[blk, off, h // 2])
            got = split_then_merge(widen(b.q[s, h]), keys, vals, float(b.scale), part)
            assert np.abs(got - ref[s, h]).max() <= 1e-13
