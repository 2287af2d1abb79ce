"""Oracle vs scalar loops with math.fsum on tiny random inputs (a second,
independent spelling of the definition; the closed forms and library checks
in test_oracle_pins.py are the primary pins)."""

import math

import numpy as np
import pytest

import oracle
from oracle_pins import small_batch, scattered, widen


def brute(q, kc, vc, table, n, scale, G):
    Hq, D = q.shape
    out = []
    for h in range(Hq):
        g = h // G
        z = []
        for i in range(n):
            blk, off = int(table[i // 16]), i % 16
            z.append(float(scale) * math.fsum(float(q[h, d]) * float(kc[blk, off, g, d]) for d in range(D)))
        m = max(z)
        w = [math.exp(x - m) for x in z]
        tot = math.fsum(w)
        out.append([math.fsum(w[i] / tot * float(vc[int(table[i // 16]), i % 16, g, d]) for i in range(n))
                    for d in range(D)])
    return np.array(out)


@pytest.mark.parametrize("seed", range(6))
def test_oracle_matches_scalar_loops(seed):
    rng = np.random.default_rng(100 + seed)
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([4, 8]))
    lens = [int(x) for x in rng.integers(1, 41, size=3)]
    b = small_batch(200 + seed, lens, hkv * G, hkv, D)
    kc, vc = scattered(oracle, b)
    out = oracle.decode(b.q, kc, vc, b.block_tables, b.context_lens, b.scale)
    qf, kf, vf = widen(b.q), widen(kc), widen(vc)
    for s, n in enumerate(lens):
        ref = brute(qf[s], kf, vf, b.block_tables[s], n, np.float32(b.scale), G)
        assert np.abs(out[s] - ref).max() <= 1e-12
