"""GPU parity on the full-size decode workloads, with the launch
configuration the benchmark times (default split policy).

The slot scatter is checked bitwise over the whole cache. Attention is
checked element by element against the float64 oracle on the longest and
shortest sequences plus a seeded sample (all sequences where the oracle is
quick enough). Seeds and sizes follow paged_kv_cache_433_amd.workloads.
"""

import numpy as np
import pytest

import oracle
from gpu_util import DevBatch, assert_attention_close, bits_of, note, to_dev, to_dev_bf16
from paged_kv_cache_433_amd import workloads as W

pytestmark = pytest.mark.gpu

SAMPLE = {"llama2_7b": 24, "llama3_8b_gqa": 40, "long_splitk": 8, "long_splitk_max": 2, "llama3_8b_gqa_tp8": 40}


@pytest.mark.parametrize("name", ["llama2_7b", "llama3_8b_gqa", "long_splitk", "long_splitk_max",
                                  "llama3_8b_gqa_tp8"])
def test_full_size_config(name):
    note(f"generate {name}")
    b = W.make_config(name)
    note(f"{name}: scatter + decode, {b.num_seqs} seqs, sum(n)={int(b.context_lens.sum())}")
    db = DevBatch(b)
    db.scatter()
    out = bits_of(db.decode())
    oracle.reshape_and_cache(b.k_cache, b.v_cache, b.new_k, b.new_v, b.slot_mapping)
    assert np.array_equal(bits_of(db.k_cache), b.k_cache), "k_cache after scatter"
    assert np.array_equal(bits_of(db.v_cache), b.v_cache), "v_cache after scatter"
    lens = b.context_lens
    rng = np.random.default_rng(1234)
    pick = {int(np.argmax(lens)), int(np.argmin(lens))}
    pick |= set(rng.choice(b.num_seqs, size=min(SAMPLE[name], b.num_seqs), replace=False).tolist())
    idx = np.array(sorted(pick))
    note(f"{name}: oracle on {len(idx)} sequences")
    ref = oracle.decode(b.q[idx], b.k_cache, b.v_cache, b.block_tables[idx], lens[idx], b.scale)
    assert_attention_close(out[idx], ref, name)


def test_beam_search_copy_on_write_steps():
    """64 prompts x 4 beams sharing a 1024-token prompt; 16 steps of fork,
    copy-on-write of diverging last blocks, one-token scatter and decode."""
    import paged_kv_cache_433_amd as pa
    note("generate beam_cow")
    wl = W.BeamSearchWorkload()
    kd, vd = to_dev_bf16(wl.k_cache), to_dev_bf16(wl.v_cache)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    rng = np.random.default_rng(55)
    total_pairs = 0
    for step in range(16):
        b = wl.step()
        total_pairs += len(b.cow_pairs)
        note(f"beam step {step}: {len(b.cow_pairs)} CoW pairs, unique blocks {wl.unique_blocks()}")
        if len(b.cow_pairs):
            pa.copy_blocks(kd, vd, to_dev(b.cow_pairs))
        oracle.copy_blocks(kc, vc, b.cow_pairs)
        pa.reshape_and_cache(to_dev_bf16(b.new_k), to_dev_bf16(b.new_v), kd, vd, to_dev(b.slot_mapping))
        oracle.reshape_and_cache(kc, vc, b.new_k, b.new_v, b.slot_mapping)
        out = bits_of(pa.decode(to_dev_bf16(b.q), kd, vd, to_dev(b.block_tables),
                                to_dev(b.context_lens), float(b.scale)))
        idx = np.arange(b.num_seqs) if step == 15 else np.sort(rng.choice(b.num_seqs, 8, replace=False))
        ref = oracle.decode(b.q[idx], kc, vc, b.block_tables[idx], b.context_lens[idx], b.scale)
        assert_attention_close(out[idx], ref, f"beam step {step}")
    assert total_pairs > 0
    assert np.array_equal(bits_of(kd), kc) and np.array_equal(bits_of(vd), vc)
