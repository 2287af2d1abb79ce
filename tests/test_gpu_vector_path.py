"""GPU parity of the two ways a single-token decode with one query head per
KV head can compute: on matrix cores (16-column tiles, one column live) and
on the vector ALU (token-parallel lanes, bf16 dot products, a per-lane
online softmax merged across lanes at each piece's end). Both must match
the float64 oracle across head sizes, work splits, block sizes, the fused
step, and the full-size MHA layer; PA_DECODE_PATH picks the path."""

import numpy as np
import pytest

import oracle
from gpu_util import DevBatch, assert_attention_close, bits_of, note, oracle_step, to_dev, to_dev_bf16
from oracle_pins import small_batch
from paged_kv_cache_433_amd import workloads as W

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 100, 511, 512, 513, 1000, 1024, 1031]
PATHS = ["vector", "mfma"]


def decode_and_step(b, what):
    """pa_decode after pa_reshape_and_cache, and pa_decode_step, against the
    oracle's scatter + decode."""
    import paged_kv_cache_433_amd as pa
    note(what)
    kc, vc, ref, _ = oracle_step(b)
    db = DevBatch(b)
    db.scatter()
    assert_attention_close(bits_of(db.decode()), ref, f"{what} decode")
    db2 = DevBatch(b)
    out = pa.decode_step(db2.q, db2.new_k, db2.new_v, db2.k_cache, db2.v_cache, db2.block_tables,
                         db2.context_lens, float(b.scale))
    assert np.array_equal(bits_of(db2.k_cache), kc) and np.array_equal(bits_of(db2.v_cache), vc)
    assert_attention_close(bits_of(out), ref, f"{what} step")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("hkv,d", [(8, 64), (8, 128), (7, 64), (1, 128), (32, 128)])
def test_one_head_per_kv_head_across_work_splits(path, hkv, d, monkeypatch):
    monkeypatch.setenv("PA_DECODE_PATH", path)
    b = small_batch(3100 + hkv + d, EDGE_LENS, hkv, hkv, d, spare=11)
    for wgs in ("1", "3", "64", "default", "5000"):
        if wgs == "default":
            monkeypatch.delenv("PA_DECODE_WGS", raising=False)
        else:
            monkeypatch.setenv("PA_DECODE_WGS", wgs)
        decode_and_step(b, f"{path} hkv={hkv} d={d} wgs={wgs}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bs", [8, 32])
def test_one_head_per_kv_head_block_sizes(path, bs, monkeypatch):
    monkeypatch.setenv("PA_DECODE_PATH", path)
    lens = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 255, 1000]
    nb = int(sum((n + bs - 1) // bs for n in lens)) + 9
    b = W.make_batch("vec", 3200 + bs, lens, 8, 8, 128, nb, block_size=bs)
    for wgs in ("1", "5", "default"):
        if wgs == "default":
            monkeypatch.delenv("PA_DECODE_WGS", raising=False)
        else:
            monkeypatch.setenv("PA_DECODE_WGS", wgs)
        decode_and_step(b, f"{path} bs={bs} wgs={wgs}")


def test_vector_path_single_token_and_indexing(monkeypatch):
    """context_len = 1 gives that token's V bit for bit on the vector path
    too, and the one-hot probe reads exactly the targeted position."""
    import paged_kv_cache_433_amd as pa
    from oracle_pins import onehot_probe
    monkeypatch.setenv("PA_DECODE_PATH", "vector")
    b = small_batch(3300, [1, 1, 1], 8, 8, 128, spare=3)
    db = DevBatch(b)
    db.scatter()
    out = bits_of(db.decode())
    assert np.array_equal(out, b.new_v.reshape(out.shape)), "n = 1 must return V exactly"
    lens = [37, 100, 16, 1, 513, 2000]
    b = small_batch(3301, lens, 8, 8, 128)
    kc, vc = b.k_cache.copy(), b.v_cache.copy()
    oracle.reshape_and_cache(kc, vc, b.new_k, b.new_v, b.slot_mapping)
    rng = np.random.default_rng(9)
    targets = [[int(rng.integers(0, n)) for _ in range(8)] for n in lens]
    q, G = onehot_probe(b, kc, vc, targets)
    note("vector path one-hot probe")
    got = oracle.bf16_bits_to_f64(bits_of(pa.decode(to_dev_bf16(q), to_dev_bf16(kc), to_dev_bf16(vc),
                                                    to_dev(b.block_tables), to_dev(b.context_lens),
                                                    float(b.scale))))
    for s, n in enumerate(lens):
        for h in range(8):
            j = targets[s][h]
            assert got[s, h, 0] == j % 256 and got[s, h, 1] == j // 256 and got[s, h, 2] == h, (s, h, j)


def test_vector_path_deterministic(monkeypatch):
    monkeypatch.setenv("PA_DECODE_PATH", "vector")
    b = small_batch(3400, EDGE_LENS, 8, 8, 128, spare=11)
    db = DevBatch(b)
    db.scatter()
    note("vector path twice")
    assert np.array_equal(bits_of(db.decode()), bits_of(db.decode()))


@pytest.mark.parametrize("path", PATHS)
def test_mha_layer_full_size(path, monkeypatch):
    """The Llama-2-7B-shaped MHA layer (64 sequences, 32/32 heads), fused
    step, every output against the oracle."""
    from oracle_pool import oracle_batch
    import paged_kv_cache_433_amd as pa
    monkeypatch.setenv("PA_DECODE_PATH", path)
    b = W.make_config("llama2_7b")
    note(f"{path}: llama2_7b full size step")
    db = DevBatch(b)
    out = pa.decode_step(db.q, db.new_k, db.new_v, db.k_cache, db.v_cache, db.block_tables, db.context_lens,
                         float(b.scale))
    oracle.reshape_and_cache(b.k_cache, b.v_cache, b.new_k, b.new_v, b.slot_mapping)
    assert np.array_equal(bits_of(db.k_cache), b.k_cache)
    ref = oracle_batch("decode", b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale)
    assert_attention_close(bits_of(out), ref, f"{path} llama2_7b full size")
