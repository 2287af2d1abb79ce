"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them."""

import pathlib
import types

import pytest

from oracle_pins import ALL_PINS

SRC = (pathlib.Path(__file__).resolve().parents[1] / "oracle" / "paged_attention.py").read_text()

MUTANTS = {
    "kv head h % Hkv instead of h // G": ("range(kv_head * group, (kv_head + 1) * group)",
                                          "range(kv_head, num_q_heads, num_kv_heads)"),
    "block index from offset": ("[positions // block_size]", "[positions % block_size]"),
    "offset from block index": ("offsets = positions % block_size", "offsets = positions // block_size"),
    "scale dropped": ("z = scale64 * (keys @ qf[h])", "z = (keys @ qf[h])"),
    "scale applied twice": ("z = scale64 * (keys @ qf[h])", "z = scale64 * scale64 * (keys @ qf[h])"),
    "weights applied to keys": ("out[h] = p @ values", "out[h] = p @ keys"),
    "normalised by max": ("p = w / w.sum()", "p = w / w.max()"),
    "wrong sign in exponent": ("w = np.exp(z - z.max())", "w = np.exp(z.max() - z)"),
    "last token dropped": ("positions = np.arange(n)", "positions = np.arange(n - 1)"),
    "K and V swapped in scatter": ("k_cache[blk, off] = k[t]", "k_cache[blk, off] = v[t]"),
    "scatter off by one": ("blk, off = divmod(int(slot), block_size)",
                           "blk, off = divmod(int(slot) + 1, block_size)"),
    "negative slot not skipped": ("if slot < 0:\n            continue", "if False:\n            continue"),
    "copy reads V into K": ("k_cache[d] = k_src[i]", "k_cache[d] = v_src[i]"),
    "copy direction reversed": ("k_src = k_cache[src].copy()", "k_src = k_cache[dst].copy()"),
    "widening shift wrong": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "causal limit off by one": ("n - q_len + j + 1, scale)", "n - q_len + j, scale)"),
    "new tokens in reverse order": ("decode_sequence(q[s, j], k_cache", "decode_sequence(q[s, q_len - 1 - j], k_cache"),
    "swap direction ignored": ('if direction == "out":', 'if direction != "out":'),
    "swap copies K into V": ("tv[d_] = fv[s_]", "tv[d_] = fk[s_]"),
    "shared prefix read through own table": ("tables[j, :e] = block_tables[lo, :e]",
                                             "tables[j, :e] = block_tables[j, :e]"),
    "shared prefix not clamped to members": ("e = max(0, min(int(shared[g]), full, tables.shape[1]))",
                                             "e = max(0, min(int(shared[g]), tables.shape[1]))"),
    "shared prefix counts partial blocks": ("full = min(int(context_lens[j]) // block_size",
                                            "full = min(-(-int(context_lens[j]) // block_size)"),
    "negative shared prefix not clamped": ("e = max(0, min(int(shared[g]), full, tables.shape[1]))",
                                           "e = min(int(shared[g]), full, tables.shape[1])"),
    "group end taken inclusive": ("for j in range(lo + 1, hi):", "for j in range(lo + 1, hi + 1):"),
    "query heads transposed": ("qf = bf16_bits_to_f64(q_s)", "qf = bf16_bits_to_f64(q_s)[::-1]"),
    "tree prefix read through own table": ("tables[i, :e] = tables[i - 1, :e]", "tables[i, :e] = tables[i, :e]"),
    "tree chain not followed": ("tables[i, :e] = tables[i - 1, :e]", "tables[i, :e] = block_tables[i - 1, :e]"),
    "tree prefix clamped to own blocks only": ("n[i] // block_size, n[i - 1] // block_size))",
                                               "n[i] // block_size))"),
    "tree negative declaration not clamped": ("e = max(0, min(int(declared[i]), n[i]",
                                              "e = (min(int(declared[i]), n[i]"),
    "tree first declaration used": ("for i in range(1, len(n)):\n        e = max(0, min(int(declared[i])",
                                    "for i in range(0, len(n)):\n        e = max(0, min(int(declared[i])"),
}


def mutant_module(old, new):
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = mutant_module(*MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the mutant '{name}'"
