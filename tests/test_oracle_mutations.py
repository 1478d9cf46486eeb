"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pin battery catches each one: a wrong head mapping, index, sign, missing
term, transposed operand or wrong rounding must fail at least one pin."""
import os
import types

import pytest

import _oracle_pins as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "paged_attention.py")
PREFIX_SRC = os.path.join(ORACLE_DIR, "prefix_cache.py")

MUTATIONS = {
    "interleaved_kv_heads": ("return h // (num_q_heads // num_kv_heads)",
                             "return h % num_kv_heads"),
    "offset_off_by_one": ("return int(block_table_row[pos // BLOCK]), pos % BLOCK",
                          "return int(block_table_row[pos // BLOCK]), (pos + 1) % BLOCK"),
    "k_reversed_dims": ("return k_cache[block, :, :, off, :].reshape(hkv, -1)",
                        "return k_cache[block, :, :, off, ::-1].reshape(hkv, -1)"),
    "k_slices_reversed": ("return k_cache[block, :, :, off, :].reshape(hkv, -1)",
                          "return k_cache[block, :, ::-1, off, :].reshape(hkv, -1)"),
    "k_slice_major_read": ("return k_cache[block, :, :, off, :].reshape(hkv, -1)",
                           "return k_cache[block, :, :, off, :].swapaxes(1, 2).reshape(hkv, -1)"),
    "v_reversed_dims": ("return v_cache[block, :, :, off]",
                        "return v_cache[block, :, :, off][:, ::-1]"),
    "slot_block_offset_swapped": ("return slot // BLOCK, slot % BLOCK",
                                  "return slot % BLOCK, slot // BLOCK"),
    "scale_dropped": ("return scale * (q_rows_h @ K_g.T)", "return (q_rows_h @ K_g.T)"),
    "score_sign": ("return scale * (q_rows_h @ K_g.T)", "return -scale * (q_rows_h @ K_g.T)"),
    "softmax_sign": ("e = np.exp(z - m)\n    s = np.sum", "e = np.exp(m - z)\n    s = np.sum"),
    "diagonal_excluded": ("return prefix_len + np.arange(n_new) + 1",
                          "return prefix_len + np.arange(n_new)"),
    "prefix_ignored_in_mask": ("return prefix_len + np.arange(n_new) + 1",
                               "return np.arange(n_new) + 1"),
    "lse_missing_max": ("part_lse[s, h, p] = m + np.log(np.sum(e))",
                        "part_lse[s, h, p] = np.log(np.sum(e))"),
    "combine_weight_sign": ("w = np.exp(lse - M)", "w = np.exp(M - lse)"),
    "bf16_widen_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "write_k_from_v": ("kc[b, :, :, o, :] = np.asarray(k_new[t])",
                       "kc[b, :, :, o, :] = np.asarray(v_new[t])"),
    "write_k_slice_major": (
        "kc[b, :, :, o, :] = np.asarray(k_new[t]).reshape(kc.shape[1], kc.shape[2], kc.shape[4])",
        "kc[b, :, :, o, :] = np.asarray(k_new[t]).reshape(kc.shape[1], kc.shape[4], kc.shape[2]).swapaxes(1, 2)"),
    "decode_excludes_self": ("np.array([n]),", "np.array([n - 1]),"),
    "partitions_overlap": ("lo, hi = p * partition_size, min(n, (p + 1) * partition_size)",
                           "lo, hi = p * partition_size, min(n, (p + 1) * partition_size + 1)"),
    "prefill_prefix_not_gathered": ("gather_sequence(k_cache, v_cache, block_tables[s], P + N)",
                                    "gather_sequence(k_cache, v_cache, block_tables[s], N)"),
    "bf16_round_truncates": ("np.rint(np.ldexp(m, 8))", "np.trunc(np.ldexp(m, 8))"),
    "multi_window_shifted": ("visible = causal_visible(n - T, T)\n        out[s] = attend",
                             "visible = causal_visible(n - T + 1, T)\n        out[s] = attend"),
    "multi_tokens_reversed": ("out[s] = attend(qf[s], K, V, scale, visible",
                              "out[s] = attend(qf[s][::-1], K, V, scale, visible"),
    "multi_short_context_not_nan": ("            out[s] = np.nan\n", "            pass\n"),
    "copy_ids_swapped": ("s = i if src_ids is None else int(src_ids[i])\n        d = i if dst_ids is None else int(dst_ids[i])",
                         "d = i if src_ids is None else int(src_ids[i])\n        s = i if dst_ids is None else int(dst_ids[i])"),
    "copy_v_dst_index": ("dv[d] = src_v[s]", "dv[d] = src_v[d % src_v.shape[0]]"),
    "copy_skip_check_dropped": ("if not (0 <= s < src_k.shape[0] and 0 <= d < dk.shape[0]):",
                                "if not (-src_k.shape[0] <= s < src_k.shape[0] and 0 <= d < dk.shape[0]):"),
    "prefix_key_ignores_earlier_blocks": (
        PREFIX_SRC, "return tuple(int(t) for t in tokens[:BLOCK * (i + 1)])",
        "return tuple(int(t) for t in tokens[BLOCK * i:BLOCK * (i + 1)])"),
    "prefix_partial_block_registered": (
        PREFIX_SRC, "n = min(len(tokens) // BLOCK, len(block_ids))",
        "n = min((len(tokens) + BLOCK - 1) // BLOCK, len(block_ids))"),
    "prefix_remove_keeps_descendants": (
        PREFIX_SRC, "gone = [k for k in self.entries if any(k[:len(r)] == r for r in roots)]",
        "gone = roots"),
    "prefix_later_copy_replaces_first": (
        PREFIX_SRC, "while i < n and self._key(tokens, i) in self.entries:",
        "while i < n and self._key(tokens, i) in self.entries and False:"),
    "multi_partials_ignore_causal": ("lo, hi = p * partition_size, min(int(vis[t]), (p + 1) * partition_size)",
                                     "lo, hi = p * partition_size, min(n, (p + 1) * partition_size)"),
}


def _mutant(path, old, new):
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), path + " (mutant)", "exec"), mod.__dict__)
    return mod


def _mutated_oracle(spec):
    """The oracle package with one of its modules replaced by a mutant: every
    name the package exports, the mutant's definitions taking precedence, so
    a pin that exercises another module still runs (and a survivor is not
    counted as caught through a missing name)."""
    import oracle
    path, old, new = spec if len(spec) == 3 else (SRC, *spec)
    mod = _mutant(path, old, new)
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle)
                                  if not k.startswith("__")})
    for k in dir(mod):
        if not k.startswith("__"):
            setattr(ns, k, getattr(mod, k))
    return ns


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod = _mutated_oracle(MUTATIONS[name])
    monkeypatch.setattr(pins, "oracle", mod)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # AssertionError or a shape/index error
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"mutation {name} survived every oracle pin"
