"""Mutation check of the oracle's pins.

Each mutation below is a plausible mistake (a dropped term, a wrong sign or
index, a transposed operand) planted in a private copy of the oracle's source
on the CPU.  The pins of test_oracle_pins.py must reject every one of them;
a mutation that survives means the pins leave that part of the oracle
unconstrained.
"""
import inspect
import types

import pytest

import oracle.uniprefill_oracle as O
import test_oracle_pins as PINS

MUTATIONS = {
    "causal_off_by_one": ("cols <= rows", "cols < rows"),
    "no_causal_mask": ("s = np.where(cols <= rows, s, -np.inf)", "s = s"),
    "softmax_over_queries": ("e / e.sum(axis=1, keepdims=True)", "e / e.sum(axis=0, keepdims=True)"),
    "scale_dropped": ("s = scale * (q_tail @ keys.T)", "s = (q_tail @ keys.T)"),
    "scale_sqrt_missing": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "gqa_interleaved": ("g = h // r", "g = h % hkv"),
    "n_not_clamped": ("n_eff = min(int(n), int(L))", "n_eff = int(n)"),
    "tail_rows_shifted": ("return L - n_eff, L", "return L - n_eff - 1, L - 1"),
    "block_mean_over_G": ("c[s0 + j0:s0 + j1].sum() / (j1 - j0)", "c[s0 + j0:s0 + j1].sum() / G"),
    "block_sum_not_mean": ("c[s0 + j0:s0 + j1].sum() / (j1 - j0)", "c[s0 + j0:s0 + j1].sum()"),
    "tail_forced_off_by_one": ("(j1 > L - tail)", "(j1 > L - tail + G)"),
    "sink_forced_inclusive": ("(j0 < sink)", "(j0 <= sink)"),
    "threshold_exclusive": ("if acc >= target:\n            break", "if acc > target:\n            break"),
    "forced_mass_ignored": ("        if forced[b]:\n            acc += float(bs[b])", "        pass"),
    "ties_high_index_first": ("key=lambda b: (-float(bs[b]), b))\n    for b in order:\n        if acc",
                              "key=lambda b: (-float(bs[b]), -b))\n    for b in order:\n        if acc"),
    "ascending_order": ("key=lambda b: (-float(bs[b]), b))\n    for b in order:\n        if acc",
                        "key=lambda b: (float(bs[b]), b))\n    for b in order:\n        if acc"),
    "p_applied_to_optional_only": ("target = p * total\n    keep = forced.copy()",
                                   "target = p * (total - sum(float(bs[x]) for x in range(nb) if forced[x]))\n    keep = forced.copy()"),
    "compact_global_block_index": ("if mask[cub[b] + j // G]:\n                rows.append",
                                   "if mask[(s0 + j) // G]:\n                rows.append"),
    "kept_tokens_full_blocks": ("kept[b] += min(blk * G + G, L) - blk * G", "kept[b] += G"),
    "history_cumulative": ("int(cu_out[b + 1]) - int(cu_out[b])", "int(cu_out[b + 1])"),
    "kv_len_strict": ("if lid <= layer and", "if lid < layer and"),
    "kv_len_first_not_latest": ("(best is None or lid >= best[0])", "(best is None)"),
    "revival_global_block_index": ("if mask[cub[b] + j // G]:\n                out[s0 + j]",
                                   "if mask[(s0 + j) // G]:\n                out[s0 + j]"),
    "revival_row_not_advanced": ("out[s0 + j] = packed[r]\n                r += 1",
                                 "out[s0 + j] = packed[r]"),
    "revival_local_row": ("out[s0 + j] = packed[r]", "out[j] = packed[r]"),
    "round_no_subnormals": ("q = np.maximum(e - p, emin - p + 1)", "q = e - p"),
    "round_truncates": ("np.ldexp(np.round(np.ldexp(x, -q)), q)", "np.ldexp(np.trunc(np.ldexp(x, -q)), q)"),
    "round_extra_bit": ("q = np.maximum(e - p, emin - p + 1)", "q = np.maximum(e - p - 1, emin - p)"),
    "rms_sum_not_mean": ("(rows * rows).sum(axis=1, keepdims=True) / rows.shape[1]",
                         "(rows * rows).sum(axis=1, keepdims=True)"),
    "rms_eps_outside_sqrt": ("y = rows / np.sqrt(ms + eps)", "y = rows / (np.sqrt(ms) + eps)"),
    "rms_gain_dropped": ("y = y * np.asarray(gamma, dtype=np.float64)[None, :]", "y = y"),
    "compact_rmsnorm_gain_dropped": ("return rms_normalize(h, gamma, eps), p_out, cu_out",
                                     "return rms_normalize(h, None, eps), p_out, cu_out"),
    "band_one_sided": ("if c1 >= p - eps and c0 <= p + eps:", "if c1 >= p + eps and c0 <= p + eps:"),
    "trace_forced_mass_ignored": ("acc = float(sum(float(bs[b]) for b in range(len(bs)) if forced[b]))",
                                  "acc = 0.0"),
    "gather_add_sign": ("return round_to_format(h + d, fmt)", "return round_to_format(h - d, fmt)"),
    "chain_sink_tail_swapped": ("mask, kept = select_topp(bsc, cu_seqlens, G, p, sink, tail)",
                                "mask, kept = select_topp(bsc, cu_seqlens, G, p, tail, sink)"),
    "chain_block_size_as_n": ("c = token_scores(q, k, cu_seqlens, n_query, scale)",
                              "c = token_scores(q, k, cu_seqlens, G, scale)"),
    "chain_n_as_block_size": ("bsc = block_scores(c, cu_seqlens, G)",
                              "bsc = block_scores(c, cu_seqlens, n_query)"),
    "chain_layer_id_ignored": ("history_append(ledger, layer_id, cu_out)",
                               "history_append(ledger, 0, cu_out)"),
    "chain_p_ignored": ("mask, kept = select_topp(bsc, cu_seqlens, G, p, sink, tail)",
                        "mask, kept = select_topp(bsc, cu_seqlens, G, 0.99, sink, tail)"),
    "gather_add_delta_shifted": ("d = np.asarray(delta, dtype=np.float64)[: len(h)]",
                                 "d = np.asarray(delta, dtype=np.float64)[1: len(h) + 1]"),
}


def _mutant(old, new):
    src = inspect.getsource(O)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    old, new = MUTATIONS[name]
    monkeypatch.setattr(PINS, "O", _mutant(old, new))
    failed = []
    for check in PINS.ALL_CHECKS:
        try:
            check()
        except Exception:  # AssertionError or a crash both count as caught
            failed.append(check.__name__)
            break
    assert failed, f"no pin rejects mutation {name}"


def test_unmutated_passes_all(monkeypatch):
    monkeypatch.setattr(PINS, "O", _mutant("import math", "import math"))
    for check in PINS.ALL_CHECKS:
        check()
