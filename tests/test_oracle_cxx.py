"""The C++ oracle (oracle/uniprefill_oracle.cpp) against the same pins as the
numpy oracle, cross-checked against the numpy oracle, and mutation-checked.

- Every pin of test_oracle_pins.py runs with steps 1-5 served by the C++
  library (closed forms, textbook special cases, brute force, the hand-worked
  golden example and the invariants cited there).
- On random packed batches the two oracles agree: token and block scores to
  1e-12 relative (the C++ dot products sum in a different order than BLAS),
  masks, kept counts, compaction and ledger exactly.
- Plausible mistakes planted in private copies of the C++ source (compiled
  with g++ into temporary libraries, on the CPU) must each be rejected by at
  least one pin.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle.cxx as CX
import oracle.uniprefill_oracle as NP
import test_oracle_pins as PINS


@pytest.fixture(scope="module")
def cxx():
    return CX.module()


@pytest.mark.parametrize("check", PINS.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin_against_cxx(check, cxx, monkeypatch):
    monkeypatch.setattr(PINS, "O", cxx)
    check()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cxx_matches_numpy_oracle(seed, cxx):
    rng = np.random.default_rng(100 + seed)
    lengths = [int(x) for x in rng.integers(0, 700, size=4)] + [129, 1]
    hq, hkv, d = [(4, 2, 16), (6, 3, 8), (8, 8, 4)][seed]
    n, G, p = [(128, 64, 0.99), (37, 16, 0.8), (5, 32, 0.5)][seed]
    sink, tail = [(128, 128), (20, 70), (0, 1)][seed]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = rng.standard_normal((T, hq, d)) * 1.5
    k = rng.standard_normal((T, hkv, d))
    hidden = rng.integers(0, 2 ** 16, size=(T, 6), dtype=np.uint16)
    pos = rng.integers(0, 10 ** 6, size=T).astype(np.int32)
    a = NP.run_chain(q, k, hidden, pos, cu, n, G, p, sink, tail, layer_id=seed + 3)
    b = cxx.run_chain(q, k, hidden, pos, cu, n, G, p, sink, tail, layer_id=seed + 3)
    np.testing.assert_allclose(b["token_scores"], a["token_scores"], rtol=1e-12, atol=0)
    np.testing.assert_allclose(b["block_scores"], a["block_scores"], rtol=1e-12, atol=0)
    # the selections agree exactly unless a cumulative mass sits within the
    # scores' rounding difference of p * total (not the case for these seeds)
    for key in ("mask", "kept", "hidden_out", "positions_out", "cu_out"):
        np.testing.assert_array_equal(b[key], a[key], err_msg=key)
    assert b["ledger"] == a["ledger"]
    # bf16 bit-pattern inputs give the same scores as their exact fp64 values
    qb = (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(cxx.token_scores(qb, kb, cu, n),
                                  cxx.token_scores(NP.widen_bf16(qb), NP.widen_bf16(kb), cu, n))


CXX_MUTATIONS = {
    "causal_off_by_one": ("        for (int64_t j = 0; j <= i; ++j) {\n          double dot",
                          "        for (int64_t j = 0; j < i; ++j) {\n          double dot"),
    "gqa_interleaved": ("const int g = h / group;", "const int g = h % hkv;"),
    "scale_sqrt_missing": ("scale = 1.0 / std::sqrt(static_cast<double>(d));",
                           "scale = 1.0 / static_cast<double>(d);"),
    "n_clamp_off_by_one": ("const int64_t n_eff = std::min<int64_t>(n_query, L);",
                           "const int64_t n_eff = std::min<int64_t>(n_query, L) - (n_query >= L);"),
    "not_normalised": ("c[s0 + j] += s[j] / l;", "c[s0 + j] += s[j];"),
    "wrong_key_operand": ("element(k, k_kind, k_tok, k_head, s0 + j, g, t);",
                          "element(k, k_kind, k_tok, k_head, s0 + i, g, t);"),
    "block_mean_over_G": ("out[nb++] = sum / static_cast<double>(j1 - j0);",
                          "out[nb++] = sum / static_cast<double>(G);"),
    "sink_inclusive": ("out[b] = (j0 < sink || j1 > L - tail) ? 1 : 0;",
                       "out[b] = (j0 <= sink || j1 > L - tail) ? 1 : 0;"),
    "tail_off_by_one": ("out[b] = (j0 < sink || j1 > L - tail) ? 1 : 0;",
                        "out[b] = (j0 < sink || j1 > L - tail + 1) ? 1 : 0;"),
    "threshold_exclusive": ("if (acc >= target) break;", "if (acc > target) break;"),
    "forced_mass_ignored": ("    if (keep[b]) acc += bs[b];\n", "    if (keep[b]) acc += 0.0;\n"),
    "ties_high_index_first": ("(bs[a] == bs[b] && a < b)", "(bs[a] == bs[b] && a > b)"),
    "ascending_order": ("return bs[a] > bs[b] ||", "return bs[a] < bs[b] ||"),
    "p_on_optional_only": ("  const double target = p * total;\n  double acc = 0.0;",
                           "  double forced_mass = 0.0;\n  for (int64_t b = 0; b < nb; ++b) if (keep[b]) forced_mass += bs[b];\n"
                           "  const double target = p * (total - forced_mass);\n  double acc = 0.0;"),
    "kept_full_blocks": ("if (mask[nb0 + b]) kept[r] += std::min<int64_t>(b * G + G, L) - b * G;",
                         "if (mask[nb0 + b]) kept[r] += G;"),
    "compact_global_block": ("if (!mask[nb0 + j / G]) continue;", "if (!mask[(s0 + j) / G]) continue;"),
    "positions_not_moved": ("if (positions) positions_out[dst] = positions[s0 + j];",
                            "if (positions) positions_out[dst] = positions[j];"),
    "history_cumulative": ("entries[2 * r + 1] = cu_out[r + 1] - cu_out[r];",
                           "entries[2 * r + 1] = cu_out[r + 1];"),
    "history_layer_dropped": ("entries[2 * r] = layer_id;", "entries[2 * r] = 0;"),
}


@pytest.fixture(scope="module")
def mutants():
    src = open(CX.SOURCE, encoding="utf-8").read()
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    libs = {}
    for name, (old, new) in CXX_MUTATIONS.items():
        assert src.count(old) == 1, f"mutation anchor not unique: {name}"
        path = os.path.join(tmp, f"{name}.cpp")
        with open(path, "w", encoding="utf-8") as f:
            f.write(src.replace(old, new))
        libs[name] = CX.build(path, os.path.join(tmp, f"lib{name}.so"))
    yield libs
    shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(CXX_MUTATIONS))
def test_cxx_mutation_is_caught(name, mutants, monkeypatch):
    monkeypatch.setattr(PINS, "O", CX.module(CX.load(mutants[name])))
    for check in PINS.ALL_CHECKS:
        try:
            check()
        except Exception:  # an assertion or a crash both count as caught
            return
    pytest.fail(f"no pin rejects C++ mutation {name}")
