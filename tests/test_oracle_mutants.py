"""The oracle's pins have teeth: each planted mistake must fail at least one.

Every mutant is a copy of oracle/tropical_oracle.c with one textual edit
(a dropped term, a wrong comparison, sign, stride, index or element),
compiled into a temporary library and run through tests/pins.py; the
Python planner of pairwise steps and trees (oracle/contract.py) gets the
same treatment, its mutated copy standing in for the module while the pins
run.  Nothing here touches a GPU.  If an edit's source text is no longer
found, the test fails so that the list is kept in step with the oracle.
"""
import os
import sys
import types

import pytest

import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tropical_oracle.c")
PY_SRC = os.path.join(ROOT, "oracle", "contract.py")

MUTANTS = [
    ("drop_last_k_f32",
     "float best = zero_f32(sr);\n        for (int64_t kk = 0; kk < k; ++kk)",
     "float best = zero_f32(sr);\n        for (int64_t kk = 0; kk < k - 1; ++kk)"),
    ("drop_last_k_i32",
     "int32_t best = zero_i32(sr);\n        for (int64_t kk = 0; kk < k; ++kk)",
     "int32_t best = zero_i32(sr);\n        for (int64_t kk = 0; kk < k - 1; ++kk)"),
    ("ties_to_last_max_f32",
     "static int better_f32(int sr, float t, float best)\n{\n    if (sr == ORC_MIN_PLUS) return t < best;\n    return t > best;",
     "static int better_f32(int sr, float t, float best)\n{\n    if (sr == ORC_MIN_PLUS) return t < best;\n    return t >= best;"),
    ("ties_to_last_min_i32",
     "static int better_i32(int sr, int32_t t, int32_t best)\n{\n    if (sr == ORC_MIN_PLUS) return t < best;",
     "static int better_i32(int sr, int32_t t, int32_t best)\n{\n    if (sr == ORC_MIN_PLUS) return t <= best;"),
    ("min_plus_uses_max",
     "static int better_f32(int sr, float t, float best)\n{\n    if (sr == ORC_MIN_PLUS) return t < best;",
     "static int better_f32(int sr, float t, float best)\n{\n    if (sr == ORC_MIN_PLUS) return t > best;"),
    ("transposed_A_f32",
     "float x = a[b * sA[2] + i * sA[0] + kk * sA[1]];",
     "float x = a[b * sA[2] + i * sA[1] + kk * sA[0]];"),
    ("transposed_B_i32",
     "int32_t y = bm[b * sB[2] + kk * sB[0] + j * sB[1]];",
     "int32_t y = bm[b * sB[2] + kk * sB[1] + j * sB[0]];"),
    ("batch_stride_ignored",
     "float y = bm[b * sB[2] + kk * sB[0] + j * sB[1]];",
     "float y = bm[kk * sB[0] + j * sB[1]];"),
    ("plus_is_minus", "    return a + b;\n}", "    return a - b;\n}"),
    ("max_mul_adds", "if (sr == ORC_MAX_MUL) return a * b;", "if (sr == ORC_MAX_MUL) return a + b;"),
    ("wrapping_i32", "    if (s > INT32_MAX) return INT32_MAX;\n", ""),
    ("maxmul_i32_adds", "(sr == ORC_MAX_MUL) ? (int64_t)a * (int64_t)b", "(sr == ORC_MAX_MUL) ? (int64_t)a + (int64_t)b"),
    ("maxmul_i32_zero_negative", "    if (sr == ORC_MAX_MUL) return 0;\n", ""),
    ("maxmul_i32_wraps_low", "    if (s < INT32_MIN) return INT32_MIN;\n", ""),
    ("max_plus_zero_finite", "if (sr == ORC_MAX_PLUS) return -INFINITY;",
     "if (sr == ORC_MAX_PLUS) return -1e30f;"),
    ("min_plus_zero_i32_off", "return sr == ORC_MIN_PLUS ? ORC_I32_INF : -ORC_I32_INF;",
     "return sr == ORC_MIN_PLUS ? ORC_I32_INF - 1 : -ORC_I32_INF;"),
    ("argmax_off_by_one",
     "best = t;\n                arg = (int32_t)kk;\n            }\n        }\n        *(float*)cval = best;",
     "best = t;\n                arg = (int32_t)kk + 1;\n            }\n        }\n        *(float*)cval = best;"),
    ("permute_unpermuted_strides", "off += digit * in_strides[perm[d]];", "off += digit * in_strides[d];"),
    ("permute_column_major_decode",
     "        for (int d = ndim - 1; d >= 0; --d) {\n            int64_t digit = rem % out_shape[d];",
     "        for (int d = 0; d < ndim; ++d) {\n            int64_t digit = rem % out_shape[d];"),
    ("diag_stride_not_summed", "str[found] += in_strides[a];", "str[found] = in_strides[a];"),
    ("trace_last_wins", "                if (better_f32(sr, t, best)) {\n                    best = t;\n                    win",
     "                if (1) {\n                    best = t;\n                    win"),
    ("brute_argmax_shifted", "bestf = t;\n                    arg = (int32_t)p;",
     "bestf = t;\n                    arg = (int32_t)(p > 0 ? p - 1 : 0);"),
    ("reduce_winner_not_kept_f32", "best = t;\n                    win = (int32_t)q;", "best = t;"),
    ("reduce_winner_off_by_one", "win = (int32_t)q;", "win = (int32_t)q + 1;"),
    ("points_swap_ij",
     "pts[3 * p], pts[3 * p + 1], pts[3 * p + 2]", "pts[3 * p], pts[3 * p + 2], pts[3 * p + 1]"),
    # backward (winner routing)
    ("bwd_maxmul_no_factor_dA", "if (mul) v = v * B[b * sB[2] + ks * sB[0] + j * sB[1]];", ""),
    ("bwd_maxmul_factor_wrong_k_dB", "if (mul) v = v * A[b * sA[2] + i * sA[0] + ks * sA[1]];",
     "if (mul) v = v * A[b * sA[2] + i * sA[0] + 0 * sA[1]];"),
    ("bwd_dB_routed_to_next_k", "float* d = &dB[b * sdB[2] + ks * sdB[0] + j * sdB[1]];",
     "float* d = &dB[b * sdB[2] + ((ks + 1) % k) * sdB[0] + j * sdB[1]];"),
    ("bwd_dA_drops_last_j", "for (int64_t j = 0; j < n; ++j) {\n                int64_t c",
     "for (int64_t j = 0; j < n - 1; ++j) {\n                int64_t c"),
    ("bwd_dA_starts_at_one", "dA[b * sdA[2] + i * sdA[0] + kk * sdA[1]] = 0.0f;",
     "dA[b * sdA[2] + i * sdA[0] + kk * sdA[1]] = 1.0f;"),
    ("bwd_gradient_ignored", "float v = G[c];", "float v = 1.0f;"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, find, repl):
    import oracle
    from oracle import build as obuild
    assert source.count(find) >= 1, f"mutation {name}: source text not found"
    mutated = source.replace(find, repl, 1)
    src = tmp_path / f"{name}.c"
    src.write_text(mutated)
    lib = obuild.build(str(src), str(tmp_path / f"lib{name}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, oracle.OracleError, ValueError, IndexError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"mutant {name} passed every pin"


PY_MUTANTS = [
    ("pair_contracted_in_b_order",
     "contracted = [c for c in _unique(la) if c in lb and c not in out]",
     "contracted = [c for c in _unique(lb) if c in la and c not in out]"),
    ("pair_output_not_permuted", "C = orc.permute(C2.reshape(shape), perm)", "C = C2.reshape(shape)"),
    ("pair_argmax_permuted_differently", "I = orc.permute(I2.reshape(shape), perm) if argmax else None",
     "I = orc.permute(I2.reshape(shape), perm[::-1]) if argmax else None"),
    ("route_drops_b_winner", "full = I2.astype(np.int64) * (ra * rb) + wa * rb + wb",
     "full = I2.astype(np.int64) * (ra * rb) + wa * rb"),
    ("route_b_before_a", "full = I2.astype(np.int64) * (ra * rb) + wa * rb + wb",
     "full = I2.astype(np.int64) * (ra * rb) + wb * ra + wa"),
    ("route_winners_at_k0", "wa = WA.reshape(nb, m, k)[bi, ii, I2]", "wa = WA.reshape(nb, m, k)[bi, ii, 0 * I2]"),
    ("tree_rhs_is_lhs", "lb, B = slots[rhs]", "lb, B = slots[lhs]"),
    ("tree_returns_first_step", "return slots[-1][1], winners", "return slots[len(subs)][1], winners"),
    ("tree_result_keeps_lhs_subscript", "slots.append((out, C))", "slots.append((la, C))"),
    ("tree_argmax_flags_shifted", "argmax=flags[s])", "argmax=flags[s - 1])"),
]


@pytest.fixture(scope="module")
def py_source():
    with open(PY_SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,find,repl", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(monkeypatch, py_source, name, find, repl):
    import oracle
    assert py_source.count(find) >= 1, f"mutation {name}: source text not found"
    mod = types.ModuleType("oracle.contract")
    mod.__package__ = "oracle"
    mod.__file__ = PY_SRC
    exec(compile(py_source.replace(find, repl, 1), f"<{name}>", "exec"), mod.__dict__)
    monkeypatch.setitem(sys.modules, "oracle.contract", mod)
    orc = oracle.default()
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, oracle.OracleError, ValueError, IndexError, KeyError, TypeError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"mutant {name} passed every pin"
