"""Plant plausible mistakes in copies of the oracle (CPU only) and check that
the pin suite catches each one: a dropped term, a wrong sign or index, a
transposed operand, the wrong log base, a mask off by one.

The mutated copies are compiled into a temporary directory; oracle.c itself is
never modified.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "scale dropped": ("S[(size_t)i * tk + j] = scale * acc;", "S[(size_t)i * tk + j] = acc;"),
    "mask off by one": ("if (j > i + (tk - tq))", "if (j >= i + (tk - tq))"),
    "mask alignment top-left": ("if (j > i + (tk - tq))", "if (j > i)"),
    "exp sign": ("row[j] = exp(row[j] - m);", "row[j] = exp(m - row[j]);"),
    "max not subtracted in lse": ("lse[i] = m + log(l);", "lse[i] = log(l);"),
    "lse base 2": ("lse[i] = m + log(l);", "lse[i] = m + log2(l);"),
    "not normalised": ("o[c] = acc / l;", "o[c] = acc;"),
    "V columns reversed": ("acc += row[j] * V[(size_t)j * d + c];",
                           "acc += row[j] * V[(size_t)j * d + (d - 1 - c)];"),
    "K used for V": ("acc += row[j] * V[(size_t)j * d + c];",
                     "acc += row[j] * K[(size_t)j * d + c];"),
    "GQA interleaved": ("kvh = h / group;", "kvh = h % Hkv;"),
    "paged slot shifted": ("t % page_size) * D;", "(t + 1) % page_size) * D;"),
    "paged head ignored": ("((page * Hkv + kvh) * page_size", "((page * Hkv + 0) * page_size"),
    "merge weights swapped": ("const double ta = wa > 0.0 ? wa * o_a[r * D + c] : 0.0;",
                              "const double ta = wa > 0.0 ? wb * o_a[r * D + c] : 0.0;"),
    "merge lse without max": ("lse_out[r] = M + log(wa + wb);", "lse_out[r] = log(wa + wb);"),
    "bf16 widened as low half": ("<< 16;\n    float f;", ";\n    float f;"),
    "fallback lower bound dropped": ("if (m - phi > window || m - phi < -window)", "if (m - phi > window)"),
    "fallback score unscaled": ("const double s = scale * dot;", "const double s = dot;"),
    "fallback over the whole sequence": ("const int c1 = c0 + split_tokens < L ? c0 + split_tokens : L;",
                                         "const int c1 = L;"),
    "e4m3 exponent bias 8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                             "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3 subnormals flushed": ("v = ldexp((double)m / 8.0, -6);", "v = 0.0;"),
    "e4m3 subnormal exponent": ("v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    "e4m3 sign dropped": ("return sign ? -v : v;", "return v;"),
    "e4m3 no NaN code": ("if (e == 15 && m == 7)\n        return NAN;", ""),
    "fp8 key scale ignored": ("K[(size_t)t * D + c] = k_scale * oracle_e4m3_value",
                              "K[(size_t)t * D + c] = oracle_e4m3_value"),
    "paged prefill reads sequence 0's table": (
        "const int32_t *table = block_table + (size_t)b * max_pages;",
        "const int32_t *table = block_table + (size_t)0 * max_pages;"),
    "paged prefill causal flag dropped": (
        "attend_rows(Q, K, V, Tq, L, D, causal, scale, S, o + qbase, lse + (size_t)bh * Tq);",
        "attend_rows(Q, K, V, Tq, L, D, 0, scale, S, o + qbase, lse + (size_t)bh * Tq);"),
    "paged prefill queries of head 0": (
        "const size_t qbase = (size_t)bh * Tq * D;",
        "const size_t qbase = (size_t)(bh - h) * Tq * D;"),
    "paged prefill gathers the wrong kv head": (
        "const int b = (int)(bh / Hq), h = (int)(bh % Hq), kvh = h / group;\n        const int L = kv_lens[b];",
        "const int b = (int)(bh / Hq), h = (int)(bh % Hq), kvh = h % Hkv;\n        const int L = kv_lens[b];"),
    "flat gemm W read transposed": ("load_elem(w, dtype, (size_t)j * k + t)",
                                    "load_elem(w, dtype, (size_t)t * n + j)"),
    "flat gemm last k dropped": ("for (int t = 0; t < k; t++)\n            acc += load_elem(a",
                                 "for (int t = 0; t < k - 1; t++)\n            acc += load_elem(a"),
    "flat gemm rows of A swapped with columns": ("const int i = (int)(ij / n), j = (int)(ij % n);",
                                                 "const int j = (int)(ij / m), i = (int)(ij % m);"),
    "fp8 scales swapped": ("V[(size_t)t * D + c] = v_scale * oracle_e4m3_value",
                           "V[(size_t)t * D + c] = k_scale * oracle_e4m3_value"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, source, tmp_path):
    old, new = MUTATIONS[name]
    assert source.count(old) >= 1, f"mutation anchor for '{name}' not found"
    mutated = source.replace(old, new)
    src = tmp_path / "oracle_mut.c"
    src.write_text(mutated)
    lib_path = oracle.build(str(tmp_path / "liboracle_mut.so"), str(src))
    lib = oracle.load(lib_path)
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, RuntimeError, ValueError):
            failures.append(check.__name__)
    assert failures, f"no pin caught the planted mistake '{name}'"
