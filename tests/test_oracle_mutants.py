"""Plant plausible mistakes in copies of the CPU oracle and check that the pins
catch every one of them.

Each mutant is the oracle's C source with one textual change, compiled with
gcc into a temporary directory (the shipped oracle is untouched). A mutant
passes this test when at least one pin fails on it. All mutants keep every
memory access in bounds, so a failure is a wrong number, never a crash.
"""

import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    # causal mask aligned to the start of the context instead of its end
    "top_left_causal": ("const int64_t p = L - q + i;", "const int64_t p = i + (L - q) / 2;"),
    # a row does not see its own key
    "drops_own_key": ("const int64_t n = p - lo + 1;", "const int64_t n = p - lo;"),
    # window one key too wide
    "window_off_by_one": ("(p - W + 1 > 0 ? p - W + 1 : 0)", "(p - W > 0 ? p - W : 0)"),
    # query head mapped to KV head by modulo instead of by group
    "gqa_modulo": ("const int g = h / G;", "const int g = h % J->Hkv;"),
    # softmax scale dropped
    "no_sigma": ("s[t] = J->sigma * dot;", "s[t] = dot;"),
    # sink left out of the denominator
    "sink_dropped": ("double Z = (z == -INFINITY) ? 0.0 : exp(z - M);", "double Z = 0.0;"),
    # sink counted with the wrong sign
    "sink_sign": ("double Z = (z == -INFINITY) ? 0.0 : exp(z - M);",
                  "double Z = (z == -INFINITY) ? 0.0 : exp(-z - M);"),
    # V's FP8 scale not applied
    "v_scale_dropped": ("return pa_oracle_e4m3_to_double(pool[idx]) * (double)sc[slot];",
                        "return pa_oracle_e4m3_to_double(pool[idx]) * (is_v ? 1.0 : (double)sc[slot]);"),
    # K's scale used for V as well
    "k_scale_for_v": ("const float *sc = is_v ? J->v_scales : J->k_scales;",
                      "const float *sc = J->k_scales;"),
    # page read token-major instead of head-major (a transposed layout)
    "page_transposed": (
        "int64_t slot = ((int64_t)blk * J->Hkv + g) * PAGE_TOKENS + (j % PAGE_TOKENS);",
        "int64_t slot = ((int64_t)blk * PAGE_TOKENS + (j % PAGE_TOKENS)) * J->Hkv + g;"),
    # wrong query row offset for later sequences
    "query_offset": ("const int64_t row = J->q_off[b] + i;", "const int64_t row = b + i;"),
    # e4m3 exponent bias off by one
    "e4m3_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    # e4m3 subnormals scaled wrongly
    "e4m3_subnormal": ("v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    # denominator forgets the keys' exponentials
    "denominator_no_keys": ("      Z += e;\n", "      Z += e * 0.5;\n"),
    # value taken from K's pool
    "v_from_k": ("const uint16_t *pool = (const uint16_t *)(is_v ? J->v_pool : J->k_pool);",
                 "const uint16_t *pool = (const uint16_t *)J->k_pool;"),
    # bf16 widened from the wrong half
    "bf16_low_half": ("uint32_t w = ((uint32_t)bits) << 16;", "uint32_t w = ((uint32_t)bits) << 15;"),
    # append: new token written one slot later in its page
    "append_slot": ("const int slot = pos % PAGE_TOKENS;", "const int slot = (pos + 1) % PAGE_TOKENS;"),
    # append: the next block-table entry's page
    "append_page": ("const int64_t page = block_table[(int64_t)b * max_blocks + pos / PAGE_TOKENS];",
                    "const int64_t page = block_table[(int64_t)b * max_blocks + pos / PAGE_TOKENS + 1];"),
    # quantiser: scale with the wrong divisor
    "scale_divisor": ("amax / 448.0f", "amax / 447.0f"),
    # encoder: ties to the odd mantissa
    "ties_to_odd": ("(d == best_d && (c & 1) == 0 && (best & 1) == 1)",
                    "(d == best_d && (c & 1) == 1 && (best & 1) == 0)"),
    # encoder: sign dropped
    "encode_no_sign": ("(signbit(v) ? 0x80 : 0)", "0"),
    # append: V rows taken from the new K
    "append_v_from_k": ("const uint16_t *vr = v_new + ", "const uint16_t *vr = k_new + "),
    # verdict: a draft compared with the argmax of its own row
    "verdict_alignment": ("input_ids[t + 1 + n] == out_ids[t + n]", "input_ids[t + 1 + n] == out_ids[t + 1 + n]"),
    # verdict: ties go to the highest index
    "verdict_ties_high": ("        if (x > best) {\n          best = x;\n          arg = v;",
                          "        if (x >= best) {\n          best = x;\n          arg = v;"),
    # verdict: NaN wins
    "verdict_nan_wins": ("        if (x > best) {\n          best = x;\n          arg = v;",
                         "        if (!(x <= best)) {\n          best = x;\n          arg = v;"),
    # verdict: the next id is the last accepted draft instead of the target's token after it
    "verdict_next_off": ("next_ids[b] = out_ids[t + n];", "next_ids[b] = out_ids[t + (n > 0 ? n - 1 : 0)];"),
    # verdict: every matching draft counts, not only the leading run
    "verdict_all_matches": ("while (n < q - 1 && input_ids[t + 1 + n] == out_ids[t + n]) ++n;",
                            "for (int j = 0; j < q - 1; ++j) n += (input_ids[t + 1 + j] == out_ids[t + j]);"),

}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new))
    lib = str(tmp_path / f"lib{name}.so")
    oracle.compile_source(str(src), lib)
    orc = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches the {name} mutant"
    os.remove(lib)
