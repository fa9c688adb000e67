"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
at least one pin of ``test_oracle_pins`` fails for each of them.  This shows the
pins constrain every part of the oracle: layout indexing, grouping, masking,
scale, the softmax and the weighted sum."""

import inspect
import os
import subprocess

import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

MUTATIONS = {
    "k_layout_token_major": (
        "return (((b * sh.Hkv + g) * (sh.D / 8) + d / 8) * sh.B + o) * 8 + d % 8;",
        "return (((b * sh.Hkv + g) * sh.B + o) * (sh.D / 8) + d / 8) * 8 + d % 8;"),
    "v_layout_dim_minor": (
        "return (((b * sh.Hkv + g) * (sh.B / bt) + o / bt) * sh.D + d) * bt + o % bt;",
        "return ((b * sh.Hkv + g) * sh.B + o) * sh.D + d;"),
    "group_by_modulo": ("h / G, lens[s],", "h % sh.Hkv, lens[s],"),
    "drop_last_token": ("for (int t = 0; t < L; ++t) {\n    const int j",
                        "for (int t = 0; t < L - (L > 1); ++t) {\n    const int j"),
    "wrong_slot": ("const int o = t % sh.B;", "const int o = (t + 1) % sh.B;"),
    "wrong_block": ("const int j = t / sh.B;", "const int j = (t / sh.B) ^ (t >= sh.B);"),
    "no_scale": ("    x[t] = scale * dot;", "    x[t] = dot;"),
    "scale_twice": ("    x[t] = scale * dot;", "    x[t] = scale * scale * dot * 8;"),
    "unnormalised": ("x[t] = x[t] / z;", "x[t] = x[t] / (z + Acc(1e-3));"),
    "value_from_key_slot": ("kv.v(sh, blk[t], g, t % sh.B, d)",
                            "kv.v(sh, blk[t], g, (t + 1) % sh.B, d)"),
    "fp8_subnormal_exponent": ("v = std::ldexp(static_cast<float>(m), -9);",
                               "v = std::ldexp(static_cast<float>(m), -10);"),
    "fp8_exponent_bias": ("v = std::ldexp(static_cast<float>(8 + m), e - 10);",
                          "v = std::ldexp(static_cast<float>(8 + m), e - 9);"),
    "fp8_k_layout_token_major": (
        "return (((b * sh.Hkv + g) * (sh.D / 16) + d / 16) * sh.B + o) * 16 + d % 16;",
        "return (((b * sh.Hkv + g) * sh.B + o) * (sh.D / 16) + d / 16) * 16 + d % 16;"),
    "fp8_v_layout_swapped": (
        "(sh.B / 4) + o / 4) * (sh.D / 16) + d / 16) * 4 + o % 4;",
        "(sh.D / 16) + d / 16) * (sh.B / 4) + o / 4) * 4 + o % 4;"),
    "fp8_encode_ties_away": ("int m = static_cast<int>(std::nearbyint((2.0 * f - 1.0) * 8.0));",
                             "int m = static_cast<int>(std::round((2.0 * f - 1.0) * 8.0));"),
    "fp8_encode_bias": ("return sign | static_cast<uint8_t>(((exp + 7) << 3) | m);",
                        "return sign | static_cast<uint8_t>(((exp + 8) << 3) | m);"),
    "fp8_encode_no_saturation": ("  if (a >= 448.0) return sign | 0x7E;\n", ""),
    "fp8_append_scale_multiplied": ("e4m3_from_float(bf16_bits_to_float(k_new[src]) / k_scale);",
                                    "e4m3_from_float(bf16_bits_to_float(k_new[src]) * k_scale);"),
    "fp8_v_scale_dropped": ("return e4m3_to_float(vp[v8_index(sh, b, g, o, d)]) * v_scale;",
                            "return e4m3_to_float(vp[v8_index(sh, b, g, o, d)]);"),
    "append_wrong_offset": ("k_pool[k_index(sh, b, g, o, d)] = k_new[src];",
                            "k_pool[k_index(sh, b, g, (o + 1) % block_size, d)] = k_new[src];"),
    "fp8_append_wrong_offset": ("v_pool[v8_index(sh, b, g, o, d)] = e4m3_from_float(",
                                "v_pool[v8_index(sh, b, g, (o + 1) % block_size, d)] = e4m3_from_float("),
    "causal_off_by_one": ("h / G, p + 1, scale, orow, nullptr);", "h / G, p, scale, orow, nullptr);"),
    "q_head_offset": ("q + (static_cast<int64_t>(s) * sh.Hq + h) * sh.D",
                      "q + (static_cast<int64_t>(s) * sh.Hq + h / G) * sh.D"),
}


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or "oracle_lib" not in inspect.signature(fn).parameters:
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argname, values = params[0].args
            for v in values:
                calls.append((name, fn, {argname: v}))
        else:
            calls.append((name, fn, {}))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(tmp_path, mutation):
    old, new = MUTATIONS[mutation]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % mutation
    path = tmp_path / "oracle_mut.cpp"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-fopenmp", "-fPIC", "-shared", str(path), "-o",
                    str(lib)], check=True)
    variant = oracle.Variant(str(lib))
    failed = []
    for name, fn, kwargs in _pin_calls():
        try:
            fn(oracle_lib=variant, **kwargs)
        except (Exception, pytest.fail.Exception):  # the pin caught it
            failed.append(name)
    assert failed, "no pin caught the planted mistake %r" % mutation
