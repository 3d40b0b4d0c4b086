"""Planted mistakes: the oracle's pins must reject a wrong oracle (CPU only).

Each case copies oracle/ep_oracle.c, or oracle/__init__.py for the scale
layouts, packing, capacity and decode glue written in Python, and plants one
plausible mistake by a textual substitution: a wrong tie rule, an off-by-one
exponent, a dropped weight, a sign error, a transposed index, another
accumulation order.  A C copy is compiled with the oracle's own build flags
into a temporary library and the oracle package is pointed at it; a Python
copy is executed as a module and handed to the pins in place of the package.
The pins of tests/test_oracle_*.py then run until one fails.  A mistake that
no pin notices fails this test.  The committed sources are never modified,
and the baseline cases run every pin against unmodified copies handled the
same way, so a harness that always fails would be caught too.
"""
import os
import types

import pytest

import oracle
from oracle import build as oracle_build
import test_oracle_backward as tb
import test_oracle_combine as tc
import test_oracle_dispatch as td
import test_oracle_fp8 as tf
import test_oracle_layout as tl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# the pins, cheapest first (a planted mistake usually fails one of the first)
PINS = [
    ("layout golden", lambda: tl.test_golden_hand_worked(GOLDEN)),
    ("combine golden", lambda: tc.test_golden_hand_worked(GOLDEN)),
    ("fp8 golden", lambda: tf.test_golden_codes_and_scales(GOLDEN)),
    ("backward golden", lambda: tb.test_golden_hand_worked(GOLDEN)),
    ("layout empty", tl.test_empty_routing),
    ("layout brute force", tl.test_brute_force_all_tiny_routings),
    ("layout out of range", tl.test_brute_force_out_of_range_ids),
    ("layout skew", tl.test_skew_all_slots_one_expert),
    ("bf16 rounding vs torch", tc.test_bf16_rounding_matches_torch),
    ("bf16 NaN", tc.test_nan_rounds_to_the_quiet_nan_with_its_sign),
    ("fma chain order", tc.test_fp32_fma_chain_in_ascending_slot_order),
    ("gathered masked", tc.test_gathered_combine_skips_masked_slots),
    ("combine closed form", tc.test_tiny_scaled_experts_closed_form),
    ("combine single slot", tc.test_single_slot_weight_one_is_copy_and_zero_weight_is_zero),
    ("combine identity", lambda: tc.test_identity_experts_return_x("tiny")),
    ("dispatch bf16 closed form", td.test_bf16_closed_form_and_padding_untouched),
    ("dispatch fp8 vs torch", td.test_fp8_rows_match_torch_cast),
    ("fp8 midpoints", tf.test_encode_midpoints_and_signed_zero),
    ("fp8 scale closed form", tf.test_scale_exponent_closed_form),
    ("fp8 dequant exact", tf.test_dequant_is_exact),
    ("fp8 roundtrip", tf.test_quantize_roundtrip_on_e4m3_grid),
    ("fp8 error bound", tf.test_quantize_row_error_bound_and_scale_rule),
    ("fp8 encode vs torch", lambda: tf.test_encode_matches_torch_cast_all_bf16(0)),
    ("fp8 encode vs torch, smallest scale", lambda: tf.test_encode_matches_torch_cast_all_bf16(-127)),
    ("fp8 encode vs search", lambda: tf.test_encode_matches_nearest_search_all_bf16(0)),
    ("f32 scale vs torch", tf.test_f32scale_quantize_matches_torch),
    ("f32 dequant bound", tf.test_f32scale_dequant_and_error_bound),
    ("pow2 closed form", tf.test_pow2_scale_closed_form_and_codes),
    ("MN-major views", tf.test_mn_major_layouts_by_memory_view),
    ("scaled dispatch and cast back", tf.test_scaled_dispatch_untouched_rows_and_cast_back),
    ("combine backward vs numpy", lambda: tb.test_combine_backward_against_numpy("tiny", None)),
    ("dispatch backward vs numpy", lambda: tb.test_dispatch_backward_against_numpy("decode", 128)),
    ("adjoint identities", lambda: tb.test_adjoint_identities("tiny", None)),
    ("layout vs numpy, tiny", lambda: tl.test_configs_against_numpy("tiny")),
    ("layout vs numpy, decode", lambda: tl.test_configs_against_numpy("decode")),
    ("combine float64 bound, tiny", lambda: tc.test_against_float64_within_summation_bound("tiny")),
    ("combine float64 bound, decode", lambda: tc.test_against_float64_within_summation_bound("decode")),
]

# (what the mistake is, source text, planted text); each source text occurs
# exactly once in oracle/ep_oracle.c
MUTANTS = [
    ("bf16 rounding ties up instead of to even",
     "up = (int)(below & 1u);", "up = 1;"),
    ("bf16 rounding truncates NaN (low-payload NaN becomes infinity)",
     "return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);", "return (uint16_t)(u >> 16);"),
    ("e4m3 encoding ties up instead of to the even code",
     "(dhi == dlo && ((lo + 1) % 2 == 0))", "(dhi == dlo)"),
    ("e4m3 encoding saturates to the NaN code",
     "        return (uint8_t)(sign | 0x7E);", "        return (uint8_t)(sign | 0x7F);"),
    ("e4m3 subnormal step 2^-10",
     "return ldexp((double)m, -9);", "return ldexp((double)m, -10);"),
    ("e4m3 exponent bias 8",
     "return ldexp(1.0 + (double)m / 8.0, ef - 7);", "return ldexp(1.0 + (double)m / 8.0, ef - 8);"),
    ("UE8M0 exponent against 256 instead of 448",
     "if ((double)amax <= ldexp(448.0, e))", "if ((double)amax <= ldexp(256.0, e))"),
    ("UE8M0 exponent with a strict comparison",
     "if ((double)amax <= ldexp(448.0, e))", "if ((double)amax < ldexp(448.0, e))"),
    ("quantisation scales by 2^e instead of 2^-e",
     "q[g * 128 + c] = eo_e4m3_encode(ldexp(v, -e));", "q[g * 128 + c] = eo_e4m3_encode(ldexp(v, e));"),
    ("UE8M0 byte with bias 128",
     "scales[g] = (uint8_t)(e + 127);", "scales[g] = (uint8_t)(e + 128);"),
    ("amax over half of the group",
     "        float amax = 0.0f;\n        for (int c = 0; c < 128; ++c) {\n"
     "            float a = fabsf(eo_bf16_to_f32(x[g * 128 + c]));\n"
     "            if (a > amax)                /* NaN never compares greater */\n"
     "                amax = a;\n        }\n        int e",
     "        float amax = 0.0f;\n        for (int c = 0; c < 64; ++c) {\n"
     "            float a = fabsf(eo_bf16_to_f32(x[g * 128 + c]));\n"
     "            if (a > amax)                /* NaN never compares greater */\n"
     "                amax = a;\n        }\n        int e"),
    ("dequantisation drops the sign",
     "        if (b & 0x80)\n            v = -v;\n        out[c] = eo_f32_to_bf16((float)ldexp(v, e));",
     "        out[c] = eo_f32_to_bf16((float)ldexp(v, e));"),
    ("tiles per expert rounded down",
     "int32_t tiles = (counts[e] + BM - 1) / BM;", "int32_t tiles = counts[e] / BM;"),
    ("every tile's arrival target is BLOCK_M",
     "tile_target[offsets[e] + j] = left < BM ? left : BM;", "tile_target[offsets[e] + j] = BM;"),
    ("receive token taken as the slot's k",
     "recv_token[next] = (int32_t)(s / K);", "recv_token[next] = (int32_t)(s % K);"),
    ("expert blocks filled in descending slot order",
     "        for (int64_t s = 0; s < S; ++s) {\n            if (idx[s] != e)",
     "        for (int64_t s = S - 1; s >= 0; --s) {\n            if (idx[s] != e)"),
    ("out-of-range expert ids not flagged",
     "            *error |= 1;", "            *error |= 0;"),
    ("combine drops the routing weight",
     "acc = fmaf(w[t * K + k], eo_bf16_to_f32(expert_out[(int64_t)r * H + c]), acc);",
     "acc = fmaf(1.0f, eo_bf16_to_f32(expert_out[(int64_t)r * H + c]), acc);"),
    ("combine uses the first slot's weight for every slot",
     "acc = fmaf(w[t * K + k], eo_bf16_to_f32(expert_out[(int64_t)r * H + c]), acc);",
     "acc = fmaf(w[t * K], eo_bf16_to_f32(expert_out[(int64_t)r * H + c]), acc);"),
    ("combine multiplies, then adds (two roundings)",
     "acc = fmaf(w[t * K + k], eo_bf16_to_f32(expert_out[(int64_t)r * H + c]), acc);",
     "acc = w[t * K + k] * eo_bf16_to_f32(expert_out[(int64_t)r * H + c]) + acc;"),
    ("combine accumulates the slots in descending order",
     "            for (int32_t k = 0; k < K; ++k) {\n                int32_t r = slot_to_row[t * K + k];\n"
     "                if (r < 0)\n                    continue;\n                acc = fmaf(",
     "            for (int32_t k = K - 1; k >= 0; --k) {\n                int32_t r = slot_to_row[t * K + k];\n"
     "                if (r < 0)\n                    continue;\n                acc = fmaf("),
    ("gathered combine includes masked slots",
     "                if (!valid[i * K + k])\n                    continue;\n", ""),
    ("combine backward's gradient rows miss the weight",
     "float p = w[t * K + k] * g;", "float p = g;"),
    ("combine backward's weight gradient has the wrong sign",
     "dot += (double)g * (double)o;", "dot -= (double)g * (double)o;"),
    ("combine backward's weight gradient uses grad_y for the expert row",
     "dot += (double)g * (double)o;", "dot += (double)g * (double)g;"),
    ("dispatch backward keeps only the last slot",
     "acc = acc + eo_bf16_to_f32(grad_pool[(int64_t)r * H + c]);",
     "acc = eo_bf16_to_f32(grad_pool[(int64_t)r * H + c]);"),
    ("float32 scale inverted",
     "float s = a / 448.0f;", "float s = 448.0f / a;"),
    ("float32 scale without the floor on amax",
     "const float floor_amax = 448.0f * 0x1p-126f;", "const float floor_amax = 0.0f;"),
    ("float32 dequantisation divides by the scale",
     "float p = v * scales[c / 128];", "float p = v / scales[c / 128];"),
    ("bf16 dispatch copies the channels reversed",
     "pool[r * H + c] = x[(int64_t)t * H + c];", "pool[r * H + c] = x[(int64_t)t * H + (H - 1 - c)];"),
    ("FP8 dispatch indexes the scales by token instead of pool row",
     "eo_quantize_row(x + (int64_t)t * H, H, pool + r * H, scales + r * (H / 128));",
     "eo_quantize_row(x + (int64_t)t * H, H, pool + r * H, scales + (int64_t)t * (H / 128));"),
]


# the same for the Python half of the oracle (oracle/__init__.py)
PY_MUTANTS = [
    ("capacity without the -1",
     "return tokens * top_k + num_experts * (block_m - 1)", "return tokens * top_k + num_experts * block_m"),
    ("power-of-two scale with bias 128",
     "e = scale_bytes.astype(np.int64) - 127", "e = scale_bytes.astype(np.int64) - 128"),
    ("packed UE8M0 words in the wrong byte order",
     "word |= int(scales[r, g]) << (8 * j)", "word |= int(scales[r, g]) << (8 * (3 - j))"),
    ("packed words per row rounded down",
     "return (groups + 3) // 4", "return groups // 4 if groups >= 4 else 1"),
    ("MN-major float32 groups reversed",
     "out[:, r] = scales[r, :]", "out[:, r] = scales[r, ::-1]"),
    ("MN-major unpacking in the wrong byte order",
     "(int(mn[g // 4, r]) >> (8 * (g % 4)))", "(int(mn[g // 4, r]) >> (8 * (3 - g % 4)))"),
    ("power-of-two flavour stores the UE8M0 byte",
     "rm[r] = b if kind == SCALE_UE8M0 else pow2_scales_from_ue8m0(b)", "rm[r] = b"),
    ("scaled dispatch overwrites the padding rows' scales",
     "scales[real] = rm[real]", "scales[:] = rm"),
    ("cast back decodes power-of-two floats as UE8M0 bytes",
     "    if kind == SCALE_UE8M0:\n        return dequant_rows(q, rm)",
     "    if kind != SCALE_F32:\n        return dequant_rows(q, rm)"),
    ("float32 dequantisation takes row 0's scales for every row",
     "lib.eo_dequant_row_f32scale(_p(q[i]), _p(scales[i]), H, _p(out[i]))",
     "lib.eo_dequant_row_f32scale(_p(q[i]), _p(scales[0]), H, _p(out[i]))"),
    ("UE8M0 dequantisation takes row 0's scales for every row",
     "lib.eo_dequant_row(_p(q[i]), _p(scales[i]), H, _p(out[i]))",
     "lib.eo_dequant_row(_p(q[i]), _p(scales[0]), H, _p(out[i]))"),
]

PIN_MODULES = [tl, tc, td, tf, tb]
PY_SOURCE = os.path.join(os.path.dirname(oracle_build.SRC), "__init__.py")


def _source() -> str:
    with open(oracle_build.SRC) as f:
        return f.read()


def _first_failing_pin(text: str, tmp_path, monkeypatch):
    """Build `text` as the oracle library and run the pins; the name of the
    first pin that fails, or None."""
    src = tmp_path / "ep_oracle_variant.c"
    src.write_text(text)
    lib = oracle_build.build(src=str(src), out=str(tmp_path / "libep_oracle_variant.so"))
    monkeypatch.setattr(oracle, "_LIB_PATH", lib)
    monkeypatch.setattr(oracle, "_lib", None)
    return _run_pins()


def _run_pins():
    for name, pin in PINS:
        try:
            pin()
        except Exception:                   # an assertion, or an error the mistake causes
            return name
    return None


def _first_failing_pin_py(text: str, monkeypatch):
    """Execute `text` as the oracle's Python half (loading the real C
    library) and hand it to the pins in place of the package."""
    oracle._load()                          # builds the C library if it is missing
    mod = types.ModuleType("oracle_variant")
    mod.__file__ = PY_SOURCE
    exec(compile(text, PY_SOURCE, "exec"), mod.__dict__)
    for m in PIN_MODULES:
        monkeypatch.setattr(m, "oracle", mod)
    return _run_pins()


def test_unmodified_copy_passes_every_pin(tmp_path, monkeypatch):
    assert _first_failing_pin(_source(), tmp_path, monkeypatch) is None


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(what, old, new, tmp_path, monkeypatch):
    text = _source()
    assert text.count(old) == 1, "the planted text must replace exactly one place"
    caught_by = _first_failing_pin(text.replace(old, new), tmp_path, monkeypatch)
    assert caught_by is not None, f"no pin notices: {what}"


def test_unmodified_python_copy_passes_every_pin(monkeypatch):
    with open(PY_SOURCE) as f:
        assert _first_failing_pin_py(f.read(), monkeypatch) is None


@pytest.mark.parametrize("what,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_python_mistake_is_caught(what, old, new, monkeypatch):
    with open(PY_SOURCE) as f:
        text = f.read()
    assert text.count(old) == 1, "the planted text must replace exactly one place"
    assert _first_failing_pin_py(text.replace(old, new), monkeypatch) is not None, f"no pin notices: {what}"
