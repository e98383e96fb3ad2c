"""Planted mistakes in a copy of the oracle's source must each fail a pin.

Each entry patches one snippet of oracle/attn_oracle.c (which must occur
exactly the stated number of times, so a change to the oracle that moves a
snippet breaks this test loudly), builds the patched copy in a temporary
directory with the same compiler flags, and runs the whole pin suite on it.
The oracle itself is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

# name: [(original snippet, replacement, expected occurrences)]
MUTANTS = {
    "scale_dropped": [("return J->scale * acc + bias;", "return acc + bias;", 1)],
    "scale_divides": [("return J->scale * acc + bias;", "return acc / J->scale + bias;", 1)],
    "self_not_visible": [("return j <= p;", "return j < p;", 1)],
    "sees_next_key": [("return j <= p;", "return j <= p + 1;", 1)],
    "top_left_alignment": [("const int p = (L - n) + i;", "const int p = i;", 1)],
    "query_count_ignores_length": [("const int n = Sq < L ? Sq : L;", "const int n = Sq;", 1)],
    "padding_ignored": [("if (j >= L) return 0;", "if (j >= J->Skv) return 0;", 1)],
    "pad_rows_computed": [("if (i >= n) return;", "", 1)],
    "transposed_key": [("kbase + (size_t)j * J->d + c", "kbase + (size_t)c * J->Skv + j", 1)],
    "last_feature_dropped": [("for (int c = 0; c < J->d; ++c)", "for (int c = 0; c < J->d - 1; ++c)", 1)],
    "value_row_from_query": [("vbase + (size_t)j * dv + c", "vbase + (size_t)i * dv + c", 1)],
    "value_stride_uses_dk": [("* (size_t)Skv * dv;", "* (size_t)Skv * J->d;", 1),
                             ("vbase + (size_t)j * dv + c", "vbase + (size_t)j * J->d + c", 1)],
    "not_normalised": [("exp(s[j] - m) / l;", "exp(s[j] - m);", 1)],
    "max_not_subtracted": [("exp(s[j] - m)", "exp(s[j])", 2)],
    "max_not_tracked": [("if (s[j] > m) m = s[j];", "", 1)],
    "mask_after_softmax": [("if (key_visible(J, b, h, i, j, p, L)) l += exp(s[j] - m);",
                            "l += exp(score(J, qrow, kbase, j, 0.0) - m);", 1)],
    "allowed_mask_ignored": [("if (J->mask && !J->mask[", "if (0 && !J->mask[", 1)],
    "allowed_mask_inverted": [("if (J->mask && !J->mask[", "if (J->mask && J->mask[", 1)],
    "allowed_mask_row_reversed": [("(long long)i * J->Skv + j]", "(long long)(J->Sq - 1 - i) * J->Skv + j]", 1)],
    "allowed_mask_batch_ignored": [("[b * J->mask_sb + h * J->mask_sh", "[h * J->mask_sh", 1)],
    "allowed_mask_head_ignored": [("[b * J->mask_sb + h * J->mask_sh", "[b * J->mask_sb", 1)],
    "bias_ignored": [("return J->scale * acc + bias;", "return J->scale * acc;", 1)],
    "bias_scaled": [("return J->scale * acc + bias;", "return J->scale * (acc + bias);", 1)],
    "bias_subtracted": [("return J->scale * acc + bias;", "return J->scale * acc - bias;", 1)],
    "bias_row_reversed": [("h * J->bias_sh + (long long)i * J->Skv + j", "h * J->bias_sh + (long long)(J->Sq - 1 - i) * J->Skv + j", 1)],
    "bias_batch_ignored": [("(size_t)(b * J->bias_sb + h * J->bias_sh", "(size_t)(h * J->bias_sh", 1)],
    "bias_head_ignored": [("(size_t)(b * J->bias_sb + h * J->bias_sh", "(size_t)(b * J->bias_sb", 1)],
    "neg_inf_bias_kept_visible": [("if (bias_at(J, b, h, i, j) == -INFINITY) return 0;", "", 1)],
    "kv_head_modulo": [("const int hk = h / (J->H / J->Hkv);", "const int hk = h % J->Hkv;", 1)],
    "kv_base_strides_query_heads": [("((size_t)b * J->Hkv + hk) * (size_t)Skv * J->d;",
                                     "((size_t)b * J->H + hk) * (size_t)Skv * J->d;", 1)],
    "bf16_widening_off": [("[idx] << 16;", "[idx] << 16 | 0x8000u;", 1)],
    "f32_read_as_rounded": [("return (double)((const float*)base)[idx];",
                             "return (double)(float)(((const float*)base)[idx] * 1.0001f);", 1)],
}


def _build(tmp_path, name, patches):
    text = open(SRC).read()
    for old, new, count in patches:
        assert text.count(old) == count, f"{name}: snippet {old!r} occurs {text.count(old)} times"
        text = text.replace(old, new)
    src = tmp_path / f"mut_{name}.c"
    src.write_text(text)
    return oracle.compile_oracle(str(src), str(tmp_path / f"libmut_{name}.so"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    lib = oracle.load(_build(tmp_path, name, MUTANTS[name]))

    def attn(*a, **kw):
        kw["lib"] = lib
        return oracle.attention(*a, **kw)

    failed = oracle_pins.failing_pins(attn)
    assert failed, f"planted mistake {name!r} passed every pin"


def test_unpatched_copy_passes(tmp_path):
    lib = oracle.load(_build(tmp_path, "none", []))

    def attn(*a, **kw):
        kw["lib"] = lib
        return oracle.attention(*a, **kw)

    assert oracle_pins.failing_pins(attn) == []
