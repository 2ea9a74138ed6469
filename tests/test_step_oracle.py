"""The decode-step oracle against its pins, and planted mistakes in copies
of it that the pins must catch (the real module is never modified)."""
import importlib.util
import os

import numpy as np
import pytest

from oracle import decode_step
from tests import step_pins

SOURCE = decode_step.__file__

MUTANTS = {
    "rms_divides_by_dim_minus_one": ("np.sum(x * x, axis=1) / dim", "np.sum(x * x, axis=1) / (dim - 1)"),
    "rms_eps_outside_sqrt": ("1.0 / np.sqrt(ms + float(np.float32(eps)))",
                             "1.0 / np.sqrt(ms) + float(np.float32(eps))"),
    "rms_weight_dropped": ("x * inv[:, None] * w[None, :]", "x * inv[:, None]"),
    "rope_frequency_over_head_dim": ("theta)), -i / half)", "theta)), -i / head_dim)"),
    "rope_sign": ("a * c - b * s", "a * c + b * s"),
    "rope_interleaved_pairs": ("a, b = x[:, :half], x[:, half:]", "a, b = x[:, 0::2], x[:, 1::2]"),
    "attention_scale_dropped": ("scores = (k @ q[h]) * scale", "scores = (k @ q[h])"),
    "attention_kv_head_modulo": ("off = (h // kv_group) * head_dim", "off = (h % kv_group) * head_dim"),
    "attention_values_are_keys": ("out[h] = p @ v", "out[h] = p @ k"),
    "attention_whole_cache": ("[:seq]\n    vc = _f64(vc).reshape(-1, kv_width)[:seq]",
                              "\n    vc = _f64(vc).reshape(-1, kv_width)"),
    "silu_sign": ("np.exp(-g)", "np.exp(g)"),
    "add_subtracts": ("return _f64(x) + _f64(y)", "return _f64(x) - _f64(y)"),
    "append_wrong_row": ("kc[pos] = ", "kc[pos - 1] = "),
    "argmax_ties_high": ("(v == best and i < besti)", "(v == best and i > besti)"),
    "argmax_ties_last": ("if v > best or", "if v >= best or"),
    "step_silu_on_up": ('silu_hadamard(mv(L["wgate"], xn, hid, inter), mv(L["wup"], xn, hid, inter))',
                        'silu_hadamard(mv(L["wup"], xn, hid, inter), mv(L["wgate"], xn, hid, inter))'),
    "step_ffn_residual_dropped": ('x = _r32(add_inplace(x, mv(L["wdown"], h, inter, hid)))',
                                  'x = _r32(mv(L["wdown"], h, inter, hid))'),
    "step_attn_residual_dropped": ('x = _r32(add_inplace(x, mv(L["wo"], a, qw, hid)))',
                                   'x = _r32(mv(L["wo"], a, qw, hid))'),
    "step_kv_group": ("pos + 1, kvw, hd, nh, nh // nkv)", "pos + 1, kvw, hd, nh, nkv)"),
    "step_rope_next_position": ("k = _r32(rope_rows(k, hd, pos, theta))", "k = _r32(rope_rows(k, hd, pos + 1, theta))"),
    "step_attention_skips_current": ("kc[l], vc[l], pos + 1,", "kc[l], vc[l], max(pos, 1),"),
    "step_k_normed_with_q_gain": ('k = _r32(rms_norm_rows(k, L["k_norm"]', 'k = _r32(rms_norm_rows(k, L["q_norm"]'),
    "step_ffn_uses_attn_norm": ('rms_norm_rows(x, L["ffn_norm"]', 'rms_norm_rows(x, L["attn_norm"]'),
    "step_final_norm_gain": ('rms_norm_rows(x, w["out_norm"]', 'rms_norm_rows(x, L["ffn_norm"]'),
}


def test_real_oracle_passes_every_pin():
    for pin in step_pins.ALL_PINS:
        pin(decode_step)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, "mutation site: %r" % old
    path = os.path.join(tmp_path, "mutant_%s.py" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("mutant_%s" % name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in step_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(pin.__name__)
    assert failed, "no pin caught mutant %s" % name
