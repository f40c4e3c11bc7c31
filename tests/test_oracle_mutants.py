"""Planted mistakes in copies of the oracle must each fail some pin.

Each mutant is the oracle's source with one plausible slip (a dropped term,
a wrong sign or index, a transposed operand, an off-by-one mask, a wrong
exponent bias), executed as a separate module on the CPU. The pins are the
ones the real oracle passes, so a mutant that passed them all would show a
blind spot in the pins.
"""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "attention.py")).read()

MUTANTS = {
    "scale_dropped": ("s = c * (q @ k.T)", "s = (q @ k.T)"),
    "causal_off_by_one": ("kj[None, :] <= qi[:, None]", "kj[None, :] < qi[:, None]"),
    "causal_flipped": ("kj[None, :] <= qi[:, None]", "kj[None, :] >= qi[:, None]"),
    "no_max_shift_lse": ("out[b, h] = p @ v[b, h]\n            lse[b, h] = m + np.log(l)",
                         "out[b, h] = p @ v[b, h]\n            lse[b, h] = np.log(l)"),
    "lse_log2": ("out[b, h] = p @ v[b, h]\n            lse[b, h] = m + np.log(l)",
                 "out[b, h] = p @ v[b, h]\n            lse[b, h] = m + np.log2(l)"),
    "decode_lse_log2": ("out[b, h] = p @ v[b, h // G]\n            lse[b, h] = m + np.log(l)",
                        "out[b, h] = p @ v[b, h // G]\n            lse[b, h] = m + np.log2(l)"),
    "pv_transposed_in_dv": ("dv[b, h] = p.T @ do[b, h]", "dv[b, h] = p @ do[b, h]"),
    "missing_D_term": ("ds = p * (dp - dd)", "ds = p * dp"),
    "dk_scale_dropped": ("dk[b, h] = c * (ds.T @ q[b, h])", "dk[b, h] = (ds.T @ q[b, h])"),
    "dq_uses_q": ("dq[b, h] = c * (ds @ k[b, h])", "dq[b, h] = c * (ds @ q[b, h])"),
    "dp_sign": ("dp = do[b, h] @ v[b, h].T", "dp = -(do[b, h] @ v[b, h].T)"),
    "chunks_no_rescale": ("xa * fa + xb * fb", "xa + xb"),
    "chunks_l_no_rescale": ("la * fa + lb * fb", "la + lb"),
    "chunks_earlier_not_rescaled": ("xa * fa + xb * fb", "xa + xb * fb"),
    "e4m3_bias8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "e4m3_subnormal": ("sub = sign * mant * 2.0 ** -9", "sub = sign * mant * 2.0 ** -10"),
    "softmax_no_normalise": ("return e / l, m[:, 0], l[:, 0]", "return e, m[:, 0], l[:, 0]"),
    "dequant_scale_dropped": ("q = dec(qc) * float(np.float32(sq))", "q = dec(qc)"),
    "quantized_bwd_do_scale_dropped": ("do = dec_do(doc) * float(np.float32(sdo))", "do = dec_do(doc)"),
    "e5m2_bias16": ("np.exp2(e - 15.0)", "np.exp2(e - 16.0)"),
    "e5m2_mantissa_bits3": ("(1.0 + mant / 4.0)", "(1.0 + mant / 8.0)"),
    "e5m2_subnormal": ("sub = sign * mant * 2.0 ** -16", "sub = sign * mant * 2.0 ** -17"),
    "gqa_head_map_modulo": ("return forward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), scale, causal, rows)",
                            "return forward(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), scale, causal, rows)"),
    "gqa_dk_first_head_only": ("dke.reshape(B, Hkv, G, N, d).sum(axis=2)", "dke.reshape(B, Hkv, G, N, d)[:, :, 0]"),
    "decode_top_left_mask": ("pos = np.arange(Nk - Nq, Nk)", "pos = np.arange(Nq)"),
    "rows_missing_D_term": ("ds_rows = p_rows * (dp_rows - d_rows)", "ds_rows = p_rows * dp_rows"),
    "rows_mask_by_rank": ("scores(_f64(q[b, h][idx]), kh, scale, causal, idx)",
                          "scores(_f64(q[b, h][idx]), kh, scale, causal)"),
    "tail_dv_uses_ds": ("dv[b, h] = p_t[:, t0:].T @ dot", "dv[b, h] = ds_t[:, t0:].T @ dot"),
    "tail_mask_from_zero": ("scores(qt, _f64(k[b, h]), scale, True, idx)", "scores(qt, _f64(k[b, h]), scale, True)"),
    "decode_head_map_modulo": ("scores(q[b, h], k[b, h // G], scale, causal, pos)",
                               "scores(q[b, h], k[b, h % k.shape[1]], scale, causal, pos)"),
}


def _load(name, old, new):
    assert SRC.count(old) == 1, f"mutant {name}: pattern not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load(name, *MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash caused by the slip
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
