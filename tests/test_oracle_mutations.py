"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one plausible mistake into the oracle -- a swapped
nibble, a tie rule, a dropped scale, a transposed operand -- and runs the
pin that should catch it; the pin must fail.  This shows the pins are
strong enough to detect that class of error.
"""

import numpy as np
import pytest

import oracle
import oracle.lora_linear as ol
import oracle.merge as om
import oracle.nf4 as on
from tests import test_oracle_levels as tl
from tests import test_oracle_linear as tlin
from tests import test_oracle_merge as tm
from tests import test_oracle_dropout as tdo
from tests import test_oracle_f16 as tf16
from tests import test_oracle_quant as tq


def _pack_odd_low(codes):
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.array([7], dtype=np.uint8)])
    return (c[1::2] | (c[0::2] << 4)).astype(np.uint8)


def _thresholds_rne():
    lv = on.nf4_levels_f32().astype(np.float64)
    return ((lv[:-1] + lv[1:]) / 2).astype(np.float32)


def _thresholds_tie_up():
    t = _ORIG["thr"]()
    # ties to the upper level: step each exact-midpoint threshold one ulp down
    lv = on.nf4_levels_f32().astype(np.float64)
    mid = (lv[:-1] + lv[1:]) / 2
    exact = t.astype(np.float64) == mid
    t = t.copy()
    t[exact] = np.nextafter(t[exact], np.float32(-np.inf))
    return t


def _levels_symmetric():
    from statistics import NormalDist
    d = NormalDist()
    pm = on.P_MAX
    pos = [d.inv_cdf(pm + (0.5 - pm) * i / 8) for i in range(8)]
    return np.array(sorted([-p for p in pos] + pos)) / d.inv_cdf(pm)


def _double_quant_half_up(absmax, blocksize2=256):
    q, step = _ORIG["dq"](absmax, blocksize2)
    s = np.ascontiguousarray(absmax, dtype=np.float32)
    st = np.repeat(step, blocksize2)[: s.size].astype(np.float64)
    ratio = (s.astype(np.float64) / np.where(st > 0, st, 1)).astype(np.float32)
    q2 = np.minimum(np.floor(ratio.astype(np.float64) + 0.5), 255)
    q2[st == 0] = 0
    return q2.astype(np.uint8), step


def _dequant_no_bf16(packed, q, step, n, blocksize=64, blocksize2=256):
    codes = on.unpack_codes(packed, n)
    scale = on.dequant_scales(q, step, blocksize2)
    prod = (on.nf4_levels_f32().astype(np.float64)[codes]
            * scale[np.arange(n) // blocksize].astype(np.float64)).astype(np.float32)
    # keep the fp32 product's upper half without rounding (truncation)
    return (prod.view(np.uint32) >> 16).astype(np.uint16)


def _bwd_dA_without_scale(x, dy, w, A, B, alpha):
    dX, dA, dB = _ORIG["bwd"](x, dy, w, A, B, alpha)
    return dX, dA / ol.lora_scale(alpha, np.asarray(A).shape[0]), dB


def _bwd_dB_without_scale(x, dy, w, A, B, alpha):
    dX, dA, dB = _ORIG["bwd"](x, dy, w, A, B, alpha)
    return dX, dA, dB / ol.lora_scale(alpha, np.asarray(A).shape[0])


def _bwd_dX_without_adapter(x, dy, w, A, B, alpha):
    dX, dA, dB = _ORIG["bwd"](x, dy, w, A, B, alpha)
    return np.asarray(dy, dtype=np.float64) @ np.asarray(w, dtype=np.float64), dA, dB


def _fwd_scale_r_over_alpha(x, w, A, B, alpha):
    r = 0 if A is None else np.asarray(A).shape[0]
    if not r:
        return _ORIG["fwd"](x, w, A, B, alpha)
    return _ORIG["fwd"](x, w, A, B, r * r / alpha)


def _fwd_wrong_sign(x, w, A, B, alpha):
    return _ORIG["fwd"](x, w, A, B, -alpha)


def _merge_transposed(w_base, A, B, alpha):
    d = _ORIG["merge"](np.zeros_like(np.asarray(w_base, dtype=np.float64)), A, B, alpha)
    return np.asarray(w_base, dtype=np.float64) + d.T


def _merge_scale_r_over_alpha(w_base, A, B, alpha):
    r = 0 if A is None else np.asarray(A).shape[0]
    return _ORIG["merge"](w_base, A, B, r * r / alpha if r else alpha)


def _merged_bf16_from_f64(w_m):
    # one rounding straight from fp64 (no fp32 step)
    v = np.asarray(w_m, dtype=np.float64)
    hi = v.astype(np.float32).view(np.uint32).astype(np.uint64) & 0xFFFF0000
    lo_v = hi.astype(np.uint32).view(np.float32).astype(np.float64)
    up = (hi + 0x10000).astype(np.uint32).view(np.float32).astype(np.float64)
    lo_c, up_c = np.minimum(lo_v, up), np.maximum(lo_v, up)
    pick_up = (np.abs(v - up_c) < np.abs(v - lo_c)) | (
        (np.abs(v - up_c) == np.abs(v - lo_c)) & ((up_c.astype(np.float32).view(np.uint32)
                                                   >> 16) % 2 == 0))
    out = np.where(pick_up, up_c, lo_c).astype(np.float32)
    return (out.view(np.uint32) >> 16).astype(np.uint16)


def _drop_without_rescale(x, keep, p):
    x64 = np.asarray(x, dtype=np.float64)
    return x64 if keep is None else x64 * np.asarray(keep, dtype=np.float64)


def _bwd_dx_adapter_unmasked(x, dy, w, A, B, alpha, keep=None, p=0.0):
    dX, dA, dB = _ORIG["bwd"](x, dy, w, A, B, alpha, keep=keep, p=p)
    if keep is None or A is None:
        return dX, dA, dB
    s = ol.lora_scale(alpha, np.asarray(A).shape[0])
    gA = s * ((np.asarray(dy, dtype=np.float64) @ np.asarray(B, dtype=np.float64))
              @ np.asarray(A, dtype=np.float64))
    base = np.asarray(dy, dtype=np.float64) @ np.asarray(w, dtype=np.float64)
    return base + gA / (1.0 - p), dA, dB


def _fwd_mask_on_base_too(x, w, A, B, alpha, keep=None, p=0.0):
    if keep is None:
        return _ORIG["fwd"](x, w, A, B, alpha)
    xd = np.asarray(x, dtype=np.float64) * np.asarray(keep, dtype=np.float64)
    return _ORIG["fwd"](xd, w, A, B, alpha, keep=keep, p=p)


def _f16_truncating(values_f32):
    # round toward zero: go through float64 -> float16 after clearing the
    # bits below fp16's precision (a plausible cheap conversion)
    v = np.ascontiguousarray(values_f32, dtype=np.float32).view(np.uint32) & 0xFFFFE000
    with np.errstate(over="ignore"):
        return v.view(np.float32).astype(np.float16).view(np.uint16)


_ORIG = {
    "merge": om.merge_adapter,
    "thr": on.nf4_thresholds_f32,
    "dq": on.double_quant,
    "bwd": ol.lora_linear_bwd,
    "fwd": ol.lora_linear_fwd,
}


CASES = [
    # (name, [(module, attr, replacement)], pin)
    ("nibble order swapped", [(on, "pack_codes", _pack_odd_low)],
     tq.test_nibble_packing_hand_example),
    ("round-to-nearest thresholds", [(on, "nf4_thresholds_f32", _thresholds_rne),
                                     (oracle, "nf4_thresholds_f32", _thresholds_rne)],
     tq.test_fp32_value_just_above_a_rounded_up_midpoint_goes_up),
    ("ties to the upper level", [(on, "nf4_thresholds_f32", _thresholds_tie_up)],
     tq.test_ties_go_to_the_lower_level),
    ("symmetric level set without zero", [(on, "nf4_levels_f64", _levels_symmetric),
                                          (oracle, "nf4_levels_f64", _levels_symmetric)],
     tl.test_sixteen_strictly_increasing_levels_with_exact_ends_and_zero),
    ("double quant rounds half up", [(on, "double_quant", _double_quant_half_up),
                                     (oracle, "double_quant", _double_quant_half_up)],
     tq.test_double_quant_rounds_half_to_even),
    ("dequant truncates instead of rounding", [(on, "dequant_nf4_bits", _dequant_no_bf16),
                                               (oracle, "dequant_nf4_bits", _dequant_no_bf16)],
     tq.test_dequant_power_of_two_scale_reduces_to_bf16_of_levels),
    ("dA missing alpha/r", [(oracle, "lora_linear_bwd", _bwd_dA_without_scale)],
     lambda: tlin.test_adjoint_identity_for_A(20)),
    ("dB missing alpha/r", [(oracle, "lora_linear_bwd", _bwd_dB_without_scale)],
     lambda: tlin.test_adjoint_identity_for_B(20)),
    ("dX missing the adapter path", [(oracle, "lora_linear_bwd", _bwd_dX_without_adapter)],
     lambda: tlin.test_adjoint_identity_for_x(20)),
    ("scale r/alpha instead of alpha/r", [(oracle, "lora_linear_fwd", _fwd_scale_r_over_alpha)],
     tlin.test_zero_base_with_identity_adapters_is_scaled_copy),
    ("adapter term subtracted", [(oracle, "lora_linear_fwd", _fwd_wrong_sign)],
     lambda: tlin.test_forward_equals_triple_loop(3, 5, 7, 2, 4.0)),
    ("merge adds (B.A)^T", [(oracle, "merge_adapter", _merge_transposed)],
     lambda: tm.test_merge_equals_triple_loop(4, 4, 1, 1.0)),
    ("merge scaled by r/alpha", [(oracle, "merge_adapter", _merge_scale_r_over_alpha)],
     tm.test_one_entry_update_lands_at_row_of_B_column_of_A),
    ("bf16 export rounded from fp64", [(oracle, "merged_bf16_bits", _merged_bf16_from_f64)],
     tm.test_bf16_export_rounds_through_fp32_to_nearest_even),
    ("dropout without 1/(1-p)", [(ol, "dropped_input", _drop_without_rescale)],
     lambda: tdo.test_forward_equals_triple_loop(3, 5, 7, 2, 4.0, 0.25)),
    ("dropout mask missing on dX's adapter term",
     [(oracle, "lora_linear_bwd", _bwd_dx_adapter_unmasked)],
     lambda: tdo.test_adjoint_identity_for_x(60)),
    ("fp16 conversion truncating", [(on, "f16_rne_bits", _f16_truncating),
                                    (oracle, "f16_rne_bits", _f16_truncating)],
     tf16.test_f16_rounding_hand_values),
    ("dropout applied to the base term too", [(oracle, "lora_linear_fwd", _fwd_mask_on_base_too)],
     tdo.test_nothing_kept_leaves_the_base_alone),
]


@pytest.mark.parametrize("name,patches,pin", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(name, patches, pin, monkeypatch):
    for mod, attr, repl in patches:
        monkeypatch.setattr(mod, attr, repl)
    with pytest.raises(AssertionError):
        pin()


@pytest.mark.parametrize("name,patches,pin", CASES, ids=[c[0] for c in CASES])
def test_pin_passes_without_the_mistake(name, patches, pin):
    pin()
