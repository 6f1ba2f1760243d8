"""Pins of the oracle's fixed-order and fixed-rounding readings with constructed
inputs whose expected results follow by hand (or from one exact rounding of an
exact rational), chosen so that each plausible alternative reading gives a
different value:

- router logits ("Kimi K2.5 donor reference", record "MoEGate.forward: logits";
  reading: 64-element block sums in ascending index, then the block sums in
  ascending block order, all fp32 from 0);
- the exact-mode group fold ("Kimi exact-generator adaptation", "The proposed
  substitution" and "Sources & provenance": group size 32, exact integer group
  MACs; reading: acc = fma(fl32(s_w * G), s_x, acc) over groups ascending), for
  8-bit and 16-bit activation codes and for 8-bit weights;
- the exact-mode combine (record "Sum the selected expert outputs with their
  routing weights"; reading: slots ascending, each product rounded, then added);
- the activation quantiser (reading: s = amax / 127 by IEEE division, codes
  rint(x / s) by IEEE division, ties to even).

Every case also checks, in numpy fp32, that the alternative it rules out would
give another value, so the case keeps discriminating if it is edited.
"""
from fractions import Fraction

import numpy as np

import oracle
from tests import refmath

F = Fraction
TWO24 = 2.0 ** 24


def _bf16(v):
    return refmath.bf16_from_f32(np.asarray(v, np.float32))


def _f32(v):
    return np.float32(v)


# ---------------------------------------------------------------- router logits

def _logit(vals):
    """One token whose products with an all-ones router row are `vals` (all exact in bf16)."""
    H = len(vals)
    x = _bf16(np.asarray(vals, np.float32))[None, :]
    w = _bf16(np.ones((1, H), np.float32))
    return float(oracle.router_logits(x, w)[0, 0])


def _flat(vals):
    acc = _f32(0)
    for v in vals:
        acc = _f32(acc + _f32(v))
    return float(acc)


def _blocked(vals, B, descending_blocks=False):
    sums = []
    for b in range(0, len(vals), B):
        s = _f32(0)
        for v in vals[b:b + B]:
            s = _f32(s + _f32(v))
        sums.append(s)
    if descending_blocks:
        sums = sums[::-1]
    acc = _f32(0)
    for s in sums:
        acc = _f32(acc + s)
    return float(acc)


def test_router_block_sums_keep_what_a_running_sum_absorbs():
    # 2^24 in block 0, sixty-four ones in block 1: block 1 sums to 64 exactly and
    # 2^24 + 64 is representable; a single running sum absorbs each 1 (2^24 + 1 ties to 2^24)
    vals = [0.0] * 128
    vals[0] = TWO24
    for i in range(64, 128):
        vals[i] = 1.0
    assert _logit(vals) == TWO24 + 64
    assert _flat(vals) == TWO24
    assert _blocked(vals, 128) == TWO24


def test_router_block_width_is_64():
    # ones at 32..63 share block 0 with 2^24 under 64-wide blocks (absorbed one by one);
    # 32-wide blocks would sum them first and keep 32 of them
    vals = [0.0] * 128
    vals[0] = TWO24
    for i in range(32, 64):
        vals[i] = 1.0
    assert _logit(vals) == TWO24
    assert _blocked(vals, 32) == TWO24 + 32


def test_router_block_sums_added_in_ascending_order():
    # block sums (2^24, 1, 1): ascending absorbs both ones, descending keeps 2
    vals = [0.0] * 192
    vals[0], vals[64], vals[128] = TWO24, 1.0, 1.0
    assert _logit(vals) == TWO24
    assert _blocked(vals, 64, descending_blocks=True) == TWO24 + 2


def test_router_block_summed_in_ascending_index():
    # block 0 = (1, 1, 2^24): ascending gives 2 + 2^24; descending absorbs both ones
    vals = [0.0] * 64
    vals[0], vals[1], vals[2] = 1.0, 1.0, TWO24
    assert _logit(vals) == TWO24 + 2
    assert _flat(vals[::-1]) == TWO24


# ---------------------------------------------------------------- exact fold, 8-bit codes

def _one_row(groups_q_w, groups_q_x):
    """Pack one weight row / one activation row from per-group code lists (zeros elsewhere)."""
    NG = len(groups_q_w)
    qw = np.zeros(32 * NG, np.int64)
    qx = np.zeros(32 * NG, np.int64)
    for g in range(NG):
        for i, (a, b) in enumerate(zip(groups_q_w[g], groups_q_x[g])):
            qw[32 * g + i], qx[32 * g + i] = a, b
    return qw, qx


def _exact8(qw, qx, sw, sx):
    packed = refmath.pack_int4_np(qw[None, :])
    return float(oracle.exact_linear(qx[None, :].astype(np.int8), np.asarray(sx, np.float32)[None, :], packed,
                                     _bf16(sw)[None, :])[0, 0])


BIG_W = [-8] * 32   # with q_x = -64 everywhere: G = 32 * 512 = 2^14
BIG_X = [-64] * 32


def test_exact_fold_ascending_groups():
    # group terms 2^14 * 2^10 * 1 = 2^24, then 1, then 1: ascending absorbs both ones
    qw, qx = _one_row([BIG_W, [1], [1]], [BIG_X, [1], [1]])
    assert _exact8(qw, qx, [2.0 ** 10, 1.0, 1.0], [1.0, 1.0, 1.0]) == TWO24
    # descending: 1, 2, then 2^24 + 2
    acc = _f32(0)
    for t in (1.0, 1.0, TWO24):
        acc = _f32(acc + _f32(t))
    assert float(acc) == TWO24 + 2


def test_exact_fold_is_fused():
    # group 1: G = 3, s_w = 1, s_x = fl32(1/3): the exact product is 1 + 2^-25.
    # fma(3, s_x, 2^24) rounds 2^24 + 1 + 2^-25 once -> 2^24 + 2;
    # a rounded product (1.0) then an add gives 2^24 + 1 -> ties to 2^24
    third = _f32(1) / _f32(3)
    qw, qx = _one_row([BIG_W, [1]], [BIG_X, [3]])
    assert _exact8(qw, qx, [2.0 ** 10, 1.0], [1.0, float(third)]) == TWO24 + 2
    assert float(_f32(_f32(TWO24) + _f32(_f32(3) * third))) == TWO24


# (q_w, q_x, s_w (a bf16 value), s_x): single-element groups where one rounding of
# s_w * G * s_x differs from fma(G, fl32(s_w * s_x)) and from fma(fl32(G * s_x), s_w)
ASSOC8 = [(5, -43, 0.016845703125, 0.01585654728114605), (-3, -112, 0.0146484375, 0.04277900978922844),
          (-4, 56, 0.017578125, 0.014812013134360313)]


def test_exact_fold_single_group_rounds_once():
    for qw_, qx_, sw, sx in ASSOC8:
        sx = float(_f32(sx))
        G = qw_ * qx_
        want = refmath.rn32(F(sw) * G * F(sx))   # s_w * G is exact for int4 x int8
        qw, qx = _one_row([[qw_]], [[qx_]])
        assert _exact8(qw, qx, [sw], [sx]) == want
        assert float(_f32(_f32(G) * _f32(_f32(sw) * _f32(sx)))) != want
        assert float(_f32(_f32(_f32(G) * _f32(sx)) * _f32(sw))) != want


# ---------------------------------------------------------------- exact fold, 16-bit codes

def _exact16(qw, qx, sw, sx):
    packed = refmath.pack_int4_np(qw[None, :])
    return float(oracle.exact_linear16(qx[None, :].astype(np.int16), np.asarray(sx, np.float32)[None, :], packed,
                                       _bf16(sw)[None, :])[0, 0])


# s_w * G is not exact here (G has up to 18 significant bits): the reading rounds it once,
# then the fma rounds once more
ASSOC16 = [(6, -31163, 0.01507568359375, 0.0004596252110786736),
           (-3, 27373, 0.01531982421875, 0.0002506778691895306),
           (-5, -21339, 0.01226806640625, 0.00018877234833780676)]


def test_exact16_fold_rounds_the_weight_product_then_fuses():
    for qw_, qx_, sw, sx in ASSOC16:
        sx = float(_f32(sx))
        G = qw_ * qx_
        want = refmath.rn32(F(refmath.rn32(F(sw) * G)) * F(sx))
        qw, qx = _one_row([[qw_]], [[qx_]])
        assert _exact16(qw, qx, [sw], [sx]) == want
        assert refmath.rn32(F(sw) * G * F(sx)) != want                       # one rounding of the triple
        assert refmath.rn32(G * F(refmath.rn32(F(sw) * F(sx)))) != want      # G * fl32(s_w * s_x)
        assert refmath.rn32(F(refmath.rn32(G * F(sx))) * F(sw)) != want      # fl32(G * s_x) * s_w


def test_exact16_fold_ascending_and_fused():
    # 2^24 from group 0 (one element -8 * -2048 = 2^14, s_w = 2^10), then G = 3 with s_x = fl32(1/3)
    third = float(_f32(1) / _f32(3))
    qw, qx = _one_row([[-8], [1]], [[-2048], [3]])
    assert _exact16(qw, qx, [2.0 ** 10, 1.0], [1.0, third]) == TWO24 + 2
    qw, qx = _one_row([[-8], [1], [1]], [[-2048], [1], [1]])
    assert _exact16(qw, qx, [2.0 ** 10, 1.0, 1.0], [1.0, 1.0, 1.0]) == TWO24


# ---------------------------------------------------------------- ExactLinear, 8-bit weights

def _exact_i8w(qw, qx, sw, sx):
    return float(oracle.exact_linear_i8w(qx[None, :].astype(np.int8), np.asarray(sx, np.float32)[None, :],
                                         qw[None, :].astype(np.int8), np.asarray(sw, np.float32)[None, :])[0, 0])


ASSOC_I8W = [(-2, 31, 0.0010470731649547815, 0.0028110251296311617),
             (38, -6, 0.0008331130957230926, 0.031080855056643486),
             (-54, -49, 0.0010755888652056456, 0.013775511644780636)]


def test_exact_i8w_fold_rounds_the_weight_product_then_fuses():
    for qw_, qx_, sw, sx in ASSOC_I8W:
        sw, sx = float(_f32(sw)), float(_f32(sx))
        G = qw_ * qx_
        want = refmath.rn32(F(refmath.rn32(F(sw) * G)) * F(sx))
        qw, qx = _one_row([[qw_]], [[qx_]])
        assert _exact_i8w(qw, qx, [sw], [sx]) == want
        assert refmath.rn32(F(sw) * G * F(sx)) != want
        assert refmath.rn32(G * F(refmath.rn32(F(sw) * F(sx)))) != want
        assert refmath.rn32(F(refmath.rn32(G * F(sx))) * F(sw)) != want


def test_exact_i8w_fold_ascending_and_fused():
    third = float(_f32(1) / _f32(3))
    big_w, big_x = [16] * 32, [32] * 32   # G = 2^14
    qw, qx = _one_row([big_w, [1]], [big_x, [3]])
    assert _exact_i8w(qw, qx, [2.0 ** 10, 1.0], [1.0, third]) == TWO24 + 2
    qw, qx = _one_row([big_w, [1], [1]], [big_x, [1], [1]])
    assert _exact_i8w(qw, qx, [2.0 ** 10, 1.0, 1.0], [1.0, 1.0, 1.0]) == TWO24


# ---------------------------------------------------------------- exact combine

def test_exact_combine_slots_ascending_product_then_add():
    # slots (2^24, 1, 1) with weight 1: ascending absorbs both ones
    y = np.array([[[TWO24], [1.0], [1.0]]], np.float32)
    w = np.ones((1, 3), np.float32)
    assert float(oracle.combine_f32(y, w)[0, 0]) == TWO24
    # slot 1: 3 * fl32(1/3) = 1 + 2^-25 rounds to 1 before the add, so 2^24 + 1 ties to 2^24;
    # a fused step would give 2^24 + 2
    third = _f32(1) / _f32(3)
    y = np.array([[[TWO24], [3.0]]], np.float32)
    w = np.array([[1.0, third]], np.float32)
    assert float(oracle.combine_f32(y, w)[0, 0]) == TWO24
    assert refmath.rn32(F(TWO24) + 3 * F(float(third))) == TWO24 + 2


# ---------------------------------------------------------------- quantiser divisions

def test_quantiser_scale_is_a_division():
    # amax / 127 and amax * fl32(1/127) round differently for these bf16 values
    for amax in (286.0, 175.0, 207.0, 87.5):
        v = np.zeros(32, np.float32)
        v[0] = amax
        _, s = oracle.quant_act_int8(_bf16(v)[None, :])
        assert float(s[0, 0]) == refmath.rn32(F(amax) / 127)
        assert float(_f32(amax) * (_f32(1) / _f32(127))) != float(s[0, 0])


# (amax, x): x / s lands next to the tie 63.5; the IEEE quotient and the product with
# fl32(1/s) fall on different sides of it
QDIV8 = [(144.0, 72.0), (112.5, 56.25), (38.0, 19.0), (72.0, 36.0), (39.25, -19.625), (28.125, 14.0625)]


def test_quantiser_codes_use_the_ieee_quotient():
    for amax, x in QDIV8:
        v = np.zeros(32, np.float32)
        v[0], v[1] = amax, x
        q, s = oracle.quant_act_int8(_bf16(v)[None, :])
        sf = F(refmath.rn32(F(amax) / 127))
        assert float(s[0, 0]) == float(sf)
        want = refmath.rint_half_even(F(refmath.rn32(F(x) / sf)))
        assert int(q[0, 1]) == want
        alt = int(np.rint(_f32(x) * (_f32(1) / _f32(float(sf)))))
        assert alt != want


QDIV16 = [(203.0, 101.5), (204.0, 102.0), (120.0, 60.0), (58.5, 29.25), (247.0, 123.5)]


def test_quantiser16_codes_use_the_ieee_quotient():
    for amax, x in QDIV16:
        v = np.zeros(32, np.float32)
        v[0], v[1] = amax, x
        q, s = oracle.quant_act_int16(_bf16(v)[None, :])
        sf = F(refmath.rn32(F(amax) / 32767))
        assert float(s[0, 0]) == float(sf)
        want = refmath.rint_half_even(F(refmath.rn32(F(x) / sf)))
        assert int(q[0, 1]) == want
        assert int(np.rint(_f32(x) * (_f32(1) / _f32(float(sf))))) != want
