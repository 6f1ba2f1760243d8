"""Pins of the oracle's exact mode: the int8 activation quantiser (constructed
groups), exact int32 group sums (int64 reference, extreme bound), the fp32
group combine (power-of-two closed form, fp64 bound) and the combine."""
import numpy as np
import pytest

import oracle
from tests import refmath


def _bf16(v):
    return refmath.bf16_from_f32(np.asarray(v, np.float32))


def test_quantiser_constructed_groups():
    # amax 127 -> scale exactly 1; then q = rint(x) with ties to even
    v = np.zeros(32, np.float32)
    v[:9] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -126.5, 100.25]
    q, s = oracle.quant_act_int8(_bf16(v)[None, :])
    assert s[0, 0] == 1.0
    np.testing.assert_array_equal(q[0, :9], [127, 2, 4, -2, 0, 2, 0, -126, 100])
    # all-zero group: scale 0, codes 0
    q, s = oracle.quant_act_int8(np.zeros((1, 64), np.uint16))
    assert np.all(s == 0) and np.all(q == 0)
    # negative extreme maps to -127, never -128
    v = np.linspace(-3.0, 1.0, 32).astype(np.float32)
    q, s = oracle.quant_act_int8(_bf16(v)[None, :])
    assert q[0, 0] == -127 and q.min() >= -127


def test_quantiser_properties_random():
    g = np.random.default_rng(0)
    x = _bf16(g.standard_normal((50, 256)) * 10.0 ** g.integers(-3, 3, (50, 1)))
    q, s = oracle.quant_act_int8(x)
    xf = refmath.bf16_to_f32(x).reshape(50, 8, 32).astype(np.float64)
    amax = np.abs(xf).max(axis=2)
    np.testing.assert_allclose(s, amax / 127.0, rtol=2 ** -23)
    qg = q.reshape(50, 8, 32).astype(np.float64)
    assert np.all(np.abs(qg).max(axis=2) == 127)
    err = np.abs(xf - qg * s[..., None].astype(np.float64))
    # x/s is an fp32 quotient: it can land on a half-integer the exact quotient
    # misses by up to half an ulp of 127
    assert np.all(err <= s[..., None] * (0.5 + 128 * 2.0 ** -24))
    # fp32 input path agrees with the bf16 input path on the same values
    q2, s2 = oracle.quant_f32_int8(refmath.bf16_to_f32(x))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s)


def test_group_sums_exact_and_bounded():
    g = np.random.default_rng(1)
    M, N, K = 6, 10, 256
    qx = g.integers(-127, 128, (M, K)).astype(np.int8)
    packed = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    G32, G64 = oracle.group_sums(qx, packed, K, with_int64=True)
    np.testing.assert_array_equal(G32.astype(np.int64), G64)
    qw = refmath.unpack_int4_np(packed, K).astype(np.int64)
    ref = np.einsum("mgi,ngi->mng", qx.astype(np.int64).reshape(M, K // 32, 32), qw.reshape(N, K // 32, 32))
    np.testing.assert_array_equal(G64, ref)
    # extreme: q_x = 127 everywhere, q_w = -8 everywhere -> -8 * 127 * 32
    qx = np.full((1, 64), 127, np.int8)
    packed = np.full((1, 32), 0x88, np.uint8)
    G = oracle.group_sums(qx, packed, 64)
    assert np.all(G == -32512)


def test_exact_linear_power_of_two_closed_form():
    g = np.random.default_rng(2)
    M, N, K = 4, 12, 7168
    qx = g.integers(-127, 128, (M, K)).astype(np.int8)
    packed = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    for a, b in ((-7, -5), (0, 0), (-12, 3)):
        sw = np.full((N, K // 32), _bf16(2.0 ** a)[()], np.uint16)
        sx = np.full((M, K // 32), 2.0 ** b, np.float32)
        y = oracle.exact_linear(qx, sx, packed, sw)
        qw = refmath.unpack_int4_np(packed, K).astype(np.int64)
        total = qx.astype(np.int64) @ qw.T  # |total| <= 224 * 32512 < 2^24: exact in fp32
        np.testing.assert_array_equal(y.astype(np.float64), total.astype(np.float64) * 2.0 ** (a + b))


def test_exact_linear_general_within_fp64_bound():
    g = np.random.default_rng(3)
    M, N, K = 3, 16, 2048
    qx = g.integers(-127, 128, (M, K)).astype(np.int8)
    sx = (g.uniform(0.001, 0.05, (M, K // 32))).astype(np.float32)
    packed = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sw = _bf16(g.uniform(0.005, 0.02, (N, K // 32)))
    y = oracle.exact_linear(qx, sx, packed, sw).astype(np.float64)
    G = oracle.group_sums(qx, packed, K).astype(np.float64)  # [M,N,g]
    terms = G * refmath.bf16_to_f32(sw)[None].astype(np.float64) * sx[:, None, :].astype(np.float64)
    exact = terms.sum(axis=2)
    bound = (K // 32) * 2.0 ** -24 * np.abs(terms).sum(axis=2) * 1.01
    assert np.all(np.abs(y - exact) <= bound)


def test_exact_expert_chain():
    """g/u by the power-of-two closed form; h = silu(g)*u quantised; y within fp64 bound."""
    g = np.random.default_rng(4)
    H, I, E = 256, 128, 3
    qx = g.integers(-127, 128, (E, H)).astype(np.int8)
    sx = np.full((E, H // 32), 2.0 ** -6, np.float32)
    W = {}
    for name, (N, K) in (("g", (I, H)), ("u", (I, H)), ("d", (H, I))):
        W["w" + name] = g.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    W["sg"] = np.full((E, I, H // 32), _bf16(2.0 ** -7)[()], np.uint16)
    W["su"] = np.full((E, I, H // 32), _bf16(2.0 ** -6)[()], np.uint16)
    W["sd"] = _bf16(g.uniform(0.005, 0.02, (E, H, I // 32)))
    experts = np.arange(E, dtype=np.int32)
    r = oracle.experts_exact(qx, sx, experts, W, want=("g", "u", "qh", "sh", "y"))
    for e in range(E):
        qg = refmath.unpack_int4_np(W["wg"][e], H).astype(np.int64)
        qu = refmath.unpack_int4_np(W["wu"][e], H).astype(np.int64)
        np.testing.assert_array_equal(r["g"][e], (qg @ qx[e].astype(np.int64)) * 2.0 ** -13)
        np.testing.assert_array_equal(r["u"][e], (qu @ qx[e].astype(np.int64)) * 2.0 ** -12)
        h64 = refmath.silu64(r["g"][e]) * r["u"][e].astype(np.float64)
        recon = r["qh"][e].astype(np.float64) * np.repeat(r["sh"][e], 32).astype(np.float64)
        assert np.all(np.abs(recon - h64) <= np.repeat(r["sh"][e], 32) * 0.5 + np.abs(h64) * 2 ** -20 + 1e-30)
        qd = refmath.unpack_int4_np(W["wd"][e], I).astype(np.float64)
        sd = np.repeat(refmath.bf16_to_f32(W["sd"][e]).astype(np.float64), 32, axis=1)
        terms = qd * sd * recon[None, :]
        exact = terms.sum(axis=1)
        assert np.all(np.abs(r["y"][e] - exact) <= (I // 32) * 2.0 ** -24 * np.abs(terms).sum(axis=1) * 1.01 + 1e-30)


def test_combine_f32():
    g = np.random.default_rng(5)
    y = g.standard_normal((4, 1, 32)).astype(np.float32)
    np.testing.assert_array_equal(oracle.combine_f32(y, np.ones((4, 1), np.float32)), y[:, 0])
    y = g.standard_normal((4, 8, 32)).astype(np.float32)
    w = g.uniform(0, 0.3, (4, 8)).astype(np.float32)
    out = oracle.combine_f32(y, w).astype(np.float64)
    exact = np.einsum("tk,tkh->th", w.astype(np.float64), y.astype(np.float64))
    bound = 8 * 2.0 ** -23 * np.einsum("tk,tkh->th", np.abs(w).astype(np.float64), np.abs(y).astype(np.float64))
    assert np.all(np.abs(out - exact) <= bound)


# ---------------------------------------------------------------- 16-bit activations (act_bits = 16)

def test_quantiser16_constructed_groups():
    # amax 2^14 -> s = fl(2^14 / 32767); the amax element maps to 32767, its negative to -32767
    v = np.zeros(32, np.float32)
    v[:4] = [16384.0, -16384.0, 1.0, 0.0]
    q, s = oracle.quant_act_int16(_bf16(v)[None, :])
    assert s[0, 0] == np.float32(16384.0) / np.float32(32767.0)
    assert q[0, 0] == 32767 and q[0, 1] == -32767 and q[0, 3] == 0
    assert q[0, 2] == int(np.rint(np.float32(1.0) / s[0, 0]))
    q, s = oracle.quant_act_int16(np.zeros((1, 64), np.uint16))
    assert np.all(s == 0) and np.all(q == 0)


def test_quantiser16_properties_random():
    g = np.random.default_rng(10)
    x = _bf16(g.standard_normal((40, 256)) * 10.0 ** g.integers(-3, 3, (40, 1)))
    q, s = oracle.quant_act_int16(x)
    xf = refmath.bf16_to_f32(x).reshape(40, 8, 32).astype(np.float64)
    amax = np.abs(xf).max(axis=2)
    np.testing.assert_allclose(s, amax / 32767.0, rtol=2 ** -23)
    qg = q.reshape(40, 8, 32).astype(np.float64)
    assert np.all(np.abs(qg).max(axis=2) == 32767) and q.min() >= -32767
    err = np.abs(xf - qg * s[..., None].astype(np.float64))
    assert np.all(err <= s[..., None] * (0.5 + 32768 * 2.0 ** -24))


def test_group_sums16_exact_and_bounded():
    g = np.random.default_rng(11)
    M, N, K = 5, 9, 256
    qx = g.integers(-32767, 32768, (M, K)).astype(np.int16)
    packed = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    G32, G64 = oracle.group_sums16(qx, packed, K, with_int64=True)
    qw = refmath.unpack_int4_np(packed, K).astype(np.int64)
    ref = np.einsum("mgi,ngi->mng", qx.astype(np.int64).reshape(M, K // 32, 32), qw.reshape(N, K // 32, 32))
    np.testing.assert_array_equal(G64, ref)
    np.testing.assert_array_equal(G32.astype(np.int64), ref)
    qx = np.full((1, 64), 32767, np.int16)
    packed = np.full((1, 32), 0x88, np.uint8)
    assert np.all(oracle.group_sums16(qx, packed, 64) == -8 * 32767 * 32)


def test_exact_linear16_power_of_two_closed_form():
    """With power-of-two scales and a total below 2^24 every step is exact."""
    g = np.random.default_rng(12)
    M, N, K = 4, 12, 256
    qx = g.integers(-2000, 2001, (M, K)).astype(np.int16)  # |total| <= 8 * 32 * 8 * 2000 < 2^24
    packed = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    qw = refmath.unpack_int4_np(packed, K).astype(np.int64)
    total = qx.astype(np.int64) @ qw.T
    for a, b in ((-7, -5), (0, 0), (-12, 3)):
        sw = np.full((N, K // 32), _bf16(2.0 ** a)[()], np.uint16)
        sx = np.full((M, K // 32), 2.0 ** b, np.float32)
        y = oracle.exact_linear16(qx, sx, packed, sw)
        np.testing.assert_array_equal(y.astype(np.float64), total.astype(np.float64) * 2.0 ** (a + b))


def test_exact_linear16_general_within_fp64_bound():
    g = np.random.default_rng(13)
    M, N, K = 3, 16, 2048
    qx = g.integers(-32767, 32768, (M, K)).astype(np.int16)
    sx = (g.uniform(1e-6, 5e-4, (M, K // 32))).astype(np.float32)
    packed = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sw = _bf16(g.uniform(0.005, 0.02, (N, K // 32)))
    y = oracle.exact_linear16(qx, sx, packed, sw).astype(np.float64)
    G = oracle.group_sums16(qx, packed, K).astype(np.float64)
    terms = G * refmath.bf16_to_f32(sw)[None].astype(np.float64) * sx[:, None, :].astype(np.float64)
    exact = terms.sum(axis=2)
    # each group: the product s_w*G rounded once, then one fma rounding
    bound = (K // 32 + 1) * 2.0 ** -24 * np.abs(terms).sum(axis=2) * 1.01
    assert np.all(np.abs(y - exact) <= bound)


def test_exact16_expert_chain():
    g = np.random.default_rng(14)
    H, I, E = 256, 128, 3
    qx = g.integers(-2000, 2001, (E, H)).astype(np.int16)
    sx = np.full((E, H // 32), 2.0 ** -10, np.float32)
    W = {}
    for name, (N, K) in (("g", (I, H)), ("u", (I, H)), ("d", (H, I))):
        W["w" + name] = g.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    W["sg"] = np.full((E, I, H // 32), _bf16(2.0 ** -7)[()], np.uint16)
    W["su"] = np.full((E, I, H // 32), _bf16(2.0 ** -6)[()], np.uint16)
    W["sd"] = _bf16(g.uniform(0.005, 0.02, (E, H, I // 32)))
    r = oracle.experts_exact16(qx, sx, np.arange(E, dtype=np.int32), W, want=("g", "u", "qh", "sh", "y"))
    for e in range(E):
        qg = refmath.unpack_int4_np(W["wg"][e], H).astype(np.int64)
        qu = refmath.unpack_int4_np(W["wu"][e], H).astype(np.int64)
        np.testing.assert_array_equal(r["g"][e], (qg @ qx[e].astype(np.int64)) * 2.0 ** -17)
        np.testing.assert_array_equal(r["u"][e], (qu @ qx[e].astype(np.int64)) * 2.0 ** -16)
        h64 = refmath.silu64(r["g"][e]) * r["u"][e].astype(np.float64)
        recon = r["qh"][e].astype(np.float64) * np.repeat(r["sh"][e], 32).astype(np.float64)
        assert np.abs(r["qh"][e]).max() <= 32767
        assert np.all(np.abs(recon - h64) <= np.repeat(r["sh"][e], 32) * 0.5 + np.abs(h64) * 2 ** -20 + 1e-30)
        qd = refmath.unpack_int4_np(W["wd"][e], I).astype(np.float64)
        sd = np.repeat(refmath.bf16_to_f32(W["sd"][e]).astype(np.float64), 32, axis=1)
        terms = qd * sd * recon[None, :]
        exact = terms.sum(axis=1)
        bound = (I // 32 + 1) * 2.0 ** -24 * np.abs(terms).sum(axis=1) * 1.01 + 1e-30
        assert np.all(np.abs(r["y"][e] - exact) <= bound)


# ---------------------------------------------------------------- ExactLinear, 8-bit weights

def test_exact_linear_i8w_power_of_two_closed_form():
    g = np.random.default_rng(20)
    M, N, K = 5, 7, 512
    qx = g.integers(-40, 41, (M, K)).astype(np.int8)  # |total| <= 512 * 40 * 40 < 2^24
    qw = g.integers(-40, 41, (N, K)).astype(np.int8)
    total = qx.astype(np.int64) @ qw.astype(np.int64).T
    for a, b in ((-7, -5), (0, 0), (-12, 3)):
        sw = np.full((N, K // 32), 2.0 ** a, np.float32)
        sx = np.full((M, K // 32), 2.0 ** b, np.float32)
        y = oracle.exact_linear_i8w(qx, sx, qw, sw)
        np.testing.assert_array_equal(y.astype(np.float64), total.astype(np.float64) * 2.0 ** (a + b))


def test_exact_linear_i8w_within_fp64_bound():
    g = np.random.default_rng(21)
    M, N, K = 4, 9, 2048
    x = _bf16(g.standard_normal((M, K)))
    w = _bf16(g.standard_normal((N, K)) * 0.02)
    qx, sx = oracle.quant_act_int8(x)
    qw, sw = oracle.quant_act_int8(w)   # weights take the same per-row, per-group quantiser
    y = oracle.exact_linear_i8w(qx, sx, qw, sw).astype(np.float64)
    G = np.einsum("mgi,ngi->mng", qx.astype(np.int64).reshape(M, -1, 32), qw.astype(np.int64).reshape(N, -1, 32))
    assert np.abs(G).max() <= 32 * 127 * 127
    terms = G.astype(np.float64) * sw[None].astype(np.float64) * sx[:, None, :].astype(np.float64)
    exact = terms.sum(axis=2)
    bound = (K // 32 + 1) * 2.0 ** -24 * np.abs(terms).sum(axis=2) * 1.01
    assert np.all(np.abs(y - exact) <= bound)
    # and close to the unquantised product (the quantisation error, not a pin of the fold)
    ref = refmath.bf16_to_f32(x).astype(np.float64) @ refmath.bf16_to_f32(w).astype(np.float64).T
    assert np.max(np.abs(y - ref)) <= 0.05 * np.max(np.abs(ref))
