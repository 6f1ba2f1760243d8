"""The HIP path on the constructed inputs that pin the oracle's fixed orders and
roundings (router block order, exact-mode group fold, exact combine, quantiser
divisions): with these inputs any other order or association gives other bits,
so bit equality with the oracle shows the kernels take the same readings.
The readings are those of the router record "MoEGate.forward: logits" ("Kimi
K2.5 donor reference") and of the exact integer group MACs of the "Kimi
exact-generator adaptation" page ("The proposed substitution", group size 32)."""
import numpy as np
import pytest
import torch

import oracle
from tests import refmath
from tests.gpu_common import bf16_dev, say

pytestmark = pytest.mark.gpu

THIRD = float(np.float32(1) / np.float32(3))
ASSOC8 = [(5, -43, 0.016845703125, 0.01585654728114605), (-3, -112, 0.0146484375, 0.04277900978922844),
          (-4, 56, 0.017578125, 0.014812013134360313)]
ASSOC16 = [(6, -31163, 0.01507568359375, 0.0004596252110786736),
           (-3, 27373, 0.01531982421875, 0.0002506778691895306),
           (-5, -21339, 0.01226806640625, 0.00018877234833780676)]
ASSOC_I8W = [(-2, 31, 0.0010470731649547815, 0.0028110251296311617),
             (38, -6, 0.0008331130957230926, 0.031080855056643486),
             (-54, -49, 0.0010755888652056456, 0.013775511644780636)]


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_routed_expert_moe_amd import moe
    return moe


def _bf16(v):
    return refmath.bf16_from_f32(np.asarray(v, np.float32))


# ---------------------------------------------------------------- router
# The oracle's constructed logit cases scaled by 2^-20 (16 plays 2^24's part: its
# half ulp is one unit), negated so the sigmoid sits on its steep exponential tail
# where one ulp of the logit moves the score by many ulps.
BIG, UNIT = -16.0, -(2.0 ** -20)


def _router_rows(H, base):
    rows = np.zeros((4, H), np.float32)
    rows[0, base + 0] = BIG
    rows[0, base + 64:base + 128] = UNIT                # blocks keep 64 units: BIG + 64 UNIT
    rows[1, base + 0] = BIG
    rows[1, base + 32:base + 64] = UNIT                 # same block: absorbed one by one
    rows[2, base + 0], rows[2, base + 64], rows[2, base + 128] = BIG, UNIT, UNIT  # block sums ascending
    rows[3, base + 0], rows[3, base + 1], rows[3, base + 2] = UNIT, UNIT, BIG     # ascending index
    return rows


@pytest.mark.parametrize("T,H,base", [(1, 256, 0), (300, 256, 0), (64, 7168, 6912), (1024, 7168, 128)])
def test_route_constructed_logit_orders(m, T, H, base):
    say(f"route constructed orders T={T} H={H} base={base}")
    w = _bf16(_router_rows(H, base))
    x = _bf16(np.ones((T, H), np.float32))
    b = np.zeros(4, np.float32)
    logits = oracle.router_logits(x[:1], w)[0]
    want = np.array([BIG + 64 * UNIT, BIG, BIG, BIG + 2 * UNIT], np.float32)
    np.testing.assert_array_equal(logits, want)
    ridx, rw = oracle.route(x, w, b, 4, False)
    idx = torch.empty((T, 4), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, 4), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.moe_route_workspace_bytes(T, H, 4), dtype=torch.uint8, device="cuda")
    m.moe_route(bf16_dev(x), bf16_dev(w), torch.from_numpy(b).cuda(), 4, False, idx, wt, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_array_equal(wt.cpu().numpy(), rw)
    # the four scores are those of the four hand-derived logits, all distinct
    assert len(set(np.float32(oracle.sigmoid_ref_n(want)).tolist())) == 3  # cases 1 and 2 share BIG
    np.testing.assert_array_equal(np.sort(rw[0]), np.sort(oracle.sigmoid_ref_n(want)))


# ---------------------------------------------------------------- exact fold in the grouped down projection
def _down_case(T, H, act_bits):
    """Weights [H, 128] and activations [T, 128] built from the constructed groups:
    group 0 gives a 2^24 term (G = 2^14, s_w = 2^9, s_x = 2) on half the pairs,
    groups 1 and 2 add 1 (or 3 fl32(1/3)), group 3 the association fixtures."""
    I = 128
    fx = ASSOC8 if act_bits == 8 else ASSOC16
    qw = np.zeros((H, I), np.int64)
    sw = np.ones((H, I // 32), np.float32)
    for n in range(H):
        if n % 2 == 0:
            qw[n, 0:32] = -8
            sw[n, 0] = 2.0 ** 9
        qw[n, 32] = 1
        qw[n, 64] = 1
        qw[n, 96] = fx[n % 3][0]
        sw[n, 3] = fx[n % 3][2]
    qx = np.zeros((T, I), np.int64)
    sx = np.zeros((T, I // 32), np.float32)
    for p in range(T):
        if p % 2 == 0:
            if act_bits == 8:
                qx[p, 0:32] = -64
            else:
                qx[p, 0] = -2048
            sx[p, 0] = 2.0
        if p % 4 < 2:
            qx[p, 32], sx[p, 1] = 3, THIRD
        else:
            qx[p, 32], sx[p, 1] = 1, 1.0
        if p % 3:
            qx[p, 64], sx[p, 2] = 1, 1.0
        qx[p, 96], sx[p, 3] = fx[p % 3][1], fx[p % 3][3]
    return qw, _bf16(sw), qx, sx


@pytest.mark.parametrize("T,act_bits", [(5, 8), (40, 8), (300, 8), (5, 16), (40, 16)])
def test_grouped_down_exact_constructed_fold(m, T, act_bits):
    """One expert, every row routed to it: few rows take the decode kernel, more the tile kernels."""
    say(f"grouped down exact constructed fold T={T} act_bits={act_bits}")
    from tests.test_gpu_kernels import _dev_experts
    H, I = 256, 128
    qw, sw, qx, sx = _down_case(T, H, act_bits)
    packed = refmath.pack_int4_np(qw)
    if act_bits == 8:
        ref = oracle.exact_linear(qx.astype(np.int8), sx, packed, sw)
        mode, hdt = m.MOE_MODE_EXACT_I8, torch.int8
        h = torch.from_numpy(qx.astype(np.int8)).cuda()
    else:
        ref = oracle.exact_linear16(qx.astype(np.int16), sx, packed, sw)
        mode, hdt = m.MOE_MODE_EXACT_I16, torch.int16
        h = torch.from_numpy(qx.astype(np.int16)).cuda()
    assert np.any(ref == np.float32(2.0 ** 24 + 2))  # the fused step of group 1 survives
    W = {"wg": np.zeros((1, I, H // 2), np.uint8), "sg": _bf16(np.ones((1, I, H // 32))),
         "wu": np.zeros((1, I, H // 2), np.uint8), "su": _bf16(np.ones((1, I, H // 32))),
         "wd": packed[None], "sd": sw[None]}
    D = _dev_experts(W)
    offsets = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    m.moe_int4_grouped_down(mode, h, torch.from_numpy(sx).cuda(), D["wd"], D["sd"], offsets, T, 1, 1, I, H, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref)


def test_exact_linear_i8w_constructed_fold(m):
    say("exact linear i8w constructed fold")
    M, N, K = 40, 64, 128
    qw = np.zeros((N, K), np.int8)
    sw = np.ones((N, K // 32), np.float32)
    qx = np.zeros((M, K), np.int8)
    sx = np.zeros((M, K // 32), np.float32)
    for n in range(N):
        if n % 2 == 0:
            qw[n, 0:32] = 16
            sw[n, 0] = 2.0 ** 9
        qw[n, 32] = 1
        qw[n, 64] = 1
        qw[n, 96] = ASSOC_I8W[n % 3][0]
        sw[n, 3] = ASSOC_I8W[n % 3][2]
    for p in range(M):
        if p % 2 == 0:
            qx[p, 0:32] = 32
            sx[p, 0] = 2.0
        qx[p, 32], sx[p, 1] = (3, THIRD) if p % 4 < 2 else (1, 1.0)
        if p % 3:
            qx[p, 64], sx[p, 2] = 1, 1.0
        qx[p, 96], sx[p, 3] = ASSOC_I8W[p % 3][1], ASSOC_I8W[p % 3][3]
    ref = oracle.exact_linear_i8w(qx, sx, qw, sw)
    assert np.any(ref == np.float32(2.0 ** 24 + 2))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    m.moe_exact_linear_i8w(torch.from_numpy(qx).cuda(), torch.from_numpy(sx).cuda(), torch.from_numpy(qw).cuda(),
                           torch.from_numpy(sw).cuda(), y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref)


# ---------------------------------------------------------------- exact combine
def test_exact_combine_constructed_order(m):
    say("exact combine constructed order")
    T, k, H = 2, 3, 256
    y = np.zeros((T, k, H), np.float32)
    w = np.zeros((T, k), np.float32)
    y[0, :, :] = np.array([2.0 ** 24, 1.0, 1.0], np.float32)[:, None]
    w[0] = 1.0
    y[1, 0, :], y[1, 1, :] = 2.0 ** 24, 3.0
    w[1] = [1.0, THIRD, 0.0]
    ref = oracle.combine_f32(y, w)
    np.testing.assert_array_equal(ref, np.float32(2.0 ** 24))
    # slot rows stored in a shuffled order: slot_pos maps (t, j) to its row
    perm = np.array([4, 0, 5, 2, 1, 3], np.int32)
    rows = np.empty((T * k, H), np.float32)
    rows[perm] = y.reshape(T * k, H)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    m.moe_combine(m.MOE_MODE_EXACT_I8, torch.from_numpy(rows).cuda(), torch.from_numpy(perm).cuda(),
                  torch.from_numpy(w).cuda(), None, T, k, H, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


# ---------------------------------------------------------------- quantiser divisions
QDIV8 = [(144.0, 72.0), (112.5, 56.25), (38.0, 19.0), (72.0, 36.0), (39.25, -19.625), (28.125, 14.0625),
         (286.0, 1.0), (175.0, -3.0)]
QDIV16 = [(203.0, 101.5), (204.0, 102.0), (120.0, 60.0), (58.5, 29.25), (247.0, 123.5)]


@pytest.mark.parametrize("bits", [8, 16])
def test_quant_constructed_divisions(m, bits):
    say(f"quant constructed divisions bits={bits}")
    fx = QDIV8 if bits == 8 else QDIV16
    K = 128
    v = np.zeros((len(fx), K), np.float32)
    for i, (amax, xv) in enumerate(fx):
        v[i, 0], v[i, 1] = amax, xv
        v[i, 64], v[i, 65] = -amax, -xv   # a second group with the signs flipped
    x = _bf16(v)
    if bits == 8:
        rq, rs = oracle.quant_act_int8(x)
        q = torch.empty((len(fx), K), dtype=torch.int8, device="cuda")
        s = torch.empty((len(fx), K // 32), dtype=torch.float32, device="cuda")
        m.moe_quant_act_int8(bf16_dev(x), q, s)
    else:
        rq, rs = oracle.quant_act_int16(x)
        q = torch.empty((len(fx), K), dtype=torch.int16, device="cuda")
        s = torch.empty((len(fx), K // 32), dtype=torch.float32, device="cuda")
        m.moe_quant_act_int16(bf16_dev(x), q, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
