"""Per-kernel parity of the HIP path against the oracle, through the C ABI, on
seeded inputs that span several tiles and a ragged tail (GPU required)."""
import numpy as np
import pytest
import torch

import oracle
from tests import refmath
from tests.gpu_common import (assert_bf16_close, assert_f32_close, bf16_dev, bf16_to_f64, f16p_values, np_bf16,
                              say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_routed_expert_moe_amd import moe
    return moe


def _rand_bf16(g, shape, std=1.0):
    return refmath.bf16_from_f32((g.standard_normal(shape) * std).astype(np.float32))


_F16P_ORDER = np.array([0, 4, 1, 5, 2, 6, 3, 7])


def _f16p_ref(bits):
    """The fp16 staging format from its definition: bf16 -> fp16 rounding toward
    zero (saturating at the largest finite fp16), each 8-element block stored as
    e0,e4,e1,e5,e2,e6,e3,e7.  Returns fp16 bit patterns."""
    f = bf16_to_f64(bits)
    with np.errstate(over="ignore"):
        h = f.astype(np.float16)                   # nearest (values past the fp16 range become inf)
    over = np.abs(h.astype(np.float64)) > np.abs(f)  # rounded away from zero (or to inf)
    h[over] = np.nextafter(h[over], np.float16(0))
    h = h.reshape(*bits.shape[:-1], bits.shape[-1] // 8, 8)[..., _F16P_ORDER]
    return h.reshape(bits.shape).view(np.uint16)


def _packed(g, shape):
    return g.integers(0, 256, shape, dtype=np.uint8)


def _scales(g, shape):
    return refmath.bf16_from_f32(g.uniform(0.005, 0.02, shape).astype(np.float32))


# ---------------------------------------------------------------- routing
def test_route_token_chunks(m):
    """More tokens than one launch of the large-batch logits kernel takes (its
    token rows stay below 2 GiB, 149,760 tokens at 7168): tokens on both sides of
    the chunk boundary and in the ragged last tile match the oracle.  x comes
    from torch's seeded generator on the device; the sampled rows go back to the
    oracle."""
    H, E, k = 7168, 16, 2
    chunk = ((2 ** 31 - 1) // (H * 2)) // 64 * 64
    T = chunk + 137
    say(f"route token chunks T={T} H={H} E={E}")
    gen = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((T, H), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    g = np.random.default_rng(11)
    w = _rand_bf16(g, (E, H), 0.02)
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.moe_route_workspace_bytes(T, H, E), dtype=torch.uint8, device="cuda")
    m.moe_route(x, bf16_dev(w), torch.from_numpy(b).cuda(), k, True, idx, wt, ws)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([np.arange(0, 64), np.arange(chunk - 70, chunk + 70), np.arange(T - 80, T),
                                     g.integers(0, T, 64)]))
    xs = np_bf16(x[torch.from_numpy(toks).cuda()])
    del x
    ridx, rw = oracle.route(xs, w, b, k, True)
    np.testing.assert_array_equal(idx.cpu().numpy()[toks], ridx)
    np.testing.assert_array_equal(wt.cpu().numpy()[toks], rw)


@pytest.mark.parametrize("T,H,E,k,seed", [
    (1, 128, 16, 1, 0), (37, 256, 16, 2, 1), (64, 7168, 384, 8, 2), (300, 1024, 384, 8, 3),
    (130, 512, 1000, 16, 4), (64, 256, 8, 8, 5),
    # large-batch paths: up to 256 workgroups (64 tokens x 64 experts each) the
    # two-chain kernel (blocks in pairs), above it the one-chain kernel
    (300, 512, 100, 4, 6),      # two-chain, ragged last expert tile
    (8192, 128, 384, 8, 7),     # one-chain, two hidden blocks
    (300, 64, 50, 4, 8),        # two-chain, one hidden block, ragged tokens and experts
    (260, 320, 70, 6, 9),       # two-chain, five hidden blocks (a loop pass plus a single block)
    (400, 192, 64, 4, 12),      # two-chain, three hidden blocks (a pair plus a single block)
    (300, 448, 64, 4, 13),      # two-chain, seven hidden blocks (a loop pass, a pair and a single block)
    (17000, 320, 70, 6, 11),    # one-chain, five hidden blocks (loop plus both tail steps), ragged
    (2048, 7168, 384, 8, 10),   # two-chain at the full hidden size (192 workgroups)
])
def test_route_bitexact(m, T, H, E, k, seed):
    say(f"route T={T} H={H} E={E} k={k}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (T, H))
    w = _rand_bf16(g, (E, H), 0.02)
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    if E >= 8:  # exact ties: duplicated router rows with equal bias
        w[3] = w[1]
        w[5] = w[1]
        b[3] = b[1]
        b[5] = b[1]
    ridx, rw = oracle.route(x, w, b, k, True)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.moe_route_workspace_bytes(T, H, E), dtype=torch.uint8, device="cuda")
    m.moe_route(bf16_dev(x), bf16_dev(w), torch.from_numpy(b).cuda(), k, True, idx, wt, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_array_equal(wt.cpu().numpy(), rw)
    # renormalisation off
    ridx2, rw2 = oracle.route(x, w, b, k, False)
    m.moe_route(bf16_dev(x), bf16_dev(w), torch.from_numpy(b).cuda(), k, False, idx, wt, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx2)
    np.testing.assert_array_equal(wt.cpu().numpy(), rw2)


@pytest.mark.parametrize("T,H,E,k,n_group,topk_group,scale,seed", [
    (64, 7168, 384, 8, 8, 4, 2.5, 0),   # decode shape, small-batch logits path
    (300, 512, 384, 8, 8, 4, 1.0, 1),   # large-batch path
    (37, 256, 64, 6, 4, 2, 1.0, 2),
    (50, 256, 96, 4, 48, 3, 0.75, 3),   # groups of two experts
    (40, 256, 64, 5, 1, 1, 1.0, 4),     # one group: plain routing
])
def test_route_grouped_bitexact(m, T, H, E, k, n_group, topk_group, scale, seed):
    say(f"route grouped T={T} H={H} E={E} k={k} groups {topk_group}/{n_group}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (T, H))
    w = _rand_bf16(g, (E, H), 0.02)
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    # exact ties: duplicated router rows with equal bias, across two groups
    w[E // 2 + 1] = w[1]
    b[E // 2 + 1] = b[1]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.moe_route_workspace_bytes(T, H, E), dtype=torch.uint8, device="cuda")
    for renorm in (True, False):
        ridx, rw = oracle.route_grouped(x, w, b, k, n_group, topk_group, renorm, scale)
        m.moe_route_grouped(bf16_dev(x), bf16_dev(w), torch.from_numpy(b).cuda(), k, renorm, n_group, topk_group,
                            scale, idx, wt, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
        np.testing.assert_array_equal(wt.cpu().numpy(), rw)


def test_sigmoid_matches_oracle_on_a_sweep(m):
    """Route with one expert row per logit value: the selected weight (renormalise
    off, k=E) is the sigmoid of that logit, bit for bit."""
    say("sigmoid sweep")
    H, E = 128, 16
    vals = np.linspace(-90, 90, 16 * 389, dtype=np.float32)
    # logit = x[0] * w[e,0] with x = (1, 0, ...): w[e,0] carries the value (bf16-rounded)
    wv = refmath.bf16_from_f32(vals)
    T = 1
    for c in range(0, len(wv), E):
        w = np.zeros((E, H), np.uint16)
        w[:, 0] = wv[c:c + E]
        x = np.zeros((T, H), np.uint16)
        x[0, 0] = 0x3F80
        b = np.zeros(E, np.float32)
        ridx, rw = oracle.route(x, w, b, E, False)
        idx = torch.empty((T, E), dtype=torch.int32, device="cuda")
        wt = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ws = torch.empty(m.moe_route_workspace_bytes(T, H, E), dtype=torch.uint8, device="cuda")
        m.moe_route(bf16_dev(x), bf16_dev(w), torch.from_numpy(b).cuda(), E, False, idx, wt, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
        np.testing.assert_array_equal(wt.cpu().numpy(), rw)


# ---------------------------------------------------------------- permutation
@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (64, 2, 16, 1), (64, 8, 384, 2),
                                        (8192, 8, 384, 3),     # blocks of 1024 slots
                                        (1000, 16, 1024, 4),   # 16000 slots: largest one-workgroup case
                                        (77, 3, 5, 5),
                                        (2048, 8, 1024, 6),    # 16384 slots: first multi-block case, largest E
                                        (3001, 7, 5, 7),       # multi-block, ragged last block, few experts
                                        (16384, 1, 1, 8)])     # multi-block, one expert
def test_permute_bitexact(m, T, k, E, seed):
    say(f"permute T={T} k={k} E={E}")
    g = np.random.default_rng(seed)
    idx = g.integers(0, E, (T, k)).astype(np.int32)
    if E > 4:
        idx[idx == 2] = 3  # an empty expert
    rc, ro, rs, rp = oracle.permute(idx, E)
    S = T * k
    d = {n: torch.empty(s, dtype=torch.int32, device="cuda") for n, s in
         (("counts", E), ("offsets", E + 1), ("ss", S), ("sp", S))}
    ws = torch.empty(max(1, m.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device="cuda")
    m.moe_permute(torch.from_numpy(idx).cuda(), E, d["counts"], d["offsets"], d["ss"], d["sp"], ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d["counts"].cpu().numpy(), rc)
    np.testing.assert_array_equal(d["offsets"].cpu().numpy(), ro)
    np.testing.assert_array_equal(d["ss"].cpu().numpy(), rs)
    np.testing.assert_array_equal(d["sp"].cpu().numpy(), rp)


def test_permute_bitexact_skewed(m):
    """Multi-block path with one expert holding most slots and most experts empty."""
    T, k, E = 2600, 8, 256
    say(f"permute skewed T={T} k={k} E={E}")
    g = np.random.default_rng(11)
    idx = np.where(g.random((T, k)) < 0.9, 7, g.integers(0, 20, (T, k))).astype(np.int32)
    rc, ro, rs, rp = oracle.permute(idx, E)
    S = T * k
    d = {n: torch.empty(s, dtype=torch.int32, device="cuda") for n, s in
         (("counts", E), ("offsets", E + 1), ("ss", S), ("sp", S))}
    ws = torch.empty(max(1, m.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 1  # the multi-block path
    m.moe_permute(torch.from_numpy(idx).cuda(), E, d["counts"], d["offsets"], d["ss"], d["sp"], ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d["counts"].cpu().numpy(), rc)
    np.testing.assert_array_equal(d["offsets"].cpu().numpy(), ro)
    np.testing.assert_array_equal(d["ss"].cpu().numpy(), rs)
    np.testing.assert_array_equal(d["sp"].cpu().numpy(), rp)


# ---------------------------------------------------------------- exact-mode primitives
@pytest.mark.parametrize("M,K,seed", [(1, 32, 0), (37, 256, 1), (64, 7168, 2)])
def test_quant_act_bitexact(m, M, K, seed):
    say(f"quant M={M} K={K}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (M, K))
    x[0, :32] = 0  # a zero group
    if K >= 64:
        x[0, 32:64] = refmath.bf16_from_f32(np.array([127.0, 2.5, -2.5, 3.5] + [0.0] * 28, np.float32))
    rq, rs = oracle.quant_act_int8(x)
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
    m.moe_quant_act_int8(bf16_dev(x), q, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("M,K,seed", [(1, 32, 0), (37, 256, 1), (64, 7168, 2)])
def test_quant_act16_bitexact(m, M, K, seed):
    say(f"quant16 M={M} K={K}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (M, K))
    x[0, :32] = 0  # a zero group
    rq, rs = oracle.quant_act_int16(x)
    q = torch.empty((M, K), dtype=torch.int16, device="cuda")
    s = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
    m.moe_quant_act_int16(bf16_dev(x), q, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("M,N,K,seed", [(16, 16, 32, 0), (48, 32, 7168, 1), (16, 64, 2048, 2)])
def test_group_sums_bitexact(m, M, N, K, seed):
    say(f"group sums M={M} N={N} K={K}")
    g = np.random.default_rng(seed)
    qx = g.integers(-127, 128, (M, K)).astype(np.int8)
    qx[0, :32] = 127
    packed = _packed(g, (N, K // 2))
    packed[0, :16] = 0x88
    ref = oracle.group_sums(qx, packed, K)
    G = torch.empty((M, N, K // 32), dtype=torch.int32, device="cuda")
    m.moe_int4_group_sums_i32(torch.from_numpy(qx).cuda(), torch.from_numpy(packed).cuda(), G)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.cpu().numpy(), ref)
    assert int(G[0, 0, 0]) == -32512


# ---------------------------------------------------------------- grouped expert GEMMs
def _expert_set(g, E, H, I):
    return {"wg": _packed(g, (E, I, H // 2)), "sg": _scales(g, (E, I, H // 32)),
            "wu": _packed(g, (E, I, H // 2)), "su": _scales(g, (E, I, H // 32)),
            "wd": _packed(g, (E, H, I // 2)), "sd": _scales(g, (E, H, I // 32))}


def _dev_experts(W):
    """Upload in the checkpoint layout and permute into the layout the grouped GEMMs read."""
    from int4_routed_expert_moe_amd.layer import prepack_experts
    out = {}
    for n in ("wg", "wu", "wd"):
        out[n] = torch.from_numpy(W[n]).cuda()
    for n in ("sg", "su", "sd"):
        out[n] = bf16_dev(W[n])
    return prepack_experts(out)


def _prepacked_ref(packed, scale):
    """The fragment layout written out with numpy index arithmetic (row group R, chunk c,
    lane l = r + 16 j, group g): the reading of the header's definition."""
    E, N, K2 = packed.shape
    K = 2 * K2
    nch = K // 128
    # packed[e, 16 R + r, 64 c + 16 g + 4 j + b] -> out[e, R, c, j, r, g, b]
    w = packed.reshape(E, N // 16, 16, nch, 4, 4, 4)          # e, R, r, c, g, j, b
    w = w.transpose(0, 1, 3, 5, 2, 4, 6)                      # e, R, c, j, r, g, b
    s = scale.reshape(E, N // 16, 16, nch, 4).transpose(0, 1, 3, 2, 4)  # e, R, c, r, g
    return np.ascontiguousarray(w).reshape(E, N, K2), np.ascontiguousarray(s).reshape(E, N, K // 32)


@pytest.mark.parametrize("E,N,K,seed", [(3, 48, 256, 0), (2, 16, 128, 1), (1, 256, 7168, 2), (0, 32, 128, 3)])
def test_prepack_layout_bitexact(m, E, N, K, seed):
    say(f"prepack E={E} N={N} K={K}")
    g = np.random.default_rng(seed)
    packed = _packed(g, (E, N, K // 2))
    scale = g.integers(0, 1 << 16, (E, N, K // 32), dtype=np.uint16)
    pw = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    ps = torch.empty((E, N, K // 32), dtype=torch.float16, device="cuda")
    m.moe_int4_prepack(torch.from_numpy(packed).cuda(), bf16_dev(scale), pw, ps)
    torch.cuda.synchronize()
    rw, rs = _prepacked_ref(packed, scale)
    np.testing.assert_array_equal(pw.cpu().numpy(), rw)
    # scales as fp16 (numpy's float32 -> float16 rounds to nearest even, subnormals and
    # overflow included); NaNs compare as NaNs
    with np.errstate(over="ignore"):
        want = refmath.bf16_to_f32(rs).astype(np.float16)
    got = ps.cpu().numpy()
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint16), want[~nan].view(np.uint16))


def _routing(g, T, E, k, skew=False):
    if skew:  # heavy head + empty experts
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.5
        p[E // 2:] = 0
        p /= p.sum()
    else:
        p = np.full(E, 1.0 / E)
    idx = np.stack([g.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.3, (T, k)).astype(np.float32)
    return idx, w


@pytest.mark.parametrize("T,H,I,E,k,skew,seed", [
    (64, 256, 128, 16, 2, False, 0),     # tiny workload shape
    (37, 512, 256, 8, 3, False, 1),      # ragged tail, one tile per expert
    (300, 256, 128, 4, 2, True, 2),      # many rows per expert (several tiles) and empty experts
    (700, 512, 256, 6, 2, False, 3),     # largest tile height
    (280, 256, 128, 8, 2, False, 4),     # 6-block tiles
    (400, 512, 256, 8, 2, True, 5),      # 8-block tiles, skewed
    (700, 256, 128, 6, 2, False, 6),     # 32x32 tiles over 2 K chunks (gate/up) and 1 (down)
    # K chunk counts against the staged 32x32 kernel's three-chunk loop and its tails:
    (700, 1024, 512, 6, 2, False, 7),    # gate/up over 8 K chunks, down over 4
    (500, 1536, 384, 5, 2, True, 8),     # gate/up over 12 K chunks, down over 3 (skewed)
    (700, 1280, 512, 6, 2, False, 9),    # gate/up over 10 K chunks, down over 4
    (200, 512, 256, 8, 2, False, 10),    # mid-size segments (about 50 rows): tiles of 3 row blocks, split segments
    (150, 768, 384, 6, 2, True, 11),     # the same, skewed (one long segment, empty experts)
    (100, 256, 128, 32, 12, False, 12),  # k = 12: the 16-slot combine
])
def test_grouped_bf16(m, T, H, I, E, k, skew, seed):
    say(f"grouped bf16 T={T} H={H} I={I} E={E} k={k}")
    g = np.random.default_rng(seed)
    W = _expert_set(g, E, H, I)
    x = _rand_bf16(g, (T, H))
    idx, w = _routing(g, T, E, k, skew)
    counts, offsets, ss, sp = oracle.permute(idx, E)
    S = T * k
    rows = x[ss // k]
    ref = oracle.experts_bf16(rows, idx.reshape(-1)[ss], W, want=("h", "y"))
    D = _dev_experts(W)
    off_d = torch.from_numpy(offsets).cuda()
    h = torch.empty((S, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((S, H), dtype=torch.bfloat16, device="cuda")
    m.moe_int4_grouped_swiglu(m.MOE_MODE_BF16, bf16_dev(x), None, D["wg"], D["sg"], D["wu"], D["su"], off_d,
                              torch.from_numpy(ss).cuda(), T, k, E, H, I, h, None)
    # down on the oracle's h so the two stages are checked separately
    m.moe_int4_grouped_down(m.MOE_MODE_BF16, bf16_dev(ref["h"]), None, D["wd"], D["sd"], off_d, T, k, E, I, H, y)
    torch.cuda.synchronize()
    assert_bf16_close(np_bf16(h), ref["h"], "h")
    assert_bf16_close(np_bf16(y), ref["y"], "y")
    # the fp16 staging-format mode: against the oracle, and bit-identical to the bf16 mode
    say(f"grouped bf16 (fp16 staging format) T={T} H={H} I={I} E={E} k={k}")
    xp = torch.empty((T, H), dtype=torch.float16, device="cuda")
    m.moe_act_f16p(bf16_dev(x), xp)
    h2 = torch.empty((S, I), dtype=torch.float16, device="cuda")
    m.moe_int4_grouped_swiglu(m.MOE_MODE_BF16_F16P, xp, None, D["wg"], D["sg"], D["wu"], D["su"], off_d,
                              torch.from_numpy(ss).cuda(), T, k, E, H, I, h2, None)
    hp_ref = torch.empty((S, I), dtype=torch.float16, device="cuda")
    m.moe_act_f16p(bf16_dev(ref["h"]), hp_ref)
    y2 = torch.empty((S, H), dtype=torch.bfloat16, device="cuda")
    m.moe_int4_grouped_down(m.MOE_MODE_BF16_F16P, hp_ref, None, D["wd"], D["sd"], off_d, T, k, E, I, H, y2)
    torch.cuda.synchronize()
    h2_bits = h2.view(torch.int16).cpu().numpy().view(np.uint16)
    got_h = f16p_values(h2_bits)
    ref_h = bf16_to_f64(ref["h"])
    scale = np.sqrt(np.mean(ref_h ** 2)) + 1e-30
    assert np.all(np.abs(got_h - ref_h) <= 1e-2 * scale + 2e-2 * np.abs(ref_h)), "h (staging format)"
    np.testing.assert_array_equal(h2_bits, _f16p_ref(np_bf16(h)))
    assert_bf16_close(np_bf16(y2), ref["y"], "y (staging format)")
    np.testing.assert_array_equal(np_bf16(y2), np_bf16(y))
    # combine on the GPU's y vs the oracle combine of the same y
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    shared = _rand_bf16(g, (T, H))
    m.moe_combine(m.MOE_MODE_BF16, y, torch.from_numpy(sp).cuda(), torch.from_numpy(w).cuda(), bf16_dev(shared),
                  T, k, H, out)
    torch.cuda.synchronize()
    y_np = np_bf16(y)
    ref_out = oracle.combine_bf16(y_np[sp].reshape(T, k, H), w, shared)
    routed = oracle.combine_bf16(y_np[sp].reshape(T, k, H), w, None)  # bf16(sum) before the shared add
    assert_bf16_close(np_bf16(out), ref_out, "combine", atol_rms=1e-3, rtol=8e-3, addends=(routed, shared))


@pytest.mark.parametrize("T,H,I,E,k,skew,seed", [
    (64, 256, 128, 16, 2, False, 0),
    (300, 256, 128, 4, 2, True, 1),
    (45, 512, 256, 5, 3, False, 2),
    (280, 256, 128, 8, 2, False, 3),     # 6-block tiles
    (400, 512, 256, 8, 2, False, 4),     # 8-block tiles
    (64, 1280, 640, 64, 8, False, 5),    # decode kernel: 8-row segments, 10 / 5 chunks through its ring
    (48, 1024, 896, 32, 8, False, 6),    # decode kernel: 12-row segments, 8 / 7 chunks
    (64, 256, 128, 32, 16, False, 7),    # k = 16 (the largest): the 16-slot combine
])
def test_grouped_exact_bitexact(m, T, H, I, E, k, skew, seed):
    say(f"grouped exact T={T} H={H} I={I} E={E} k={k}")
    g = np.random.default_rng(seed)
    W = _expert_set(g, E, H, I)
    x = _rand_bf16(g, (T, H))
    idx, w = _routing(g, T, E, k, skew)
    counts, offsets, ss, sp = oracle.permute(idx, E)
    S = T * k
    qx, sx = oracle.quant_act_int8(x)
    ref = oracle.experts_exact(qx[ss // k], sx[ss // k], idx.reshape(-1)[ss], W, want=("g", "u", "qh", "sh", "y"))
    D = _dev_experts(W)
    off_d = torch.from_numpy(offsets).cuda()
    qh = torch.empty((S, I), dtype=torch.int8, device="cuda")
    sh = torch.empty((S, I // 32), dtype=torch.float32, device="cuda")
    y = torch.empty((S, H), dtype=torch.float32, device="cuda")
    m.moe_int4_grouped_swiglu(m.MOE_MODE_EXACT_I8, torch.from_numpy(qx).cuda(), torch.from_numpy(sx).cuda(),
                              D["wg"], D["sg"], D["wu"], D["su"], off_d, torch.from_numpy(ss).cuda(), T, k, E, H, I,
                              qh, sh)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sh.cpu().numpy(), ref["sh"])
    np.testing.assert_array_equal(qh.cpu().numpy(), ref["qh"])
    m.moe_int4_grouped_down(m.MOE_MODE_EXACT_I8, qh, sh, D["wd"], D["sd"], off_d, T, k, E, I, H, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref["y"])
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    m.moe_combine(m.MOE_MODE_EXACT_I8, y, torch.from_numpy(sp).cuda(), torch.from_numpy(w).cuda(), None, T, k, H, out)
    torch.cuda.synchronize()
    ref_out = oracle.combine_f32(ref["y"][sp].reshape(T, k, H), w)
    np.testing.assert_array_equal(out.cpu().numpy(), ref_out)


@pytest.mark.parametrize("mode_name", ["bf16", "exact"])
def test_grouped_decode_kernel_odd_chunk_counts(m, mode_name):
    """The decode kernel's weight ring over odd chunk counts: gate/up over 9 chunks of
    128 (H = 1152), down over 5 (I = 640), with segments of about 8 rows."""
    say(f"grouped decode kernel odd chunks mode={mode_name}")
    g = np.random.default_rng(31)
    T, E, k = 64, 64, 8
    idx, _ = _routing(g, T, E, k)
    counts, offsets, ss, sp = oracle.permute(idx, E)
    off_d = torch.from_numpy(offsets).cuda()
    S = T * k
    # gate/up: H = 1152, I = 256
    H, I = 1152, 256
    W = _expert_set(g, E, H, I)
    D = _dev_experts(W)
    x = _rand_bf16(g, (T, H))
    if mode_name == "bf16":
        ref = oracle.experts_bf16(x[ss // k], idx.reshape(-1)[ss], W, want=("h",))
        h = torch.empty((S, I), dtype=torch.bfloat16, device="cuda")
        m.moe_int4_grouped_swiglu(m.MOE_MODE_BF16, bf16_dev(x), None, D["wg"], D["sg"], D["wu"], D["su"], off_d,
                                  torch.from_numpy(ss).cuda(), T, k, E, H, I, h, None)
        torch.cuda.synchronize()
        assert_bf16_close(np_bf16(h), ref["h"], "h")
    else:
        qx, sx = oracle.quant_act_int8(x)
        ref = oracle.experts_exact(qx[ss // k], sx[ss // k], idx.reshape(-1)[ss], W, want=("qh", "sh"))
        qh = torch.empty((S, I), dtype=torch.int8, device="cuda")
        sh = torch.empty((S, I // 32), dtype=torch.float32, device="cuda")
        m.moe_int4_grouped_swiglu(m.MOE_MODE_EXACT_I8, torch.from_numpy(qx).cuda(), torch.from_numpy(sx).cuda(),
                                  D["wg"], D["sg"], D["wu"], D["su"], off_d, torch.from_numpy(ss).cuda(), T, k, E,
                                  H, I, qh, sh)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(sh.cpu().numpy(), ref["sh"])
        np.testing.assert_array_equal(qh.cpu().numpy(), ref["qh"])
    # down: I = 640, H = 256, fed the oracle's h of a second expert set
    H, I = 256, 640
    W = _expert_set(g, E, H, I)
    D = _dev_experts(W)
    x = _rand_bf16(g, (T, H))
    rows_e = idx.reshape(-1)[ss]
    if mode_name == "bf16":
        ref = oracle.experts_bf16(x[ss // k], rows_e, W, want=("h", "y"))
        y = torch.empty((S, H), dtype=torch.bfloat16, device="cuda")
        m.moe_int4_grouped_down(m.MOE_MODE_BF16, bf16_dev(ref["h"]), None, D["wd"], D["sd"], off_d, T, k, E, I, H, y)
        torch.cuda.synchronize()
        assert_bf16_close(np_bf16(y), ref["y"], "y")
    else:
        qx, sx = oracle.quant_act_int8(x)
        ref = oracle.experts_exact(qx[ss // k], sx[ss // k], rows_e, W, want=("qh", "sh", "y"))
        y = torch.empty((S, H), dtype=torch.float32, device="cuda")
        m.moe_int4_grouped_down(m.MOE_MODE_EXACT_I8, torch.from_numpy(ref["qh"]).cuda(),
                                torch.from_numpy(ref["sh"]).cuda(), D["wd"], D["sd"], off_d, T, k, E, I, H, y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref["y"])


@pytest.mark.parametrize("rows,K,seed", [(1, 8, 0), (37, 7168, 1), (300, 2048, 2)])
def test_act_f16p_layout(m, rows, K, seed):
    """The staging conversion against its definition, bit for bit, with values
    below the fp16 normal range, above its largest finite value, and signed zeros."""
    say(f"act_f16p rows={rows} K={K}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (rows, K), std=4.0)
    flat = x.reshape(-1)
    special = refmath.bf16_from_f32(np.array([1e-6, -3e-5, 7e4, -1e6, 0.0, -0.0, 65504.0, 2.0 ** -14],
                                             dtype=np.float32))
    flat[: min(flat.size, special.size)] = special[: min(flat.size, special.size)]
    out = torch.empty((rows, K), dtype=torch.float16, device="cuda")
    m.moe_act_f16p(bf16_dev(x), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), _f16p_ref(x))


@pytest.mark.parametrize("T,H,I,E,k,skew,seed", [
    (64, 256, 128, 16, 2, False, 0),
    (300, 256, 128, 4, 2, True, 1),      # several tiles per expert, empty experts
    (45, 512, 256, 5, 3, False, 2),      # ragged tiles
    (200, 512, 256, 8, 2, False, 3),
])
def test_grouped_exact16_bitexact(m, T, H, I, E, k, skew, seed):
    """Exact mode with 16-bit activation codes: q_h, s_h and y bit-exact."""
    say(f"grouped exact16 T={T} H={H} I={I} E={E} k={k}")
    g = np.random.default_rng(seed)
    W = _expert_set(g, E, H, I)
    x = _rand_bf16(g, (T, H))
    idx, w = _routing(g, T, E, k, skew)
    counts, offsets, ss, sp = oracle.permute(idx, E)
    S = T * k
    qx, sx = oracle.quant_act_int16(x)
    ref = oracle.experts_exact16(qx[ss // k], sx[ss // k], idx.reshape(-1)[ss], W, want=("qh", "sh", "y"))
    D = _dev_experts(W)
    off_d = torch.from_numpy(offsets).cuda()
    qh = torch.empty((S, I), dtype=torch.int16, device="cuda")
    sh = torch.empty((S, I // 32), dtype=torch.float32, device="cuda")
    y = torch.empty((S, H), dtype=torch.float32, device="cuda")
    m.moe_int4_grouped_swiglu(m.MOE_MODE_EXACT_I16, torch.from_numpy(qx).cuda(), torch.from_numpy(sx).cuda(),
                              D["wg"], D["sg"], D["wu"], D["su"], off_d, torch.from_numpy(ss).cuda(), T, k, E, H, I,
                              qh, sh)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sh.cpu().numpy(), ref["sh"])
    np.testing.assert_array_equal(qh.cpu().numpy(), ref["qh"])
    m.moe_int4_grouped_down(m.MOE_MODE_EXACT_I16, qh, sh, D["wd"], D["sd"], off_d, T, k, E, I, H, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref["y"])


@pytest.mark.parametrize("M,N,K,seed", [(64, 64, 128, 0), (100, 200, 512, 1), (37, 96, 7168, 2),
                                        (256, 2048, 256, 3)])
def test_exact_linear_i8w_bitexact(m, M, N, K, seed):
    """ExactLinear with 8-bit weights (both operands quantised on the GPU) against the oracle, bit for bit."""
    say(f"exact linear i8w M={M} N={N} K={K}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (M, K))
    w = _rand_bf16(g, (N, K), 0.02)
    qx, sx = oracle.quant_act_int8(x)
    qw, sw = oracle.quant_act_int8(w)
    ref = oracle.exact_linear_i8w(qx, sx, qw, sw)
    dqx = torch.empty((M, K), dtype=torch.int8, device="cuda")
    dsx = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
    dqw = torch.empty((N, K), dtype=torch.int8, device="cuda")
    dsw = torch.empty((N, K // 32), dtype=torch.float32, device="cuda")
    m.moe_quant_act_int8(bf16_dev(x), dqx, dsx)
    m.moe_quant_act_int8(bf16_dev(w), dqw, dsw)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    m.moe_exact_linear_i8w(dqx, dsx, dqw, dsw, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dqw.cpu().numpy(), qw)
    np.testing.assert_array_equal(y.cpu().numpy(), ref)


# ---------------------------------------------------------------- dense pieces
@pytest.mark.parametrize("M,N,K,with_add,seed", [
    (1, 64, 128, False, 0), (64, 2048, 7168, False, 1), (40, 192, 512, True, 2), (200, 256, 384, True, 3),
    (700, 512, 256, False, 4),
    (300, 320, 384, True, 5),       # 32x32 tiles: ragged rows and a part-filled column chunk
    (4100, 4096, 128, True, 6),     # 32x32 tiles, many row tiles, ragged rows
    (6200, 320, 384, True, 7),      # 192-row 32x32 tiles: ragged rows and a part-filled column chunk
    (255, 192, 256, False, 8),      # last row count of the 16x16 kernel
    (256, 192, 256, True, 9),       # first row count of the 32x32 kernel (two whole 128-row tiles)
    (6144, 64, 128, False, 10),     # first row count of the 192-row tiles (32 whole tiles)
    (16, 512, 2048, False, 11),     # split K, 16-row tiles
    (30, 320, 1024, True, 12),      # split K, 32-row tiles, ragged rows and columns
    (50, 128, 2560, True, 13),      # split K into splits of 2 and 3 chunks
    (130, 320, 256, True, 14),      # 16x16 tiles unsplit with an addend: ragged rows and columns
    (2000, 6464, 384, True, 15),    # 256-row tiles: ragged rows, a part-filled column chunk, odd chunk count
    (1800, 7168, 256, False, 16),   # 256-row tiles, no addend
])
def test_linear_bf16(m, M, N, K, with_add, seed):
    say(f"linear M={M} N={N} K={K}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (M, K))
    w = _rand_bf16(g, (N, K), 1.0 / np.sqrt(K))
    add = _rand_bf16(g, (M, N)) if with_add else None
    ref = oracle.linear_bf16(x, w, add)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    nb = m.moe_dense_workspace_bytes(M, N, K)
    ws = torch.empty(max(1, nb), dtype=torch.uint8, device="cuda")
    m.moe_linear_bf16(bf16_dev(x), bf16_dev(w), None if add is None else bf16_dev(add), y, ws)
    torch.cuda.synchronize()
    assert_bf16_close(np_bf16(y), ref, "linear")


@pytest.mark.parametrize("M,H,I,seed", [(64, 256, 128, 0), (64, 7168, 2048, 1), (130, 512, 192, 2),
                                        (300, 256, 192, 3),     # 32x32 tiles, ragged rows and columns
                                        (4096, 128, 2048, 4),   # 32x32 tiles, many row tiles
                                        (6150, 256, 192, 5),    # 192-row tiles, ragged rows and columns
                                        (2000, 384, 3264, 6)])  # 256-row tiles, ragged rows and columns
def test_dense_swiglu_and_silu_mul(m, M, H, I, seed):
    say(f"dense swiglu M={M} H={H} I={I}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (M, H))
    wg = _rand_bf16(g, (I, H), 1.0 / np.sqrt(H))
    wu = _rand_bf16(g, (I, H), 1.0 / np.sqrt(H))
    wd = _rand_bf16(g, (H, I), 1.0 / np.sqrt(I))
    ref_h, _ = oracle.dense_swiglu_bf16(x, wg, wu, wd, want_h=True)
    h = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, m.moe_dense_workspace_bytes(M, 2 * I, H)), dtype=torch.uint8, device="cuda")
    m.moe_dense_swiglu_bf16(bf16_dev(x), bf16_dev(wg), bf16_dev(wu), h, ws)
    torch.cuda.synchronize()
    assert_bf16_close(np_bf16(h), ref_h, "dense swiglu h")
    # elementwise silu*mul against the oracle's rounding chain on given g, u
    gg = _rand_bf16(g, (M, I), 3.0)
    uu = _rand_bf16(g, (M, I), 3.0)
    hh = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    m.moe_silu_mul_bf16(bf16_dev(gg), bf16_dev(uu), hh)
    torch.cuda.synchronize()
    ref = oracle.silu_mul_bf16(gg, uu)
    # the GPU's SiLU is the pinned fp32 one, the oracle's fp64: at most one bf16 step apart, rarely
    diff = np.abs(np_bf16(hh).astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 0.01
    assert_bf16_close(np_bf16(hh), ref, "silu_mul")


@pytest.mark.parametrize("M,N,seed", [(1, 3584, 0), (70, 3584, 1), (5, 256, 2)])
def test_rmsnorm(m, M, N, seed):
    say(f"rmsnorm M={M} N={N}")
    g = np.random.default_rng(seed)
    x = _rand_bf16(g, (M, N), 2.0)
    x[0] = refmath.bf16_from_f32(np.full(N, 0.75, np.float32))
    gain = refmath.bf16_from_f32(g.uniform(0.9, 1.1, N).astype(np.float32))
    ref = oracle.rmsnorm_bf16(x, gain, 1e-6)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    m.moe_rmsnorm_bf16(bf16_dev(x), bf16_dev(gain), 1e-6, y)
    torch.cuda.synchronize()
    got = np_bf16(y)
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1, "rmsnorm differs by more than one bf16 step"
    np.testing.assert_array_equal(got[0], ref[0])


def test_check_scales(m):
    """The load-time scale check: zeros and magnitudes in [2^-14, 2^9] pass; the first
    values outside (either side), NaN and infinity are counted."""
    say("check scales")
    good = np.array([0.0, -0.0, 2.0 ** -14, -(2.0 ** -14), 2.0 ** 9, -(2.0 ** 9), 0.01, 300.0], np.float32)
    bad = np.array([2.0 ** 9 * (1 + 2.0 ** -7), 2.0 ** -15, -(2.0 ** 10), np.inf, -np.inf, np.nan], np.float32)
    g = np.random.default_rng(0)
    base = refmath.bf16_from_f32(g.uniform(0.005, 0.02, 100000).astype(np.float32))
    ok = np.concatenate([base, refmath.bf16_from_f32(good)])
    m.moe_int4_check_scales(bf16_dev(ok))
    for i in range(len(bad)):
        arr = ok.copy()
        pos = g.integers(0, len(arr), 1 + i)
        arr[pos] = refmath.bf16_from_f32(np.full(len(pos), bad[i], np.float32))
        with pytest.raises(m.MoEError) as ei:
            m.moe_int4_check_scales(bf16_dev(arr))
        assert ei.value.status == m.MOE_ERR_UNSUPPORTED
        assert f" {len(np.unique(pos))} of {len(arr)} " in str(ei.value)
