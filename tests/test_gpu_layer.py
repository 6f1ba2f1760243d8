"""End-to-end parity of the whole layer (route -> permute -> experts -> combine,
+ shared expert, + latent wrapper, + exact mode) on the five workloads, at
their full sizes, in the launch configuration the benchmark times.

Routing and the permutation are compared on every token; expert outputs on
all tokens where the oracle finishes in seconds, otherwise on a seeded token
sample (the layer is token-independent after routing)."""
import numpy as np
import pytest
import torch

import oracle
from int4_routed_expert_moe_amd import synthetic
from tests.gpu_common import (act_bits_bf16, assert_bf16_close, assert_f32_close, bf16_dev, inputs, layer, np_bf16,
                              say)

pytestmark = pytest.mark.gpu

SAMPLE = {1: None, 2: None, 3: 128, 4: 128, 5: 128}


def _sample_tokens(cfg, ridx, n):
    """n tokens: the seeded sample, plus the tokens of the hottest expert's sorted rows on
    both sides of every boundary of balanced tiles of 16 to 192 rows (the first and last
    rows of the grouped kernels' tiles, whichever height they chose)."""
    T, k, E = cfg["T"], cfg["k"], cfg["E"]
    counts, offsets, ss, _ = oracle.permute(ridx, E)
    e = int(np.argmax(counts))
    cnt, off = int(counts[e]), int(offsets[e])
    pos = {off, off + cnt - 1}
    for bm in (16, 32, 48, 64, 96, 128, 192):
        nt = -(-cnt // bm)
        rpt = -(-cnt // nt)
        for t in range(1, min(nt, 4)):
            pos.update({off + t * rpt - 1, off + t * rpt})
    edge = {int(ss[p]) // k for p in pos if off <= p < off + cnt}
    rest = synthetic.token_sample(cfg, max(0, n - len(edge)))
    return np.array(sorted(edge | set(int(t) for t in rest)), dtype=np.int64)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(cfg_id):
    inp = inputs(cfg_id)
    L = layer(cfg_id)
    x = bf16_dev(inp["x"])
    say(f"layer forward workload {cfg_id} ({inp['cfg']['name']}) T={inp['cfg']['T']}")
    out = L.forward(x)
    torch.cuda.synchronize()
    return inp, L, x, out


@pytest.mark.parametrize("cfg_id", [1, 2, 5, 3, 4])
def test_layer_parity(cfg_id):
    inp, L, x, out = _run(cfg_id)
    cfg = inp["cfg"]
    T, k, E = cfg["T"], cfg["k"], cfg["E"]
    ws = L.workspace(T)
    # routing: bit-exact on every token
    ridx, rw = oracle.route(inp["x"], inp["router_w"], inp["router_b"], k, True)
    np.testing.assert_array_equal(ws["topk_idx"].cpu().numpy(), ridx)
    np.testing.assert_array_equal(ws["topk_w"].cpu().numpy(), rw)
    # permutation: bit-exact
    rc, ro, rs, rp = oracle.permute(ridx, E)
    np.testing.assert_array_equal(ws["counts"].cpu().numpy(), rc)
    np.testing.assert_array_equal(ws["offsets"].cpu().numpy(), ro)
    np.testing.assert_array_equal(ws["sorted_slot"].cpu().numpy(), rs)
    np.testing.assert_array_equal(ws["slot_pos"].cpu().numpy(), rp)
    if cfg.get("zipf"):
        dead = inp["router_b"] == np.float32(-4.0)
        assert rc[dead].sum() == 0 and dead.sum() == round(0.2 * E)
    # outputs on all tokens or a sample
    n = SAMPLE[cfg_id]
    toks = np.arange(T) if n is None else _sample_tokens(cfg, ridx, n)
    say(f"oracle on {len(toks)} tokens of workload {cfg_id}")
    ref, inter = oracle.layer_tokens(inp, toks, topk_idx=ridx, topk_w=rw, want_intermediates=True)
    slots = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    pos = rp[slots]
    if cfg["mode"] == "exact":
        np.testing.assert_array_equal(ws["qx"].cpu().numpy()[toks], inter["qx"])
        np.testing.assert_array_equal(ws["sx"].cpu().numpy()[toks], inter["sx"])
        np.testing.assert_array_equal(ws["h_scale"].cpu().numpy()[pos], inter["sh"])
        np.testing.assert_array_equal(ws["h"].cpu().numpy()[pos], inter["qh"])
        np.testing.assert_array_equal(ws["y"].cpu().numpy()[pos], inter["y"])
        got = out.cpu().numpy()[toks]
        assert_f32_close(got, ref, "exact out", 1e-5)
        np.testing.assert_array_equal(got, ref)
    else:
        assert_bf16_close(act_bits_bf16(ws["h"])[pos], inter["h"], "h")
        if cfg.get("L"):
            assert_bf16_close(np_bf16(ws["x_lat"])[toks], inter["x_lat"], "x_lat")
            assert_bf16_close(np_bf16(ws["routed"])[toks], inter["routed"], "routed")
        if inp.get("shared") is not None:
            assert_bf16_close(np_bf16(ws["shared_out"])[toks], inter["shared"], "shared")
        terms = ()
        if inp.get("shared") is not None:
            terms = (inter["up"] if cfg.get("L") else inter["routed"], inter["shared"])
        else:
            assert_bf16_close(np_bf16(out)[toks], inter["routed"], "routed out")
        worst = assert_bf16_close(np_bf16(out)[toks], ref, "out", addends=terms)
        say(f"workload {cfg_id}: worst |err|/rms = {worst:.3g}")


@pytest.mark.parametrize("cfg_id", [2, 4])
def test_layer_deterministic(cfg_id):
    inp, L, x, out = _run(cfg_id)
    a = out.clone()
    ws = L.workspace(inp["cfg"]["T"])
    h1 = ws["h"].clone()
    out2 = L.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       out2.view(torch.int32) if out2.dtype == torch.float32 else out2.view(torch.int16))
    assert torch.equal(h1, ws["h"])


def test_layer_edge_token_counts():
    """T = 1 and a ragged T on the tiny layer; every row checked against the oracle."""
    inp = inputs(1)
    L = layer(1)
    for T in (1, 7, 50):
        say(f"tiny layer T={T}")
        x = inp["x"][:T]
        out = L.forward(bf16_dev(x))
        torch.cuda.synchronize()
        ref, inter = oracle.layer_tokens(dict(inp, x=x), np.arange(T), want_intermediates=True)
        assert_bf16_close(np_bf16(out), ref, f"T={T}", addends=(inter["routed"], inter["shared"]))
    # empty input is a no-op
    out = L.forward(bf16_dev(inp["x"][:0]))
    assert out.shape[0] == 0


def test_layer_group_limited_routing():
    """The tiny workload with group-limited routing (4 groups of 4 experts, 2 kept,
    routed scaling factor 1.5): routing bit-exact, outputs within the bf16 bar."""
    from int4_routed_expert_moe_amd.layer import MoELayer
    base = inputs(1)
    inp = dict(base)
    inp["cfg"] = dict(base["cfg"], n_group=4, topk_group=2, routed_scale=1.5)
    cfg = inp["cfg"]
    L = MoELayer.from_numpy(inp, "cuda")
    say("layer forward workload 1 with group-limited routing")
    out = L.forward(bf16_dev(inp["x"]))
    torch.cuda.synchronize()
    ws = L.workspace(cfg["T"])
    ridx, rw = oracle.route_grouped(inp["x"], inp["router_w"], inp["router_b"], cfg["k"], 4, 2, True, 1.5)
    np.testing.assert_array_equal(ws["topk_idx"].cpu().numpy(), ridx)
    np.testing.assert_array_equal(ws["topk_w"].cpu().numpy(), rw)
    plain, _ = oracle.route(inp["x"], inp["router_w"], inp["router_b"], cfg["k"], True)
    assert (plain != ridx).any()  # the grouping changes some selections on this input
    ref, inter = oracle.layer_tokens(inp, np.arange(cfg["T"]), want_intermediates=True)
    terms = (inter["routed"], inter["shared"]) if inp.get("shared") is not None else ()
    assert_bf16_close(np_bf16(out), ref, "out", addends=terms)


def test_layer_exact16_on_skewed_routing():
    """The skewed exact workload with 16-bit activation codes: routing, the codes,
    h and y bit-exact on a token sample, the output within 1e-5."""
    from int4_routed_expert_moe_amd.layer import MoELayer
    base = inputs(4)
    inp = dict(base)
    inp["cfg"] = dict(base["cfg"], act_bits=16)
    cfg = inp["cfg"]
    T, k = cfg["T"], cfg["k"]
    L = MoELayer.from_numpy(inp, "cuda")
    say("layer forward workload 4 with 16-bit activation codes")
    out = L.forward(bf16_dev(inp["x"]))
    torch.cuda.synchronize()
    ws = L.workspace(T)
    ridx = ws["topk_idx"].cpu().numpy()
    rw = ws["topk_w"].cpu().numpy()
    oidx, ow = oracle.route(inp["x"], inp["router_w"], inp["router_b"], k, True)
    np.testing.assert_array_equal(ridx, oidx)
    np.testing.assert_array_equal(rw, ow)
    toks = synthetic.token_sample(cfg, 12)
    say(f"oracle on {len(toks)} tokens of workload 4 (16-bit codes)")
    ref, inter = oracle.layer_tokens(inp, toks, topk_idx=oidx, topk_w=ow, want_intermediates=True)
    rp = ws["slot_pos"].cpu().numpy()
    pos = rp[(toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)]
    np.testing.assert_array_equal(ws["qx"].cpu().numpy()[toks], inter["qx"])
    np.testing.assert_array_equal(ws["sx"].cpu().numpy()[toks], inter["sx"])
    np.testing.assert_array_equal(ws["h"].cpu().numpy()[pos], inter["qh"])
    np.testing.assert_array_equal(ws["h_scale"].cpu().numpy()[pos], inter["sh"])
    np.testing.assert_array_equal(ws["y"].cpu().numpy()[pos], inter["y"])
    got = out.cpu().numpy()[toks]
    assert_f32_close(got, ref, "exact16 out", 1e-5)
    np.testing.assert_array_equal(got, ref)


def _tiny_latent_inputs():
    """A small latent block of the K3 shape family: hidden 512, latent 256, 16 experts,
    top-2, intermediate 128, shared expert 128 (seeded like the workloads)."""
    cfg = dict(synthetic.WORKLOADS[1], name="tiny_latent", H=512, L=256, layer_seed=11, x_seed=11)
    w, b = synthetic.gen_router(cfg)
    return {"cfg": cfg, "x": synthetic.gen_x(cfg), "router_w": w, "router_b": b,
            "experts": synthetic.gen_experts(cfg), "shared": synthetic.gen_shared(cfg),
            "latent": synthetic.gen_latent(cfg)}


@pytest.mark.parametrize("renormalize,latent_norm,latent", [
    (False, True, False),   # the tiny layer with raw sigmoid weights
    (True, True, True),     # the latent block as the K3 page runs it
    (True, False, True),    # the latent block without the RMSNorm
    (False, False, True),   # both switches off
])
def test_layer_switches(renormalize, latent_norm, latent):
    """The K3 block's switches ("Kimi-K3 latent MoE" page, Code: __init__'s
    moe_renormalize and latent_moe_use_norm): routing bit-exact, every output
    row within the bf16 bar of the oracle taking the same switches."""
    from int4_routed_expert_moe_amd.layer import MoELayer
    base = _tiny_latent_inputs() if latent else inputs(1)
    inp = dict(base)
    inp["cfg"] = dict(base["cfg"], renormalize=renormalize, latent_norm=latent_norm)
    cfg = inp["cfg"]
    L = MoELayer.from_numpy(inp, "cuda")
    say(f"layer forward {cfg['name']} renormalize={renormalize} latent_norm={latent_norm}")
    out = L.forward(bf16_dev(inp["x"]))
    torch.cuda.synchronize()
    ws = L.workspace(cfg["T"])
    ridx, rw = oracle.route(inp["x"], inp["router_w"], inp["router_b"], cfg["k"], renormalize)
    np.testing.assert_array_equal(ws["topk_idx"].cpu().numpy(), ridx)
    np.testing.assert_array_equal(ws["topk_w"].cpu().numpy(), rw)
    ref, inter = oracle.layer_tokens(inp, np.arange(cfg["T"]), want_intermediates=True)
    if latent:
        assert_bf16_close(np_bf16(ws["routed"]), inter["routed"], "routed")
        terms = (inter["up"], inter["shared"])
    else:
        terms = (inter["routed"], inter["shared"])
    assert_bf16_close(np_bf16(out), ref, "out", addends=terms)
    # the switch changes the result
    other = oracle.layer_tokens(dict(inp, cfg=dict(cfg, renormalize=True, latent_norm=True)), np.arange(4))
    if not (renormalize and latent_norm):
        assert (other != ref[:4]).any()


def test_layer_rejects_out_of_range_scales():
    from int4_routed_expert_moe_amd import moe as _m
    from int4_routed_expert_moe_amd.layer import MoELayer
    base = inputs(1)
    ex = dict(base["experts"])
    sd = ex["sd"].copy()
    sd[3, 5, 1] = 0x4480  # bf16 1024.0, past 2^9
    ex["sd"] = sd
    say("layer load with an out-of-range down scale")
    with pytest.raises(_m.MoEError) as ei:
        MoELayer.from_numpy(dict(base, experts=ex), "cuda")
    assert ei.value.status == _m.MOE_ERR_UNSUPPORTED


def test_layer_activation_beyond_fp16_range():
    """An activation past the fp16 range saturates to 65504 in the routed experts (the
    documented conversion), while the router sees it as it is.  The tiny layer without
    its shared expert, token 9 with x[37] = 2^17 and x[38] = 0, and weight column 38 a
    copy of column 37 in every gate/up row: the GPU output of that token matches the
    oracle given x[37] = 65280 and x[38] = 224 (bf16 values whose products with the
    shared column sum to 65504 times it), with the routing of the real input, and is far
    from the oracle given the real value.  Every other token matches as usual.  Column
    37's scale group gets the smallest exact scale (2^-14) in every gate/up row, so h
    stays inside the fp16 range of the down projection's operands."""
    from int4_routed_expert_moe_amd.layer import MoELayer
    base = inputs(1)
    t, i = 9, 37
    ex = dict(base["experts"])
    for n in ("sg", "su"):
        sc = ex[n].copy()
        sc[:, :, i // 32] = 0x3880
        ex[n] = sc
    for n in ("wg", "wu"):
        w = ex[n].copy()
        hi37 = w[:, :, i // 2] >> 4                  # element 37: high nibble of byte 18
        w[:, :, (i + 1) // 2] = (w[:, :, (i + 1) // 2] & 0xF0) | hi37  # element 38: low nibble of byte 19
        ex[n] = w
    x = base["x"].copy()
    x[t, i] = 0x4800      # bf16 2^17
    x[t, i + 1] = 0       # 0.0
    inp = dict(base, shared=None, experts=ex, x=x, cfg=dict(base["cfg"], shared_I=None))
    L = MoELayer.from_numpy(inp, "cuda")
    say("tiny layer (no shared expert) with one activation of 2^17")
    out = L.forward(bf16_dev(x))
    torch.cuda.synchronize()
    T, k = inp["cfg"]["T"], inp["cfg"]["k"]
    ridx, rw = oracle.route(x, inp["router_w"], inp["router_b"], k, True)
    ws = L.workspace(T)
    np.testing.assert_array_equal(ws["topk_idx"].cpu().numpy(), ridx)
    got = np_bf16(out)
    others = np.array([s for s in range(T) if s != t])
    ref = oracle.layer_tokens(inp, others, topk_idx=ridx, topk_w=rw)
    assert_bf16_close(got[others], ref, "other tokens")
    x_sat = x.copy()
    x_sat[t, i] = 0x477F      # bf16 65280
    x_sat[t, i + 1] = 0x4360  # bf16 224
    ref_sat = oracle.layer_tokens(dict(inp, x=x_sat), [t], topk_idx=ridx, topk_w=rw)
    assert_bf16_close(got[t:t + 1], ref_sat, "saturated token")
    ref_raw = oracle.layer_tokens(inp, [t], topk_idx=ridx, topk_w=rw)
    with pytest.raises(AssertionError):
        assert_bf16_close(got[t:t + 1], ref_raw, "unsaturated reference")
