"""Whole-layer pins of the oracle: token independence (a permutation of the
tokens permutes the outputs, duplicated tokens give identical rows), sampled
evaluation equals full evaluation, and the latent variant's wiring."""
import numpy as np
import pytest

import oracle
from int4_routed_expert_moe_amd import synthetic


def _small_latent_inputs():
    cfg = dict(synthetic.WORKLOADS[1], id=99, name="tiny_latent", L=128, layer_seed=99, x_seed=99)
    return {
        "cfg": cfg,
        "x": synthetic.gen_x(cfg),
        "router_w": synthetic.gen_router(cfg)[0],
        "router_b": synthetic.gen_router(cfg)[1],
        "experts": synthetic.gen_experts(cfg),
        "shared": synthetic.gen_shared(cfg),
        "latent": synthetic.gen_latent(cfg),
    }


@pytest.mark.parametrize("which", ["tiny", "latent"])
def test_token_permutation_equivariance(which):
    inp = synthetic.make_inputs(1) if which == "tiny" else _small_latent_inputs()
    T = inp["cfg"]["T"]
    tokens = np.arange(T)
    out, inter = oracle.layer_tokens(inp, tokens, want_intermediates=True)
    perm = np.random.default_rng(7).permutation(T)
    inp2 = dict(inp, x=inp["x"][perm])
    out2, inter2 = oracle.layer_tokens(inp2, tokens, want_intermediates=True)
    np.testing.assert_array_equal(out2, out[perm])
    np.testing.assert_array_equal(inter2["idx"], inter["idx"][perm])
    np.testing.assert_array_equal(inter2["w"], inter["w"][perm])


def test_duplicate_tokens_give_identical_rows():
    inp = synthetic.make_inputs(1)
    x = inp["x"].copy()
    x[10] = x[3]
    x[40] = x[3]
    out = oracle.layer_tokens(dict(inp, x=x), np.arange(inp["cfg"]["T"]))
    np.testing.assert_array_equal(out[10], out[3])
    np.testing.assert_array_equal(out[40], out[3])


def test_sampled_tokens_equal_full_evaluation():
    inp = synthetic.make_inputs(1)
    T = inp["cfg"]["T"]
    full = oracle.layer_tokens(inp, np.arange(T))
    sample = synthetic.token_sample(inp["cfg"], 9)
    np.testing.assert_array_equal(oracle.layer_tokens(inp, sample), full[sample])


def test_latent_wiring():
    """Routing sees the full-width input; experts see the latent; the shared expert
    sees the full-width input and is added after the up-projection."""
    inp = _small_latent_inputs()
    cfg = inp["cfg"]
    T, k = cfg["T"], cfg["k"]
    tokens = np.arange(T)
    out, inter = oracle.layer_tokens(inp, tokens, want_intermediates=True)
    idx, _ = oracle.route(inp["x"], inp["router_w"], inp["router_b"], k, True)
    np.testing.assert_array_equal(inter["idx"], idx)
    x_lat = oracle.linear_bf16(inp["x"], inp["latent"]["w_down"])
    np.testing.assert_array_equal(inter["x_lat"], x_lat)
    assert inter["y"].shape == (T * k, cfg["L"])
    sh = oracle.dense_swiglu_bf16(inp["x"], inp["shared"]["wg"], inp["shared"]["wu"], inp["shared"]["wd"])
    up = oracle.linear_bf16(inter["normed"], inp["latent"]["w_up"], add=sh)
    np.testing.assert_array_equal(out, up)
    assert out.shape == (T, cfg["H"])


def test_exact_mode_tiny_layer_consistency():
    cfg = dict(synthetic.WORKLOADS[1], id=98, mode="exact", shared_I=None)
    inp = {
        "cfg": cfg, "x": synthetic.gen_x(cfg), "router_w": synthetic.gen_router(cfg)[0],
        "router_b": synthetic.gen_router(cfg)[1], "experts": synthetic.gen_experts(cfg),
        "shared": None, "latent": None,
    }
    T, k = cfg["T"], cfg["k"]
    out, inter = oracle.layer_tokens(inp, np.arange(T), want_intermediates=True)
    assert out.dtype == np.float32
    y = inter["y"].reshape(T, k, -1)
    np.testing.assert_array_equal(out, oracle.combine_f32(y, inter["w"]))
    # the bf16 and exact paths agree to quantisation accuracy on the same layer
    bf = oracle.layer_tokens(dict(inp, cfg=dict(cfg, mode="bf16")), np.arange(T))
    bff = (bf.astype(np.uint32) << 16).view(np.float32)
    rms = np.sqrt(np.mean(bff.astype(np.float64) ** 2))
    assert np.max(np.abs(out - bff)) / rms < 0.1
