"""Helpers shared by the GPU parity tests: cached workloads (host arrays for the
oracle, device tensors for the HIP path), conversions, and the tolerances."""
import os
import sys

import numpy as np
import torch

from int4_routed_expert_moe_amd import synthetic

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_experts = {}
_inputs = {}
_layers = {}


def say(msg):
    """Name the case before a GPU step (visible even if the step never returns)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def inputs(cfg_id):
    """Workload cfg_id as numpy arrays; expert weights are shared by workloads of one layer."""
    if cfg_id in _inputs:
        return _inputs[cfg_id]
    cfg = synthetic.WORKLOADS[cfg_id]
    bias = None
    if cfg.get("zipf"):
        bias = synthetic.load_bias_file(os.path.join(GOLD, "zipf_bias_k25.txt"))
    inp = synthetic.make_inputs(cfg_id, router_bias=bias, with_experts=False)
    key = (cfg["layer_seed"], cfg["L"] or cfg["H"], cfg["I"], cfg["E"])
    if key not in _experts:
        _experts[key] = synthetic.gen_experts(inp["cfg"])
    inp["experts"] = _experts[key]
    _inputs[cfg_id] = inp
    return inp


def layer(cfg_id):
    from int4_routed_expert_moe_amd.layer import MoELayer
    if cfg_id not in _layers:
        inp = inputs(cfg_id)
        key = ("dev",) + (inp["cfg"]["layer_seed"], inp["cfg"]["mode"], cfg_id if inp["cfg"].get("zipf") else 0)
        _layers[cfg_id] = MoELayer.from_numpy(inp, "cuda")
    return _layers[cfg_id]


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def np_bf16(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


_F16P_ORDER = np.array([0, 4, 1, 5, 2, 6, 3, 7])


def f16p_values(bits16):
    """fp16 staging format (8-element blocks stored as e0,e4,e1,e5,e2,e6,e3,e7)
    -> float64 in element order."""
    h = np.asarray(bits16, np.uint16).view(np.float16).astype(np.float64)
    blocks = h.reshape(*h.shape[:-1], h.shape[-1] // 8, 8)
    out = np.empty_like(blocks)
    out[..., _F16P_ORDER] = blocks
    return out.reshape(h.shape)


def act_bits_bf16(t):
    """A bf16-path activation buffer as bf16 bit patterns in element order: bf16
    as is, or the fp16 staging format (whose values are bf16 values, so the
    conversion back is exact in the fp16 normal range)."""
    if t.dtype == torch.float16:
        from tests import refmath
        v = f16p_values(t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        return refmath.bf16_from_f32(v.astype(np.float32))
    return np_bf16(t)


def bf16_to_f64(a):
    return ((np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)).astype(np.float64)


def assert_bf16_close(got, ref, what="", atol_rms=1e-2, rtol=2e-2, addends=()):
    """bf16-path tolerance: |g - r| <= atol_rms * rms(r) + rtol * m elementwise, with
    m = |r|, or, for an output that is the bf16 sum of bf16 terms (the shared-expert
    add), m = the sum of the terms' magnitudes: one bf16 step of a term survives a
    cancellation in the sum.  The absolute part is scaled by the reference's rms so
    it means the same at any output scale."""
    g = bf16_to_f64(got)
    r = bf16_to_f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    rms = float(np.sqrt(np.mean(r * r))) or 1.0
    err = np.abs(g - r)
    mag = np.abs(r)
    if addends:
        mag = np.maximum(mag, sum(np.abs(bf16_to_f64(a)) for a in addends))
    bound = atol_rms * rms + rtol * mag
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"got {g[i]!r} ref {r[i]!r} (rms {rms:.4g})")
    return float(np.max(err) / rms)


def assert_f32_close(got, ref, what="", rel=1e-5):
    """exact-mode tolerance: max|g - r| / max|r| <= rel."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref))) or 1.0
    err = float(np.max(np.abs(got - ref))) / scale
    assert err <= rel, f"{what}: max rel err {err:.3g} > {rel}"
    return err
