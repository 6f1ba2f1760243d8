"""Seeded synthetic inputs for the routed-expert MoE layer workloads.

This module draws random numbers and packs nothing: it holds none of the
layer's arithmetic, so both the HIP path and the CPU oracle can be fed from it.
Every tensor comes from its own PCG64 stream seeded with
``SeedSequence([layer_seed, tensor_id(, expert)])``.

Workload shapes follow the Kimi K2.5 layer (7168 hidden, 384 routed experts,
top-8, one shared expert; Kimi K2.5 donor reference, "What the archive
contains") and the Kimi-K3 latent block (3584-wide latent, RMSNorm before a
3584->7168 up-projection; Kimi-K3 latent MoE page, Parameters table and Code).
Value distributions:
  x            bf16( N(0,1) )
  router W     bf16( N(0, 0.02) ),  correction bias f32 U(-b, b) with b = 0.1 on the
               tiny layer and b = 0.003 on the K2.5/K3-shaped layers, whose routing is
               specified as uniform (with b = 0.1 the bias, not the logits, would decide
               most selections: the top scores sit near 1 where the sigmoid is flat)
  expert W     uniform random bytes (two int4 per byte -> uniform on [-8, 7]),
               bf16 group-32 scales U(0.005, 0.02)
  shared/latent bf16( N(0, 1/sqrt(fan_in)) ), RMSNorm gain bf16 U(0.9, 1.1)
The skewed-routing workload takes a calibrated router bias as an argument.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

# tensor ids of the seed streams
T_X, T_ROUTER_W, T_ROUTER_B = 0, 1, 2
T_WG, T_SG, T_WU, T_SU, T_WD, T_SD = 3, 4, 5, 6, 7, 8
T_SH_G, T_SH_U, T_SH_D = 9, 10, 11
T_LAT_DOWN, T_LAT_UP, T_GAIN = 12, 13, 14
T_ZIPF_CAL, T_SAMPLE = 15, 16

WORKLOADS = {
    1: dict(id=1, name="tiny", T=64, H=256, E=16, k=2, I=128, shared_I=128, L=None,
            mode="bf16", layer_seed=1, x_seed=1, rms_eps=1e-6, bias_range=0.1),
    2: dict(id=2, name="k25_decode", T=64, H=7168, E=384, k=8, I=2048, shared_I=2048, L=None,
            mode="bf16", layer_seed=2, x_seed=2, rms_eps=1e-6, bias_range=0.003),
    3: dict(id=3, name="k25_prefill", T=8192, H=7168, E=384, k=8, I=2048, shared_I=2048, L=None,
            mode="bf16", layer_seed=2, x_seed=3, rms_eps=1e-6, bias_range=0.003),
    4: dict(id=4, name="k25_exact_zipf", T=4096, H=7168, E=384, k=8, I=2048, shared_I=None,
            L=None, mode="exact", layer_seed=2, x_seed=4, rms_eps=1e-6, zipf=True, bias_range=0.003),
    5: dict(id=5, name="k3_latent", T=2048, H=7168, E=384, k=8, I=2048, shared_I=2048, L=3584,
            mode="bf16", layer_seed=5, x_seed=5, rms_eps=1e-6, bias_range=0.003),
}


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def uniform_bf16(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    v = g.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    return f32_to_bf16_bits(v)


def expert_dims(cfg):
    """(K_in, I) of the routed experts: they see the latent width when present."""
    return (cfg["L"] or cfg["H"]), cfg["I"]


def gen_experts(cfg, experts=None, threads: int | None = None):
    """Packed int4 expert weights and bf16 scales for the listed experts (all by default).

    Returns dict wg, sg, wu, su [n, I, K/2 | K/32] and wd, sd [n, K, I/2 | I/32]."""
    K, I = expert_dims(cfg)
    ids = list(range(cfg["E"])) if experts is None else [int(e) for e in experts]
    n = len(ids)
    out = {
        "wg": np.empty((n, I, K // 2), np.uint8), "sg": np.empty((n, I, K // 32), np.uint16),
        "wu": np.empty((n, I, K // 2), np.uint8), "su": np.empty((n, I, K // 32), np.uint16),
        "wd": np.empty((n, K, I // 2), np.uint8), "sd": np.empty((n, K, I // 32), np.uint16),
    }
    seed = cfg["layer_seed"]

    def one(j):
        e = ids[j]
        for name, tid in (("wg", T_WG), ("wu", T_WU), ("wd", T_WD)):
            a = out[name][j]
            a[...] = np.frombuffer(rng(seed, tid, e).bytes(a.size), dtype=np.uint8).reshape(a.shape)
        for name, tid in (("sg", T_SG), ("su", T_SU), ("sd", T_SD)):
            a = out[name][j]
            a[...] = uniform_bf16(rng(seed, tid, e), a.shape, 0.005, 0.02)

    threads = threads or min(16, os.cpu_count() or 1)
    if n > 1 and threads > 1:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n)))
    else:
        for j in range(n):
            one(j)
    return out


def gen_x(cfg, T=None):
    T = cfg["T"] if T is None else T
    return normal_bf16(rng(cfg["x_seed"], T_X), (T, cfg["H"]))


def gen_router(cfg):
    s = cfg["layer_seed"]
    w = normal_bf16(rng(s, T_ROUTER_W), (cfg["E"], cfg["H"]), 0.02)
    br = np.float32(cfg.get("bias_range", 0.1))
    b = (rng(s, T_ROUTER_B).random(cfg["E"], dtype=np.float32) * (np.float32(2) * br) - br).astype(np.float32)
    return w, b


def gen_shared(cfg):
    if not cfg["shared_I"]:
        return None
    s, H, I = cfg["layer_seed"], cfg["H"], cfg["shared_I"]
    return {
        "wg": normal_bf16(rng(s, T_SH_G), (I, H), 1.0 / np.sqrt(H)),
        "wu": normal_bf16(rng(s, T_SH_U), (I, H), 1.0 / np.sqrt(H)),
        "wd": normal_bf16(rng(s, T_SH_D), (H, I), 1.0 / np.sqrt(I)),
    }


def gen_latent(cfg):
    if not cfg["L"]:
        return None
    s, H, L = cfg["layer_seed"], cfg["H"], cfg["L"]
    return {
        "w_down": normal_bf16(rng(s, T_LAT_DOWN), (L, H), 1.0 / np.sqrt(H)),
        "w_up": normal_bf16(rng(s, T_LAT_UP), (H, L), 1.0 / np.sqrt(L)),
        "gain": uniform_bf16(rng(s, T_GAIN), (L,), 0.9, 1.1),
    }


def make_inputs(cfg_id: int, router_bias: np.ndarray | None = None, with_experts: bool = True,
                T: int | None = None):
    """All inputs of one workload as numpy arrays (see module docstring).

    ``router_bias`` replaces the drawn correction bias (the skewed-routing
    workload requires its calibrated bias here)."""
    cfg = dict(WORKLOADS[cfg_id])
    if T is not None:
        cfg["T"] = T
    if cfg.get("zipf") and router_bias is None:
        raise ValueError("the skewed-routing workload needs its calibrated router bias")
    w, b = gen_router(cfg)
    if router_bias is not None:
        b = np.ascontiguousarray(router_bias, dtype=np.float32)
        assert b.shape == (cfg["E"],)
    return {
        "cfg": cfg,
        "x": gen_x(cfg),
        "router_w": w,
        "router_b": b,
        "experts": gen_experts(cfg) if with_experts else None,
        "shared": gen_shared(cfg),
        "latent": gen_latent(cfg),
    }


def token_sample(cfg, n: int, salt: int = 0) -> np.ndarray:
    """A seeded sorted sample of n distinct token indices."""
    T = cfg["T"]
    n = min(n, T)
    return np.sort(rng(cfg["x_seed"], T_SAMPLE, salt).choice(T, size=n, replace=False)).astype(np.int64)


def calibration_x(cfg, T: int) -> np.ndarray:
    """Activations of a separate calibration batch (used to fit the skewed router bias)."""
    return normal_bf16(rng(cfg["layer_seed"], T_ZIPF_CAL), (T, cfg["H"]))


def load_bias_file(path: str) -> np.ndarray:
    """Read a router-bias fixture: one float32 per line written as a hex float; '#' lines skipped."""
    vals = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals.append(float.fromhex(line))
    return np.asarray(vals, dtype=np.float32)
