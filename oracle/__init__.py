"""CPU oracle for the int4 routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
built with gcc, contraction off, no fast-math) through ctypes and composes its
steps into a whole-layer reference for a sample of tokens.  It shares no code
with the HIP library and does not import it.

Every step cites the page passage it follows inside ``moe_oracle.c``.  Arrays
are numpy: bf16 tensors are ``uint16`` bit patterns, packed int4 weights are
``uint8`` ([rows, cols/2], low nibble = even column), scales are bf16
``uint16`` ([rows, cols/32]).

Parity pinning: every function here is pinned by a ``-m "not gpu"`` test
against closed forms, brute force or library routines (tests/test_oracle_*.py).
Parity against the pages' own implementation is unpinned: the pages print no
implementation of the exact path and no outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_LIB selects another build of the same source (the sanitizer build below)
_LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "libmoe_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc into oracle/libmoe_oracle.so, or with AddressSanitizer and
    UndefinedBehaviorSanitizer into oracle/libmoe_oracle_san.so (load it with MOE_ORACLE_LIB and
    gcc's libasan/libubsan preloaded)."""
    if sanitize:
        out = os.path.join(_HERE, "libmoe_oracle_san.so")
        subprocess.check_call(["gcc", *CFLAGS, *SAN_FLAGS, _SRC, "-o", out, "-lm"])
        return out
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I32 = ctypes.c_int
F32 = ctypes.c_float


def _declare(L):
    L.oracle_f32_to_bf16.argtypes = [F32]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    L.oracle_f64_to_bf16.restype = ctypes.c_uint16
    L.oracle_threads.argtypes = []
    L.oracle_threads.restype = I32
    L.oracle_const.argtypes = [I32]
    L.oracle_const.restype = F32
    for name in ("oracle_exp_ref", "oracle_sigmoid_ref", "oracle_silu_ref"):
        getattr(L, name).argtypes = [F32]
        getattr(L, name).restype = F32
    L.oracle_unpack_int4.argtypes = [P, I32, I32, P]
    L.oracle_router_logits.argtypes = [P, P, I32, I32, I32, P]
    L.oracle_topk_from_scores.argtypes = [P, P, I32, I32, I32, I32, P, P]
    L.oracle_route.argtypes = [P, P, P, I32, I32, I32, I32, I32, P, P, P, P]
    L.oracle_permute.argtypes = [P, I32, I32, I32, P, P, P, P]
    L.oracle_experts_bf16.argtypes = [P, P, I32, I32, I32] + [P] * 6 + [P] * 4
    L.oracle_combine_bf16.argtypes = [P, P, P, I32, I32, I32, P]
    L.oracle_silu_mul_bf16.argtypes = [P, P, ctypes.c_long, P]
    L.oracle_linear_bf16.argtypes = [P, P, P, I32, I32, I32, P]
    L.oracle_dense_swiglu_bf16.argtypes = [P, P, P, P, I32, I32, I32, P, P]
    L.oracle_rmsnorm_bf16.argtypes = [P, P, F32, I32, I32, P]
    L.oracle_quant_f32_int8.argtypes = [P, I32, I32, P, P]
    L.oracle_quant_act_int8.argtypes = [P, I32, I32, P, P]
    L.oracle_group_sums.argtypes = [P, P, I32, I32, I32, P, P]
    L.oracle_exact_linear.argtypes = [P, P, P, P, I32, I32, I32, P]
    L.oracle_experts_exact.argtypes = [P, P, P, I32, I32, I32] + [P] * 6 + [P] * 5
    L.oracle_combine_f32.argtypes = [P, P, I32, I32, I32, P]
    L.oracle_topk_grouped_from_scores.argtypes = [P, P, I32, I32, I32, I32, I32, I32, F32, P, P]
    L.oracle_quant_act_int16.argtypes = [P, I32, I32, P, P]
    L.oracle_group_sums16.argtypes = [P, P, I32, I32, I32, P, P]
    L.oracle_exact_linear16.argtypes = [P, P, P, P, I32, I32, I32, P]
    L.oracle_experts_exact16.argtypes = [P, P, P, I32, I32, I32] + [P] * 6 + [P] * 5
    L.oracle_exact_linear_i8w.argtypes = [P, P, P, P, I32, I32, I32, P]
    for name in ("oracle_exp_ref_n", "oracle_sigmoid_ref_n", "oracle_silu_ref_n",
                 "oracle_f64_to_bf16_n", "oracle_f32_to_bf16_n"):
        getattr(L, name).argtypes = [P, I32, P]
        getattr(L, name).restype = None
    for fn in ("oracle_unpack_int4", "oracle_router_logits", "oracle_topk_from_scores",
               "oracle_route", "oracle_permute", "oracle_experts_bf16", "oracle_combine_bf16",
               "oracle_linear_bf16", "oracle_dense_swiglu_bf16", "oracle_rmsnorm_bf16",
               "oracle_quant_f32_int8", "oracle_quant_act_int8", "oracle_group_sums",
               "oracle_exact_linear", "oracle_experts_exact", "oracle_combine_f32",
               "oracle_topk_grouped_from_scores", "oracle_quant_act_int16", "oracle_group_sums16",
               "oracle_exact_linear16", "oracle_experts_exact16", "oracle_exact_linear_i8w",
               "oracle_silu_mul_bf16"):
        getattr(L, fn).restype = None


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def f32_to_bf16(v: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(np.float32(v))))


def f64_to_bf16(v: float) -> int:
    return int(lib().oracle_f64_to_bf16(float(v)))


def threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(lib().oracle_threads())


def const(which: int) -> float:
    return float(lib().oracle_const(which))


def exp_ref(t: float) -> float:
    return float(np.float32(lib().oracle_exp_ref(float(np.float32(t)))))


def sigmoid_ref(z: float) -> float:
    return float(np.float32(lib().oracle_sigmoid_ref(float(np.float32(z)))))


def silu_ref(z: float) -> float:
    return float(np.float32(lib().oracle_silu_ref(float(np.float32(z)))))


def _vec(fn, a, in_dtype, out_dtype):
    a = _c(a, in_dtype).ravel()
    out = np.empty(a.shape, dtype=out_dtype)
    getattr(lib(), fn)(_p(a), a.size, _p(out))
    return out


def exp_ref_n(t):
    return _vec("oracle_exp_ref_n", t, np.float32, np.float32)


def sigmoid_ref_n(z):
    return _vec("oracle_sigmoid_ref_n", z, np.float32, np.float32)


def silu_ref_n(z):
    return _vec("oracle_silu_ref_n", z, np.float32, np.float32)


def f64_to_bf16_n(d):
    return _vec("oracle_f64_to_bf16_n", d, np.float64, np.uint16)


def f32_to_bf16_n(f):
    return _vec("oracle_f32_to_bf16_n", f, np.float32, np.uint16)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K), dtype=np.int8)
    lib().oracle_unpack_int4(_p(packed), N, K, _p(out))
    return out


# --------------------------------------------------------------------------
# routing and permutation
# --------------------------------------------------------------------------

def router_logits(x, wr):
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_logits(_p(x), _p(wr), T, H, E, _p(out))
    return out


def topk_from_scores(scores, bias, k, renormalize=True):
    scores = _c(scores, np.float32)
    bias = _c(bias, np.float32)
    T, E = scores.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    lib().oracle_topk_from_scores(_p(scores), _p(bias), T, E, k, int(bool(renormalize)), _p(idx), _p(w))
    return idx, w


def topk_grouped_from_scores(scores, bias, k, n_group, topk_group, renormalize=True, scale=1.0):
    """Group-limited selection (see oracle_topk_grouped_from_scores)."""
    scores = _c(scores, np.float32)
    bias = _c(bias, np.float32)
    T, E = scores.shape
    if (n_group < 1 or E % n_group or not 1 <= topk_group <= n_group or k > topk_group * (E // n_group)
            or (n_group > 1 and E // n_group < 2)):
        raise ValueError("bad group configuration")
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    lib().oracle_topk_grouped_from_scores(_p(scores), _p(bias), T, E, k, n_group, topk_group,
                                          int(bool(renormalize)), float(scale), _p(idx), _p(w))
    return idx, w


def route_grouped(x, wr, bias, k, n_group, topk_group, renormalize=True, scale=1.0):
    """Routing with group-limited selection: logits and sigmoid as route(), then
    topk_grouped_from_scores."""
    _, _, _, scores = route(x, wr, bias, k, renormalize, return_scores=True)
    return topk_grouped_from_scores(scores, bias, k, n_group, topk_group, renormalize, scale)


def route(x, wr, bias, k, renormalize=True, return_scores=False):
    """Returns (topk_idx [T,k] int32, topk_w [T,k] f32[, logits, scores])."""
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    logits = np.empty((T, E), dtype=np.float32)
    scores = np.empty((T, E), dtype=np.float32)
    lib().oracle_route(_p(x), _p(wr), _p(bias), T, H, E, k, int(bool(renormalize)), _p(idx), _p(w),
                       _p(logits), _p(scores))
    if return_scores:
        return idx, w, logits, scores
    return idx, w


def permute(topk_idx, E):
    """Returns (counts [E], offsets [E+1], sorted_slot [S], slot_pos [S])."""
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    S = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_slot = np.empty(S, dtype=np.int32)
    slot_pos = np.empty(S, dtype=np.int32)
    lib().oracle_permute(_p(topk_idx), T, k, E, _p(counts), _p(offsets), _p(sorted_slot), _p(slot_pos))
    return counts, offsets, sorted_slot, slot_pos


# --------------------------------------------------------------------------
# bf16 path
# --------------------------------------------------------------------------

def experts_bf16(rows, experts, W, want=("h", "y")):
    """rows [P,H] bf16, experts [P] int32, W: dict with wg, sg, wu, su, wd, sd.
    Returns dict with the requested outputs among g, u, h, y (bf16)."""
    rows = _c(rows, np.uint16)
    experts = _c(experts, np.int32)
    P_, H = rows.shape
    I = W["wg"].shape[1]
    out = {}
    for name, n in (("g", I), ("u", I), ("h", I), ("y", H)):
        out[name] = np.empty((P_, n), dtype=np.uint16) if name in want else None
    lib().oracle_experts_bf16(_p(rows), _p(experts), P_, H, I,
                              _p(_c(W["wg"], np.uint8)), _p(_c(W["sg"], np.uint16)),
                              _p(_c(W["wu"], np.uint8)), _p(_c(W["su"], np.uint16)),
                              _p(_c(W["wd"], np.uint8)), _p(_c(W["sd"], np.uint16)),
                              _p(out["g"]), _p(out["u"]), _p(out["h"]), _p(out["y"]))
    return {k_: v for k_, v in out.items() if v is not None}


def silu_mul_bf16(g, u):
    """h = bf16(bf16(silu(g)) * u) elementwise on bf16 bit patterns (the SwiGLU join)."""
    g = _c(g, np.uint16)
    u = _c(u, np.uint16)
    assert g.shape == u.shape
    h = np.empty_like(g)
    lib().oracle_silu_mul_bf16(_p(g), _p(u), g.size, _p(h))
    return h


def combine_bf16(y, w, shared=None):
    """y [T,k,H] bf16 (slot order), w [T,k] f32, shared [T,H] bf16 or None."""
    y = _c(y, np.uint16)
    w = _c(w, np.float32)
    T, k, H = y.shape
    out = np.empty((T, H), dtype=np.uint16)
    sh = None if shared is None else _c(shared, np.uint16)
    lib().oracle_combine_bf16(_p(y), _p(w), _p(sh), T, k, H, _p(out))
    return out


def linear_bf16(x, w, add=None):
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    y = np.empty((M, N), dtype=np.uint16)
    ad = None if add is None else _c(add, np.uint16)
    lib().oracle_linear_bf16(_p(x), _p(w), _p(ad), M, N, K, _p(y))
    return y


def dense_swiglu_bf16(x, wg, wu, wd, want_h=False):
    x = _c(x, np.uint16)
    M, H = x.shape
    I = wg.shape[0]
    y = np.empty((M, H), dtype=np.uint16)
    h = np.empty((M, I), dtype=np.uint16) if want_h else None
    lib().oracle_dense_swiglu_bf16(_p(x), _p(_c(wg, np.uint16)), _p(_c(wu, np.uint16)),
                                   _p(_c(wd, np.uint16)), M, H, I, _p(h), _p(y))
    return (h, y) if want_h else y


def rmsnorm_bf16(x, gain, eps):
    x = _c(x, np.uint16)
    M, N = x.shape
    y = np.empty((M, N), dtype=np.uint16)
    lib().oracle_rmsnorm_bf16(_p(x), _p(_c(gain, np.uint16)), float(eps), M, N, _p(y))
    return y


# --------------------------------------------------------------------------
# exact mode
# --------------------------------------------------------------------------

def quant_act_int8(x):
    x = _c(x, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M, K // 32), dtype=np.float32)
    lib().oracle_quant_act_int8(_p(x), M, K, _p(q), _p(s))
    return q, s


def quant_f32_int8(x):
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M, K // 32), dtype=np.float32)
    lib().oracle_quant_f32_int8(_p(x), M, K, _p(q), _p(s))
    return q, s


def group_sums(qx, packed, K, with_int64=False):
    qx = _c(qx, np.int8)
    packed = _c(packed, np.uint8)
    M = qx.shape[0]
    N = packed.shape[0]
    G32 = np.empty((M, N, K // 32), dtype=np.int32)
    G64 = np.empty((M, N, K // 32), dtype=np.int64) if with_int64 else None
    lib().oracle_group_sums(_p(qx), _p(packed), M, N, K, _p(G32), _p(G64))
    return (G32, G64) if with_int64 else G32


def exact_linear(qx, sx, packed, scale):
    qx = _c(qx, np.int8)
    sx = _c(sx, np.float32)
    M, K = qx.shape
    N = packed.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    lib().oracle_exact_linear(_p(qx), _p(sx), _p(_c(packed, np.uint8)), _p(_c(scale, np.uint16)),
                              M, N, K, _p(y))
    return y


def experts_exact(qx, sx, experts, W, want=("y",)):
    qx = _c(qx, np.int8)
    sx = _c(sx, np.float32)
    experts = _c(experts, np.int32)
    P_, H = qx.shape
    I = W["wg"].shape[1]
    g = np.empty((P_, I), np.float32) if "g" in want else None
    u = np.empty((P_, I), np.float32) if "u" in want else None
    qh = np.empty((P_, I), np.int8) if "qh" in want else None
    sh = np.empty((P_, I // 32), np.float32) if "sh" in want else None
    y = np.empty((P_, H), np.float32)
    lib().oracle_experts_exact(_p(qx), _p(sx), _p(experts), P_, H, I,
                               _p(_c(W["wg"], np.uint8)), _p(_c(W["sg"], np.uint16)),
                               _p(_c(W["wu"], np.uint8)), _p(_c(W["su"], np.uint16)),
                               _p(_c(W["wd"], np.uint8)), _p(_c(W["sd"], np.uint16)),
                               _p(g), _p(u), _p(qh), _p(sh), _p(y))
    out = {"y": y}
    for name, v in (("g", g), ("u", u), ("qh", qh), ("sh", sh)):
        if v is not None:
            out[name] = v
    return out


# exact mode with 16-bit activations (act_bits = 16)

def quant_act_int16(x):
    x = _c(x, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int16)
    s = np.empty((M, K // 32), dtype=np.float32)
    lib().oracle_quant_act_int16(_p(x), M, K, _p(q), _p(s))
    return q, s


def group_sums16(qx, packed, K, with_int64=False):
    qx = _c(qx, np.int16)
    packed = _c(packed, np.uint8)
    M = qx.shape[0]
    N = packed.shape[0]
    G32 = np.empty((M, N, K // 32), dtype=np.int32)
    G64 = np.empty((M, N, K // 32), dtype=np.int64) if with_int64 else None
    lib().oracle_group_sums16(_p(qx), _p(packed), M, N, K, _p(G32), _p(G64))
    return (G32, G64) if with_int64 else G32


def exact_linear16(qx, sx, packed, scale):
    qx = _c(qx, np.int16)
    sx = _c(sx, np.float32)
    M, K = qx.shape
    N = packed.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    lib().oracle_exact_linear16(_p(qx), _p(sx), _p(_c(packed, np.uint8)), _p(_c(scale, np.uint16)), M, N, K, _p(y))
    return y


def experts_exact16(qx, sx, experts, W, want=("y",)):
    qx = _c(qx, np.int16)
    sx = _c(sx, np.float32)
    experts = _c(experts, np.int32)
    P_, H = qx.shape
    I = W["wg"].shape[1]
    g = np.empty((P_, I), np.float32) if "g" in want else None
    u = np.empty((P_, I), np.float32) if "u" in want else None
    qh = np.empty((P_, I), np.int16) if "qh" in want else None
    sh = np.empty((P_, I // 32), np.float32) if "sh" in want else None
    y = np.empty((P_, H), np.float32)
    lib().oracle_experts_exact16(_p(qx), _p(sx), _p(experts), P_, H, I,
                                 _p(_c(W["wg"], np.uint8)), _p(_c(W["sg"], np.uint16)),
                                 _p(_c(W["wu"], np.uint8)), _p(_c(W["su"], np.uint16)),
                                 _p(_c(W["wd"], np.uint8)), _p(_c(W["sd"], np.uint16)),
                                 _p(g), _p(u), _p(qh), _p(sh), _p(y))
    out = {"y": y}
    for name, v in (("g", g), ("u", u), ("qh", qh), ("sh", sh)):
        if v is not None:
            out[name] = v
    return out


def exact_linear_i8w(qx, sx, qw, sw):
    """ExactLinear with 8-bit weights: int8 codes and fp32 group scales on both sides."""
    qx = _c(qx, np.int8)
    sx = _c(sx, np.float32)
    qw = _c(qw, np.int8)
    sw = _c(sw, np.float32)
    M, K = qx.shape
    N = qw.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    lib().oracle_exact_linear_i8w(_p(qx), _p(sx), _p(qw), _p(sw), M, N, K, _p(y))
    return y


def combine_f32(y, w):
    y = _c(y, np.float32)
    w = _c(w, np.float32)
    T, k, H = y.shape
    out = np.empty((T, H), dtype=np.float32)
    lib().oracle_combine_f32(_p(y), _p(w), T, k, H, _p(out))
    return out


# --------------------------------------------------------------------------
# whole layer on a sample of tokens (token-independent after routing)
# --------------------------------------------------------------------------

def layer_tokens(inp, tokens, topk_idx=None, topk_w=None, want_intermediates=False):
    """Reference output of the MoE layer for the tokens listed in ``tokens``.

    ``inp`` is the dict produced by the seeded input generator (keys: cfg, x,
    router_w, router_b, experts{wg,sg,wu,su,wd,sd}, shared{wg,wu,wd} or None,
    latent{w_down,w_up,gain} or None).  Routing is computed here for the listed
    tokens unless ``topk_idx``/``topk_w`` (full [T,k]) are given.  The
    configuration's ``renormalize`` and ``latent_norm`` switches ("Kimi-K3
    latent MoE" page, Code: __init__'s moe_renormalize and latent_moe_use_norm)
    default to on.  Returns
    out [n, H] (bf16 uint16 for the bf16 path, float32 for exact mode) and,
    when asked, the per-slot intermediates.
    """
    cfg = inp["cfg"]
    k = cfg["k"]
    tokens = np.asarray(tokens, dtype=np.int64)
    x = inp["x"][tokens]
    renorm = bool(cfg.get("renormalize", True))
    if topk_idx is None:
        if cfg.get("n_group", 1) != 1 or cfg.get("routed_scale", 1.0) != 1.0:
            idx, w = route_grouped(x, inp["router_w"], inp["router_b"], k, int(cfg.get("n_group", 1)),
                                   int(cfg.get("topk_group", 1)), renorm, float(cfg.get("routed_scale", 1.0)))
        else:
            idx, w = route(x, inp["router_w"], inp["router_b"], k, renorm)
    else:
        idx, w = topk_idx[tokens], topk_w[tokens]
    n = len(tokens)
    H = cfg["H"]
    lat = inp.get("latent")
    xr = x
    if lat is not None:
        xr = linear_bf16(x, lat["w_down"])
    rows = np.repeat(xr, k, axis=0)
    experts = idx.reshape(-1)
    inter = {"idx": idx, "w": w}
    if cfg["mode"] == "exact":
        act16 = int(cfg.get("act_bits", 8)) == 16
        qx, sx = (quant_act_int16 if act16 else quant_act_int8)(xr)
        qrows = np.repeat(qx, k, axis=0)
        srows = np.repeat(sx, k, axis=0)
        r = (experts_exact16 if act16 else experts_exact)(
            qrows, srows, experts, inp["experts"],
            want=("g", "u", "qh", "sh", "y") if want_intermediates else ("y",))
        out = combine_f32(r["y"].reshape(n, k, -1), w)
        inter.update(r)
        inter.update({"qx": qx, "sx": sx})
    else:
        r = experts_bf16(rows, experts, inp["experts"],
                         want=("g", "u", "h", "y") if want_intermediates else ("y",))
        Hr = r["y"].shape[1]
        sh_out = None
        if inp.get("shared") is not None:
            s = inp["shared"]
            sh_out = dense_swiglu_bf16(x, s["wg"], s["wu"], s["wd"])
            inter["shared"] = sh_out
        routed = combine_bf16(r["y"].reshape(n, k, Hr), w, None)
        inter["routed"] = routed
        if lat is None:
            out = combine_bf16(r["y"].reshape(n, k, Hr), w, sh_out)
        else:
            # the K3 block's latent_moe_use_norm switch (on unless the configuration turns it off)
            nrm = rmsnorm_bf16(routed, lat["gain"], cfg["rms_eps"]) if cfg.get("latent_norm", True) else routed
            out = linear_bf16(nrm, lat["w_up"], add=sh_out)
            inter.update({"x_lat": xr, "normed": nrm})
            if want_intermediates:
                inter["up"] = linear_bf16(nrm, lat["w_up"])
        inter.update(r)
    assert out.shape[1] == H
    return (out, inter) if want_intermediates else out
