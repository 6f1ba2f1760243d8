"""One MoE layer forward as a sequence of C-ABI calls on one HIP stream.

Kimi-K3 latent MoE page, Code (forward / moe_infer): the router sees the
full-width hidden state; the latent variant projects it down before the
routed experts and back up after an RMSNorm; the shared expert runs on the
full-width input and is added last.  The same Code's __init__ makes two steps
optional, and the configuration carries them: ``renormalize`` (the selected
weights divided by their sum, default on) and ``latent_norm`` (the RMSNorm
before the up-projection, default on).  For the K2.5-shaped layer there is no
latent step and the shared add happens inside the combine.

Nothing here computes: the class owns device buffers (weights and a
per-token-count workspace) and issues the library calls in order.  No call
synchronises with the host.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe as _m


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def _u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def prepack_experts(ex: dict) -> dict:
    """Checkpoint-layout expert tensors (wg/sg, wu/su, wd/sd) -> the fragment layout
    the grouped GEMMs read (one exact byte permutation per matrix, scales as fp16, on the GPU)."""
    out = {}
    for w, s in (("wg", "sg"), ("wu", "su"), ("wd", "sd")):
        pw, ps = torch.empty_like(ex[w]), torch.empty_like(ex[s], dtype=torch.float16)
        _m.moe_int4_prepack(ex[w], ex[s], pw, ps)
        out[w], out[s] = pw, ps
    return out


class MoELayer:
    """Routed int4 experts + shared bf16 expert (+ optional K3 latent wrapper).

    `experts` holds the routed weights in the checkpoint layout; their scales
    are checked (moe_int4_check_scales) and they are permuted once into the
    fragment layout here."""

    SIDE_STREAM_MIN_T = 64  # tokens from which the shared expert runs on its own stream
    # tokens from which the bf16 expert input is converted once to the fp16 staging
    # format instead of by every tile of the grouped GEMMs: always (the decode kernel
    # then skips its per-wave conversion, measured 3.9% faster at 64 tokens)
    STAGED_ACT_MIN_T = 1

    def __init__(self, cfg: dict, router_w, router_b, experts: dict, shared: dict | None = None,
                 latent: dict | None = None):
        self.cfg = dict(cfg)
        # exact mode: 8-bit activation codes, or 16-bit with act_bits = 16
        if cfg["mode"] == "exact":
            self.mode = _m.MOE_MODE_EXACT_I16 if int(cfg.get("act_bits", 8)) == 16 else _m.MOE_MODE_EXACT_I8
        else:
            self.mode = _m.MOE_MODE_BF16
        self.router_w = router_w
        self.router_b = router_b
        # weight load: the scales must keep the fp16 dequantisation exact
        count = torch.empty(1, dtype=torch.int32, device=router_w.device)
        for name in ("sg", "su", "sd"):
            _m.moe_int4_check_scales(experts[name], count)
        self.ex = prepack_experts(experts)
        self.shared = shared
        self.latent = latent
        self.E, self.k, self.H, self.I = cfg["E"], cfg["k"], cfg["H"], cfg["I"]
        self.Kin = cfg.get("L") or cfg["H"]  # width the routed experts see
        # the K3 block's switches: renormalise the selected weights, RMSNorm the
        # routed sum before the latent up-projection (both on by default)
        self.renormalize = bool(cfg.get("renormalize", True))
        self.latent_norm = bool(cfg.get("latent_norm", True))
        # group-limited routing (1 group, scale 1: plain sigmoid top-k)
        self.n_group = int(cfg.get("n_group", 1))
        self.topk_group = int(cfg.get("topk_group", 1))
        self.routed_scale = float(cfg.get("routed_scale", 1.0))
        self._ws = {}
        self._side = None
        self.device = router_w.device
        if self.mode in (_m.MOE_MODE_EXACT_I8, _m.MOE_MODE_EXACT_I16) and (shared is not None or latent is not None):
            raise ValueError("exact mode is defined for the routed experts alone")

    @classmethod
    def from_numpy(cls, inp: dict, device="cuda"):
        """Upload the generator's numpy arrays (bf16 as uint16 bits)."""
        cfg = inp["cfg"]
        ex = inp["experts"]
        experts = {
            "wg": _u8(ex["wg"], device), "sg": _bf16(ex["sg"], device),
            "wu": _u8(ex["wu"], device), "su": _bf16(ex["su"], device),
            "wd": _u8(ex["wd"], device), "sd": _bf16(ex["sd"], device),
        }
        shared = None
        if inp.get("shared") is not None:
            shared = {n: _bf16(inp["shared"][n], device) for n in ("wg", "wu", "wd")}
        latent = None
        if inp.get("latent") is not None:
            latent = {n: _bf16(inp["latent"][n], device) for n in ("w_down", "w_up", "gain")}
        return cls(cfg, _bf16(inp["router_w"], device),
                   torch.from_numpy(np.ascontiguousarray(inp["router_b"], dtype=np.float32)).to(device),
                   experts, shared, latent)

    # ------------------------------------------------------------------
    def workspace(self, T: int) -> dict:
        """Device buffers for T tokens (allocated once per T and reused)."""
        if T in self._ws:
            return self._ws[T]
        dev, E, k, H, I, Kin = self.device, self.E, self.k, self.H, self.I, self.Kin
        S = T * k
        exact = self.mode in (_m.MOE_MODE_EXACT_I8, _m.MOE_MODE_EXACT_I16)
        codes = torch.int16 if self.mode == _m.MOE_MODE_EXACT_I16 else torch.int8
        staged = not exact and T >= self.STAGED_ACT_MIN_T
        w = {
            "route_ws": torch.empty(max(1, _m.moe_route_workspace_bytes(T, self.H, E)), dtype=torch.uint8, device=dev),
            "perm_ws": torch.empty(max(1, _m.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device=dev),
            "topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
            "counts": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_slot": torch.empty(S, dtype=torch.int32, device=dev),
            "slot_pos": torch.empty(S, dtype=torch.int32, device=dev),
            "h": torch.empty((S, I), dtype=codes if exact else torch.float16 if staged else torch.bfloat16,
                             device=dev),
            "h_scale": torch.empty((S, I // 32), dtype=torch.float32, device=dev) if exact else None,
            "y": torch.empty((S, Kin), dtype=torch.float32 if exact else torch.bfloat16, device=dev),
            "out": torch.empty((T, H), dtype=torch.float32 if exact else torch.bfloat16, device=dev),
        }
        if staged:
            w["act16"] = torch.empty((T, Kin), dtype=torch.float16, device=dev)
        if exact:
            w["qx"] = torch.empty((T, Kin), dtype=codes, device=dev)
            w["sx"] = torch.empty((T, Kin // 32), dtype=torch.float32, device=dev)
        dense_bytes = 0
        if self.shared is not None:
            Is = self.shared["wg"].shape[0]
            w["shared_h"] = torch.empty((T, Is), dtype=torch.bfloat16, device=dev)
            w["shared_out"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            shared_bytes = max(_m.moe_dense_workspace_bytes(T, 2 * Is, H), _m.moe_dense_workspace_bytes(T, H, Is))
            w["shared_ws"] = torch.empty(max(1, shared_bytes), dtype=torch.uint8, device=dev)
        if self.latent is not None:
            L = Kin
            w["x_lat"] = torch.empty((T, L), dtype=torch.bfloat16, device=dev)
            w["routed"] = torch.empty((T, L), dtype=torch.bfloat16, device=dev)
            w["normed"] = torch.empty((T, L), dtype=torch.bfloat16, device=dev)
            dense_bytes = max(dense_bytes, _m.moe_dense_workspace_bytes(T, L, H),
                              _m.moe_dense_workspace_bytes(T, H, L))
        w["dense_ws"] = torch.empty(max(1, dense_bytes), dtype=torch.uint8, device=dev)
        self._ws[T] = w
        return w

    def forward(self, x: torch.Tensor, marks: list | None = None) -> torch.Tensor:
        """x [T, H] bf16 -> out [T, H] (bf16, or fp32 in exact mode).  Returns the
        workspace's output buffer; the intermediates stay in ``workspace(T)``.

        The shared expert depends only on x, so for batches of at least
        ``SIDE_STREAM_MIN_T`` tokens it runs on a second stream, overlapping the
        router, the permutation and the routed GEMMs; the combine (or the latent
        up-projection) waits for it.  (At 64 tokens this measured 1% faster once the
        decode kernel's weight loads were non-temporal, slower before; smaller
        batches keep one stream.)  The side stream first
        waits for an event recorded on the current stream, which orders it after
        x and after the previous forward's use of its buffers.
        ``marks``: when a list is given, every call runs on the current stream and
        a timing event is appended after each as (call name, event)."""
        T = x.shape[0]
        w = self.workspace(T)
        if T == 0:
            return w["out"]
        side = None
        if self.shared is not None and marks is None and T >= self.SIDE_STREAM_MIN_T:
            if self._side is None:
                self._side = torch.cuda.Stream(device=self.device)
                self._ev_fork = torch.cuda.Event()
                self._ev_join = torch.cuda.Event()
            side = self._side
            self._ev_fork.record()
            side.wait_event(self._ev_fork)
            with torch.cuda.stream(side):
                self._shared_expert(x, w)
                self._ev_join.record()

        def mark(name):
            if marks is not None:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record()
                marks.append((name, ev))

        mark("start")
        E, k, H, I, Kin = self.E, self.k, self.H, self.I, self.Kin
        ex = self.ex
        if self.n_group == 1 and self.routed_scale == 1.0:
            _m.moe_route(x, self.router_w, self.router_b, k, self.renormalize, w["topk_idx"], w["topk_w"],
                         w["route_ws"])
        else:
            _m.moe_route_grouped(x, self.router_w, self.router_b, k, self.renormalize, self.n_group, self.topk_group,
                                 self.routed_scale, w["topk_idx"], w["topk_w"], w["route_ws"])
        mark("moe_route")
        _m.moe_permute(w["topk_idx"], E, w["counts"], w["offsets"], w["sorted_slot"], w["slot_pos"], w["perm_ws"])
        mark("moe_permute")
        act = x
        if self.latent is not None:
            _m.moe_linear_bf16(x, self.latent["w_down"], None, w["x_lat"], w["dense_ws"])
            mark("latent_down")
            act = w["x_lat"]
        shared_out = None
        if self.shared is not None:
            if side is None:
                self._shared_expert(x, w, mark)
            shared_out = w["shared_out"]
        if self.mode in (_m.MOE_MODE_EXACT_I8, _m.MOE_MODE_EXACT_I16):
            if self.mode == _m.MOE_MODE_EXACT_I16:
                _m.moe_quant_act_int16(act, w["qx"], w["sx"])
                mark("moe_quant_act_int16")
            else:
                _m.moe_quant_act_int8(act, w["qx"], w["sx"])
                mark("moe_quant_act_int8")
            _m.moe_int4_grouped_swiglu(self.mode, w["qx"], w["sx"], ex["wg"], ex["sg"], ex["wu"], ex["su"],
                                       w["offsets"], w["sorted_slot"], T, k, E, Kin, I, w["h"], w["h_scale"])
            gmode = self.mode
        elif "act16" in w:
            # bf16 arithmetic on activations converted once to the fp16 staging
            # format; h stays in that format between the two grouped calls
            _m.moe_act_f16p(act, w["act16"])
            mark("moe_act_f16p")
            gmode = _m.MOE_MODE_BF16_F16P
            _m.moe_int4_grouped_swiglu(gmode, w["act16"], None, ex["wg"], ex["sg"], ex["wu"], ex["su"],
                                       w["offsets"], w["sorted_slot"], T, k, E, Kin, I, w["h"], None)
        else:
            gmode = self.mode
            _m.moe_int4_grouped_swiglu(gmode, act, None, ex["wg"], ex["sg"], ex["wu"], ex["su"],
                                       w["offsets"], w["sorted_slot"], T, k, E, Kin, I, w["h"], None)
        mark("moe_int4_grouped_swiglu")
        _m.moe_int4_grouped_down(gmode, w["h"], w["h_scale"], ex["wd"], ex["sd"], w["offsets"], T, k, E, I,
                                 Kin, w["y"])
        mark("moe_int4_grouped_down")
        if side is not None:
            torch.cuda.current_stream().wait_event(self._ev_join)
        # the combine sees fp32 y in either exact mode
        cmode = _m.MOE_MODE_EXACT_I8 if self.mode == _m.MOE_MODE_EXACT_I16 else self.mode
        if self.latent is None:
            _m.moe_combine(cmode, w["y"], w["slot_pos"], w["topk_w"], shared_out, T, k, H, w["out"])
            mark("moe_combine")
        else:
            _m.moe_combine(self.mode, w["y"], w["slot_pos"], w["topk_w"], None, T, k, Kin, w["routed"])
            mark("moe_combine")
            up_in = w["routed"]
            if self.latent_norm:
                _m.moe_rmsnorm_bf16(w["routed"], self.latent["gain"], self.cfg["rms_eps"], w["normed"])
                mark("moe_rmsnorm_bf16")
                up_in = w["normed"]
            _m.moe_linear_bf16(up_in, self.latent["w_up"], shared_out, w["out"], w["dense_ws"])
            mark("latent_up")
        return w["out"]

    def capture(self, x: torch.Tensor) -> "LayerGraph":
        """Record one forward on the buffer ``x`` as a HIP graph (see LayerGraph)."""
        return LayerGraph(self, x)

    def _shared_expert(self, x, w, mark=None):
        _m.moe_dense_swiglu_bf16(x, self.shared["wg"], self.shared["wu"], w["shared_h"], w["shared_ws"])
        if mark:
            mark("shared_gate_up")
        _m.moe_linear_bf16(w["shared_h"], self.shared["wd"], None, w["shared_out"], w["shared_ws"])
        if mark:
            mark("shared_down")

    __call__ = forward


class LayerGraph:
    """One forward of a layer for a fixed batch size, recorded as a HIP graph
    (torch.cuda.CUDAGraph): a replay relaunches every call of the forward -- the
    same kernels, grids and buffers, the shared expert's side stream included --
    with one host call, so a decode loop pays no per-call launch gaps.

    ``x`` is the graph's input buffer: write the next batch into it (same shape),
    then ``replay()``.  The output buffer that replay() returns is the layer's
    workspace output for that T, overwritten by every replay and by eager
    forwards of the same T.  The forward allocates nothing and issues no memory
    set or copy, so the graph holds kernel nodes and the stream-fork/join
    dependencies only."""

    def __init__(self, layer: MoELayer, x: torch.Tensor):
        self.layer = layer
        self.x = x
        # one eager forward first, off the capture: it allocates the workspace
        # for this T, the side stream and its events
        s = torch.cuda.Stream(device=x.device)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            layer.forward(x)
        torch.cuda.current_stream().wait_stream(s)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out = layer.forward(x)

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        return self.out
