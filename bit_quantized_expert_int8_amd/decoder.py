"""Decode-step runtime over the C ABI: device-resident weights of a stack of MoE layers, caller-owned
workspaces, and the per-token sequence of library calls (RMSNorm -> router/top-k -> expert GEMVs ->
combine), optionally captured into one HIP graph per token.

PyTorch is used only to own device memory and streams; every step of the path runs in libmoeq4.so.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import torch

from . import moeq4 as q


@dataclasses.dataclass
class Shape:
    d: int
    n_experts: int
    k: int
    F: int
    S: int
    sb_dtype: int = q.MOE_BF16
    x_dtype: int = q.MOE_BF16
    act: int = q.MOE_ACT_GELU_TANH
    rms_norm: bool = False
    eps: float = 1e-6


@dataclasses.dataclass
class LayerWeights:
    pool: torch.Tensor            # uint8 [E][record_bytes]
    shared: Optional[torch.Tensor]  # uint8 [1][shared_record_bytes]
    router_w: torch.Tensor        # int8 [E][d]
    router_s: torch.Tensor        # float32 [E]
    gamma: Optional[torch.Tensor]  # float32 [d]


def _torch_dtype(dt: int):
    return torch.bfloat16 if dt == q.MOE_BF16 else torch.float32


def pack_layer(shape: Shape, fill_expert: Callable, fill_shared: Optional[Callable], router_w: torch.Tensor,
               router_s: torch.Tensor, gamma: Optional[torch.Tensor], device="cuda", stream=None) -> LayerWeights:
    """Quantize one layer's experts into device records with the library's encoder.

    ``fill_expert(e, w_gate_up, w_down)`` writes expert e's fp32 weights ([2F][d] and [d][F] CUDA tensors)
    in place; ``fill_shared(w_gate_up, w_down)`` the same for the shared expert (width S)."""
    d, F, S, E = shape.d, shape.F, shape.S, shape.n_experts
    rb = q.moe_record_bytes(d, F, shape.sb_dtype)
    pool = torch.empty((E, rb), dtype=torch.uint8, device=device)
    wgu = torch.empty((2 * F, d), dtype=torch.float32, device=device)
    wd = torch.empty((d, F), dtype=torch.float32, device=device)
    for e in range(E):
        fill_expert(e, wgu, wd)
        q.q4_pack_expert(wgu, wd, d, F, shape.sb_dtype, pool[e].data_ptr(), stream)
    shared = None
    if fill_shared is not None:
        srb = q.moe_record_bytes(d, S, shape.sb_dtype)
        shared = torch.empty((1, srb), dtype=torch.uint8, device=device)
        sgu = torch.empty((2 * S, d), dtype=torch.float32, device=device)
        sd = torch.empty((d, S), dtype=torch.float32, device=device)
        fill_shared(sgu, sd)
        q.q4_pack_expert(sgu, sd, d, S, shape.sb_dtype, shared.data_ptr(), stream)
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return LayerWeights(pool, shared, router_w.to(device).contiguous(), router_s.to(device).contiguous(),
                        None if gamma is None else gamma.to(device).contiguous())


def layer_kernel_fits(shape: Shape, T: int) -> bool:
    """Whether moe_decode_layer (batch 1) supports this shape."""
    return (T == 1 and shape.d <= 4096 and shape.S <= 4096 and shape.F <= 1024 and shape.n_experts <= 256
            and 1 <= shape.k <= min(32, shape.n_experts))


class MoEDecoder:
    """Runs T tokens through a stack of MoE layers (T = 1 is decode).

    Four ways to run the layers, all through the library:
      "layer"     moe_decode_layer per layer: one launch each; the default for T = 1 within that kernel's
                  limits
      "stack"     one launch for the whole step (moe_decode_stack, <= 32 layers); layer() as "layer"
      "fused"     moe_norm_router_topk (RMSNorm inside the router) then q4_expert_gemv_combine (expert
                  GEMVs with the combine + residual in the down launch's tail); the default otherwise
      "separate"  moe_rmsnorm, moe_router_topk, q4_expert_gemv, moe_combine
    "fused" and "separate" give the same routing and, on the same normalized input, the same output bits."""

    def __init__(self, shape: Shape, layers: list, T: int = 1, device="cuda", mode: Optional[str] = None,
                 record_u: bool = False):
        self.shape, self.layers, self.T = shape, layers, T
        if mode is None:
            mode = "layer" if layer_kernel_fits(shape, T) else "fused"
        if mode not in ("stack", "layer", "fused", "separate") or \
                (mode in ("stack", "layer") and not layer_kernel_fits(shape, T)) or (mode == "stack" and len(layers) > 32):
            raise ValueError(f"mode {mode!r} not available for this shape / batch")
        self.mode = mode
        s = shape
        self.device = device
        self.routed_pools = [q.pool(L.pool, L.pool.shape[1], s.n_experts, s.d, s.F, s.sb_dtype) for L in layers]
        self.shared_pools = [None if L.shared is None else q.pool(L.shared, L.shared.shape[1], 1, s.d, s.S, s.sb_dtype)
                             for L in layers]
        xdt = _torch_dtype(s.x_dtype)
        self.u = torch.empty((T, s.d), dtype=xdt, device=device)            # expert/router input
        L = len(layers)
        # routing of every layer is kept (the last token's), so it can be inspected or replayed
        self.ids_all = torch.empty((L, T, s.k), dtype=torch.int32, device=device)
        self.weights_all = torch.empty((L, T, s.k), dtype=torch.float32, device=device)
        self.logits_all = torch.empty((L, T, s.n_experts), dtype=torch.float32, device=device)
        self.ids, self.weights, self.logits = self.ids_all[0], self.weights_all[0], self.logits_all[0]
        # with record_u, the single-launch modes also keep every layer's normalized activation (the last token's)
        self.u_all = torch.empty((L, T, s.d), dtype=xdt, device=device) if record_u else None
        self.y_routed = torch.empty((T, s.k, s.d), dtype=torch.float32, device=device)
        self.y_shared = torch.empty((T, s.d), dtype=torch.float32, device=device)
        self.router_ws_bytes = q.moe_router_workspace_bytes(T, s.n_experts)
        self.router_ws = torch.zeros(self.router_ws_bytes, dtype=torch.uint8, device=device)
        self.gemv_ws_bytes = max(q.q4_expert_gemv_workspace_bytes(rp, s.k, sp, T)
                                 for rp, sp in zip(self.routed_pools, self.shared_pools))
        self.gemv_ws = torch.empty(max(self.gemv_ws_bytes, 256), dtype=torch.uint8, device=device)
        # the fused call's workspace ends in per-tile counters that must start at zero (calls leave them zero)
        self.fused_ws_bytes = max(q.q4_expert_gemv_combine_workspace_bytes(rp, s.k, sp, T)
                                  for rp, sp in zip(self.routed_pools, self.shared_pools))
        self.fused_ws = torch.zeros(max(self.fused_ws_bytes, 256), dtype=torch.uint8, device=device)
        # the single-launch layer's workspace: counters at the front start at zero and calls leave them zero
        self.layer_ws_bytes = q.moe_decode_layer_workspace_bytes(s.d, s.n_experts, s.k, s.F,
                                                                 s.S if layers and layers[0].shared is not None else 0)
        self.layer_ws = torch.zeros(max(self.layer_ws_bytes, 256), dtype=torch.uint8, device=device)
        if mode == "stack":
            S_ = s.S if layers and layers[0].shared is not None else 0
            self.stack_ws_bytes = q.moe_decode_stack_workspace_bytes(L, s.d, s.n_experts, s.k, s.F, S_)
            self.stack_ws = torch.zeros(self.stack_ws_bytes, dtype=torch.uint8, device=device)
            self.stack_descs = q.stack_layers([
                {"router_w_dev": W.router_w, "router_scale_dev": W.router_s,
                 "gamma_dev": W.gamma if s.rms_norm else None, "routed_base_dev": W.pool, "shared_base_dev": W.shared,
                 "ids_dev": self.ids_all[l], "weights_dev": self.weights_all[l], "logits_dev": self.logits_all[l],
                 "u_dev": None if self.u_all is None else self.u_all[l]}
                for l, W in enumerate(layers)])
        self.graph = None

    # one layer: x_in -> x_out (both [T][d] in the activation dtype)
    def layer(self, l: int, x_in: torch.Tensor, x_out: torch.Tensor, forced_ids: Optional[torch.Tensor] = None,
              routed_pool=None, ids: Optional[torch.Tensor] = None, stream=None) -> None:
        s, L, T = self.shape, self.layers[l], self.T
        if self.mode in ("stack", "layer"):
            self._layer_single_launch(l, x_in, x_out, forced_ids, routed_pool, ids, stream)
            return
        if self.mode == "fused":
            self._layer_fused(l, x_in, x_out, forced_ids, routed_pool, ids, stream)
            return
        if s.rms_norm:
            q.moe_rmsnorm(x_in, s.x_dtype, L.gamma, s.eps, T, s.d, self.u, s.x_dtype, stream)
            u = self.u
        else:
            u = x_in
        lid, lw, lg = self.ids_all[l], self.weights_all[l], self.logits_all[l]
        q.moe_router_topk(u, s.x_dtype, T, s.d, L.router_w, L.router_s, s.n_experts, s.k, forced_ids, lid, lw, lg,
                          self.router_ws, self.router_ws_bytes, stream)
        q.q4_expert_gemv(routed_pool or self.routed_pools[l], lid if ids is None else ids, s.k, self.shared_pools[l],
                         u, s.x_dtype, T, s.act, self.y_routed, self.y_shared, self.gemv_ws, self.gemv_ws_bytes, stream)
        q.moe_combine(self.y_routed, lw, self.y_shared if self.shared_pools[l] is not None else None,
                      x_in if s.rms_norm else None, s.x_dtype, T, s.k, s.d, x_out, s.x_dtype, stream)

    def _layer_single_launch(self, l, x_in, x_out, forced_ids, routed_pool, ids, stream) -> None:
        s, L = self.shape, self.layers[l]
        q.moe_decode_layer(x_in, s.x_dtype, L.gamma if s.rms_norm else None, s.eps, s.rms_norm, L.router_w, L.router_s,
                           s.n_experts, s.k, forced_ids, routed_pool or self.routed_pools[l], ids,
                           self.shared_pools[l], s.act, self.ids_all[l], self.weights_all[l], self.logits_all[l], x_out,
                           self.layer_ws, self.layer_ws_bytes, stream,
                           u=None if self.u_all is None else self.u_all[l])

    def layer_part(self, part: int, l: int, x_in: torch.Tensor, x_out: torch.Tensor,
                   forced_ids: Optional[torch.Tensor] = None, routed_pool=None, ids: Optional[torch.Tensor] = None,
                   stream=None) -> None:
        """One layer as two launches (moe_decode_layer_part): part 1 = router + shared expert, part 2 = routed
        experts + combine; call 1 then 2 (an expert cache may fill the routed slots in between)."""
        s, L = self.shape, self.layers[l]
        q.moe_decode_layer_part(part, x_in, s.x_dtype, L.gamma if s.rms_norm else None, s.eps, s.rms_norm, L.router_w,
                                L.router_s, s.n_experts, s.k, forced_ids, routed_pool or self.routed_pools[l], ids,
                                self.shared_pools[l], s.act, self.ids_all[l], self.weights_all[l], self.logits_all[l],
                                None if self.u_all is None else self.u_all[l], x_out, self.layer_ws,
                                self.layer_ws_bytes, stream)

    def _layer_fused(self, l, x_in, x_out, forced_ids, routed_pool, ids, stream) -> None:
        s, L, T = self.shape, self.layers[l], self.T
        lid, lw, lg = self.ids_all[l], self.weights_all[l], self.logits_all[l]
        if s.rms_norm:
            q.moe_norm_router_topk(x_in, s.x_dtype, L.gamma, s.eps, T, s.d, L.router_w, L.router_s, s.n_experts, s.k,
                                   forced_ids, lid, lw, lg, self.u, self.router_ws, self.router_ws_bytes, stream)
            u = self.u
        else:
            q.moe_router_topk(x_in, s.x_dtype, T, s.d, L.router_w, L.router_s, s.n_experts, s.k, forced_ids, lid, lw,
                              lg, self.router_ws, self.router_ws_bytes, stream)
            u = x_in
        q.q4_expert_gemv_combine(routed_pool or self.routed_pools[l], lid if ids is None else ids, s.k,
                                 self.shared_pools[l], u, s.x_dtype, T, s.act, lw, x_in if s.rms_norm else None,
                                 s.x_dtype, x_out, s.x_dtype, self.fused_ws, self.fused_ws_bytes, stream)

    def step(self, x: torch.Tensor, out: torch.Tensor, stream=None) -> None:
        """Run every layer: x -> out (one launch in "stack" mode, else layer by layer through an internal
        buffer)."""
        n = len(self.layers)
        if self.mode == "stack":
            s = self.shape
            q.moe_decode_stack(self.stack_descs, n, x, s.x_dtype, s.eps, s.rms_norm, s.n_experts, s.k,
                               self.routed_pools[0], self.shared_pools[0], s.act, out, self.stack_ws,
                               self.stack_ws_bytes, stream)
            return
        if not hasattr(self, "_tmp"):
            self._tmp = torch.empty_like(out)
        bufs = [self._tmp, out] if n % 2 == 0 else [out, self._tmp]
        src = x
        for l in range(n):
            dst = bufs[l % 2]
            self.layer(l, src, dst, stream=stream)
            src = dst

    def status(self) -> int:
        """The sticky error words of the single-launch kernels' workspaces, OR-ed (0 = every bounded wait inside
        them completed; nonzero = a wait ran out and the results of that call are invalid): the layer workspace
        (moe_decode_layer, its two parts) and the stack workspace (moe_decode_stack), whichever this decoder
        holds, whatever its mode.  Synchronizes."""
        torch.cuda.synchronize()
        st = 0
        for ws in (getattr(self, "layer_ws", None), getattr(self, "stack_ws", None)):
            if ws is not None:
                st |= int(ws[:4].view(torch.int32).item())
        return st

    def check_status(self) -> None:
        """Raise if a bounded wait inside the single-launch kernels ran out since the workspace was zeroed."""
        st = self.status()
        if st:
            raise RuntimeError(f"MoE decode kernel: a bounded wait ran out (status word {st:#x}); results are invalid")

    def capture(self, x: torch.Tensor, out: torch.Tensor) -> torch.cuda.CUDAGraph:
        """Capture one whole-stack step into a HIP graph (replay with graph.replay())."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step(x, out, stream=s)          # warm-up outside capture
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(x, out, stream=torch.cuda.current_stream())
        self.graph = g
        return g
