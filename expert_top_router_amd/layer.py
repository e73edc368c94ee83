"""Device buffers of one MoE layer and the call sequence of its forward step.

The buffers are laid out as the C ABI describes them (include/occ.h); torch
only allocates them.  ``forward()`` issues occ_route_topk, occ_build_brim,
occ_dispatch, occ_expert_ffn and occ_combine back to back on one stream with
no host synchronisation; ``coactivation()`` is the placement side output.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import (desc_of, make_brim, occ_backward_workspace_bytes, occ_build_brim,
               occ_build_brim_pruned, occ_coactivation, occ_combine, occ_expert_backward,
               occ_expert_backward_kept, occ_expert_ffn_keep,
               occ_grad_combine, occ_grad_dispatch, occ_router_backward, occ_shared_backward,
               occ_combine_direct, occ_dispatch, occ_dispatch_direct, occ_expert_down,
               occ_expert_ffn, occ_expert_up, occ_ffn_workspace_bytes, occ_route_topk,
               occ_route_topk_ws, occ_route_workspace_bytes,
               occ_workspace_bytes)


def _torch():
    import torch
    return torch


def to_device(a: np.ndarray, device="cuda"):
    """numpy (float32, or bfloat16 kept as uint16 bits, or int32) -> torch."""
    torch = _torch()
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_host(t) -> np.ndarray:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@dataclass
class Weights:
    x: object
    w_router: object
    w_gate_up: object
    w_down: object
    w_gate_up_sh: Optional[object] = None
    w_down_sh: Optional[object] = None


class MoELayer:
    """All device buffers of one layer configuration (duck-typed ``cfg`` with
    T, d, E, I, k, D, dtype, renorm, n_shared, I_shared)."""

    def __init__(self, cfg, weights: Weights, slot_expert, with_logits=False, device="cuda",
                 budget=None, rescale=1):
        """budget: None for the exact layer, else the all-to-all budget of
        collaboration pruning (devices kept per token, occ_build_brim_pruned)."""
        torch = _torch()
        self.cfg = cfg
        self.device = device
        self.budget = budget
        self.rescale = rescale
        self.desc = desc_of(cfg)
        self.slot_expert = np.ascontiguousarray(slot_expert, dtype=np.int32)
        self.w = weights
        T, d, E, k, D = cfg.T, cfg.d, cfg.E, cfg.k, cfg.D
        L = E // D
        S_max = T * min(k, D)
        R = T * k
        el = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        i32, f32 = torch.int32, torch.float32

        def buf(shape, dt):
            # at least one element so that no pointer is NULL at T = 0
            n = int(np.prod(shape))
            return torch.empty(max(n, 1), dtype=dt, device=device)[:n].view(*shape)

        self.topk_idx = buf((T, k), i32)
        self.topk_w = buf((T, k), f32)
        self.logits = buf((T, E), f32) if with_logits else None
        self.brim0 = buf((D, T), i32)
        self.brim1 = buf((L, S_max), i32)
        self.sfd_offset = buf((D + 1,), i32)
        self.slot_offset = buf((E + 1,), i32)
        self.sfd_token = buf((S_max,), i32)
        self.epd_token = buf((R,), i32)
        self.epd_sfd = buf((R,), i32)
        self.epd_w = buf((R,), f32)
        self.S = buf((1,), i32)
        self.brim = make_brim(brim0=self.brim0, brim1=self.brim1, sfd_offset=self.sfd_offset,
                              slot_offset=self.slot_offset, sfd_token=self.sfd_token,
                              epd_token=self.epd_token, epd_sfd=self.epd_sfd, epd_w=self.epd_w,
                              S=self.S)
        self.ws_bytes = occ_workspace_bytes(self.desc)
        self.ws = buf((self.ws_bytes,), torch.uint8)
        # routing without logits goes through the candidate filter
        # (occ_route_topk_ws) where it measured faster than the plain kernel
        # (at least 96 experts and 32768 tokens: the plain kernel's work grows
        # with E, the filter's with the candidates) and the router is
        # bf16-representable (checked once here); route_filtered = False
        # forces the plain kernel
        wr = weights.w_router
        self.route_filtered = (cfg.E >= 96 and cfg.T >= 32768 and
                               bool(torch.equal(wr, wr.to(torch.bfloat16).to(wr.dtype))))
        self.route_ws_bytes = occ_route_workspace_bytes(self.desc)
        self.route_ws = buf((self.route_ws_bytes,), torch.uint8) if self.route_ws_bytes else None
        self.sfd = buf((S_max, d), el)
        self.epd = buf((R, d), el)
        self.h_bytes = occ_ffn_workspace_bytes(self.desc)
        self.h_ws = buf((self.h_bytes,), torch.uint8)
        self.out_epd = buf((R, d), el)
        self.shared_out = buf((T, d), el) if cfg.n_shared else None
        self.out_sfd = buf((S_max, d), el)
        self.y = buf((T, d), el)
        self.counts = buf((E, E), i32)

    # ---- the hot path ------------------------------------------------------
    def route(self, stream=None):
        if self.logits is None and self.route_filtered and self.route_ws is not None:
            occ_route_topk_ws(self.desc, self.w.x, self.w.w_router, self.topk_idx, self.topk_w,
                              self.route_ws, self.route_ws_bytes, stream)
        else:
            occ_route_topk(self.desc, self.w.x, self.w.w_router, self.topk_idx, self.topk_w,
                           self.logits, stream)
        # the router gradient needs the logits of the forward it differentiates
        self._routed_with_logits = self.logits is not None

    def build_brim(self, stream=None):
        if self.budget is None:
            occ_build_brim(self.desc, self.topk_idx, self.topk_w, self.slot_expert, self.brim,
                           self.ws, self.ws_bytes, stream)
        else:
            occ_build_brim_pruned(self.desc, self.topk_idx, self.topk_w, self.slot_expert,
                                  self.budget, self.rescale, self.brim, self.ws, self.ws_bytes,
                                  stream)

    def dispatch(self, stream=None):
        occ_dispatch(self.desc, self.w.x, self.brim, self.sfd, self.epd, stream)

    def _shared(self):
        if self.cfg.n_shared:
            return self.w.x, self.w.w_gate_up_sh, self.w.w_down_sh, self.shared_out
        return None, None, None, None

    def expert_ffn(self, stream=None):
        x, gu, dn, so = self._shared()
        occ_expert_ffn(self.desc, self.epd, self.brim, self.slot_expert, self.w.w_gate_up,
                       self.w.w_down, self.h_ws, self.h_bytes, self.out_epd, x, gu, dn, so,
                       stream)

    def expert_up(self, stream=None):
        x, gu, _, _ = self._shared()
        occ_expert_up(self.desc, self.epd, self.brim, self.slot_expert, self.w.w_gate_up,
                      self.h_ws, self.h_bytes, x, gu, stream)

    def expert_down(self, stream=None):
        _, _, dn, so = self._shared()
        occ_expert_down(self.desc, self.brim, self.slot_expert, self.w.w_down, self.h_ws,
                        self.h_bytes, self.out_epd, dn, so, stream)

    def combine(self, stream=None):
        occ_combine(self.desc, self.out_epd, self.brim, self.shared_out, self.out_sfd, self.y,
                    stream)

    def forward(self, stream=None):
        self.route(stream)
        self.build_brim(stream)
        self.dispatch(stream)
        self.expert_ffn(stream)
        self.combine(stream)

    # ---- the conventional per-(token, expert) strategy ------------------------
    def dispatch_direct(self, stream=None):
        occ_dispatch_direct(self.desc, self.w.x, self.brim, self.epd, stream)

    def combine_direct(self, stream=None):
        occ_combine_direct(self.desc, self.out_epd, self.brim, self.shared_out, self.y, stream)

    def forward_direct(self, stream=None):
        self.route(stream)
        self.build_brim(stream)
        self.dispatch_direct(stream)
        self.expert_ffn(stream)
        self.combine_direct(stream)

    # ---- backward (bf16) -----------------------------------------------------
    def _grad_buffers(self):
        if getattr(self, "dy", None) is not None:
            return
        torch = _torch()
        cfg = self.cfg
        T, d, E, k, D = cfg.T, cfg.d, cfg.E, cfg.k, cfg.D
        S_max, R = T * min(k, D), T * k
        el = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        f32 = torch.float32

        def buf(shape, dt):
            n = int(np.prod(shape))
            return torch.empty(max(n, 1), dtype=dt, device=self.device)[:n].view(*shape)

        if self.logits is None:
            self.logits = buf((T, E), f32)
        self.dy = buf((T, d), el)
        self.d_out_sfd = buf((S_max, d), el)
        self.d_out_epd = buf((R, d), el)
        self.dw_epd = buf((R,), f32)
        self.bwd_bytes = occ_backward_workspace_bytes(self.desc)
        self.bwd_ws = buf((self.bwd_bytes,), torch.uint8)
        self.d_epd = buf((R, d), el)
        self.dw_gate_up = buf((E, 2 * cfg.I, d), f32)
        self.dw_down = buf((E, d, cfg.I), f32)
        self.dlogits = buf((T, E), f32)
        self.dx_router = buf((T, d), f32)
        self.dw_router = buf((E, d), f32)
        self.d_sfd = buf((S_max, d), el)
        self.dx = buf((T, d), el)
        self.gu = buf((R, 2 * cfg.I), el)  # kept [G | U] (forward_keep)
        if cfg.n_shared:
            self.dx_shared = buf((T, d), el)
            self.dw_gate_up_sh = buf((cfg.n_shared, 2 * cfg.I_shared, d), f32)
            self.dw_down_sh = buf((cfg.n_shared, d, cfg.I_shared), f32)
        else:
            self.dx_shared = self.dw_gate_up_sh = self.dw_down_sh = None

    def grad_combine(self, stream=None):
        occ_grad_combine(self.desc, self.dy, self.brim, self.out_epd, self.d_out_sfd,
                         self.d_out_epd, self.dw_epd, stream)

    def expert_backward(self, stream=None):
        occ_expert_backward(self.desc, self.epd, self.brim, self.slot_expert, self.w.w_gate_up,
                            self.w.w_down, self.h_ws, self.h_bytes, self.d_out_epd, self.bwd_ws,
                            self.bwd_bytes, self.d_epd, self.dw_gate_up, self.dw_down, stream)

    # ---- training steps that keep [G | U] instead of recomputing it -----------
    def expert_ffn_keep(self, stream=None):
        self._grad_buffers()
        occ_expert_ffn_keep(self.desc, self.epd, self.brim, self.slot_expert, self.w.w_gate_up,
                            self.w.w_down, self.h_ws, self.h_bytes, self.gu, self.out_epd, stream)

    def expert_backward_kept(self, stream=None):
        occ_expert_backward_kept(self.desc, self.epd, self.brim, self.slot_expert,
                                 self.w.w_gate_up, self.w.w_down, self.h_ws, self.h_bytes,
                                 self.gu, self.d_out_epd, self.bwd_ws, self.bwd_bytes, self.d_epd,
                                 self.dw_gate_up, self.dw_down, stream)

    def forward_keep(self, stream=None):
        """forward() with the expert FFN keeping [G | U] for backward_kept()
        (and the logits the router gradient needs)."""
        self._grad_buffers()
        self.route(stream)
        self.build_brim(stream)
        self.dispatch(stream)
        self.expert_ffn_keep(stream)
        self.combine(stream)

    def backward_kept(self, dy=None, stream=None):
        """backward() after forward_keep(): the expert backward reads the kept
        [G | U] instead of recomputing it."""
        self._require_logits()
        self._grad_buffers()
        if dy is not None:
            self.dy.copy_(dy)
        self.grad_combine(stream)
        self.expert_backward_kept(stream)
        self.router_backward(stream)
        self.grad_dispatch(stream)

    def router_backward(self, stream=None):
        occ_router_backward(self.desc, self.w.x, self.w.w_router, self.logits, self.topk_idx,
                            self.topk_w, self.slot_expert, self.brim, self.dw_epd, self.dlogits,
                            self.dx_router, self.dw_router, self.bwd_ws, self.bwd_bytes, stream)

    def shared_backward(self, stream=None):
        """The shared experts' gradients (layers with shared experts)."""
        if self.cfg.n_shared:
            occ_shared_backward(self.desc, self.w.x, self.w.w_gate_up_sh, self.w.w_down_sh,
                                self.h_ws, self.h_bytes, self.dy, self.bwd_ws, self.bwd_bytes,
                                self.dx_shared, self.dw_gate_up_sh, self.dw_down_sh, stream)

    def grad_dispatch(self, stream=None):
        occ_grad_dispatch(self.desc, self.d_epd, self.brim, self.dx_router, self.d_sfd, self.dx,
                          stream, dx_shared=self.dx_shared)

    def backward(self, dy=None, stream=None):
        """Gradients of the last forward (which must have kept its logits:
        construct with with_logits=True, or call prepare_backward() first)
        for the upstream gradient dy (bf16 [T, d]; self.dy when None)."""
        self._require_logits()
        self._grad_buffers()
        if dy is not None:
            self.dy.copy_(dy)
        self.grad_combine(stream)
        self.expert_backward(stream)
        self.router_backward(stream)
        self.shared_backward(stream)
        self.grad_dispatch(stream)

    def _require_logits(self):
        if not getattr(self, "_routed_with_logits", False):
            raise RuntimeError("the last forward did not keep its logits: construct the layer "
                               "with with_logits=True or call prepare_backward() (or use "
                               "forward_keep()) before the forward")

    def prepare_backward(self):
        """Allocate the gradient buffers (and the logits the router gradient needs)."""
        self._grad_buffers()

    def coactivation(self, accumulate=0, stream=None):
        occ_coactivation(self.desc, self.topk_idx, self.counts, accumulate, stream)

    # ---- test support --------------------------------------------------------
    def poison(self):
        """Fill every output with a recognisable pattern (unwritten entries
        then show up in the comparisons)."""
        torch = _torch()
        for t in (self.topk_idx, self.brim0, self.brim1, self.sfd_offset, self.slot_offset,
                  self.sfd_token, self.epd_token, self.epd_sfd, self.S, self.counts):
            t.fill_(0x7A7A7A7A)
        for t in (self.topk_w, self.epd_w):
            t.fill_(float("nan"))
        for t in (self.sfd, self.epd, self.out_epd, self.out_sfd, self.y, self.shared_out,
                  self.logits):
            if t is not None:
                t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(-1)

    def host(self, name):
        return to_host(getattr(self, name))


def router_f32(w_router: np.ndarray) -> np.ndarray:
    """The router in fp32, as occ_route_topk takes it (bf16 widens exactly)."""
    if w_router.dtype == np.uint16:
        return (w_router.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(w_router, dtype=np.float32)


def upload_inputs(inp, device="cuda") -> Weights:
    """Device copies of ``workloads.LayerInputs`` (router widened to fp32)."""
    def dev(a):
        return None if a is None else to_device(a, device)
    return Weights(dev(inp.x), dev(router_f32(inp.w_router)), dev(inp.w_gate_up),
                   dev(inp.w_down), dev(inp.w_gate_up_sh), dev(inp.w_down_sh))
