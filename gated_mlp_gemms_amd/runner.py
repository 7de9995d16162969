"""Device buffers for one MLP problem and the calls of one training step through the C ABI.

A ``MlpRunner`` holds the inputs, the outputs, the saved pre-activation and the workspaces of a
problem in HBM, so a caller (bench, tests, smoke) can run ``forward()`` / ``backward()`` /
``forward_infer()`` repeatedly without allocating. It only marshals: every step runs in the
library's kernels.
"""
from __future__ import annotations

import torch

from . import (GATED_ACTS, make_desc, make_fp8, mlp_bwd, mlp_fp8_next_scale, mlp_fwd, mlp_fwd_infer,
               mlp_quantize_e4m3, mlp_quantize_weight_e4m3, mlp_quantize_workspace_bytes, mlp_weight_amax_slots,
               workspace_bytes)

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
POST_HEADROOM = 1.03   # delayed post scale = amax * 1.03 / 448, floor 1e-6
POST_FLOOR = 1e-6
GRAD_SCALE = 2.0 ** -6  # static e5m2 scale of dout; also the bootstrap dpre scale
DPRE_HEADROOM = 1.25    # delayed dpre scale = amax * 1.25 / 57344, floor 1e-12
DPRE_FLOOR = 1e-12
EXACT_SCALE_CALLS = 16  # weight scales are exact for this many quantize() calls, then one call delayed


class MlpRunner:
    def __init__(self, *, act, dtype, M, d_in, hidden, d_out, gate_mult=1.0, down_mult=1.0,
                 gate_mode="outside", recompute=False, grad_accum=False, fp8_fwd=False, fp8_bwd=False,
                 save_act=False, tensors: dict, device="cuda", dpreact_in_place=False):
        self.gated = act in GATED_ACTS
        self.grad_accum = grad_accum
        self.fp8 = fp8_fwd
        self.fp8_bwd = fp8_bwd
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}.get(dtype, dtype)
        self.desc = make_desc(M, d_in, hidden, d_out, act, tdt, gate_mult, down_mult, gate_mode,
                              recompute, fp8_fwd, fp8_bwd, save_act)
        dev = torch.device(device)
        up = {k: v.to(dev) for k, v in tensors.items()}
        self.t = up
        self.x, self.dout = up["x"], up["dout"]
        self.w_gate = up["w_gate"] if self.gated else up["w1"]
        self.w_up = up["w_up"] if self.gated else None
        self.w_down = up["w_down"] if self.gated else up["w2"]
        P = 2 * hidden if self.gated else hidden
        self.out = torch.empty(M, d_out, dtype=tdt, device=dev)
        self.out_infer = torch.empty(M, d_out, dtype=tdt, device=dev)
        # the fp8-gradient backward keeps its pre-activation in fp32; with save_act the [M, P]
        # pre-activation is followed by the [M, H] activation in one buffer
        sdt = torch.float32 if fp8_bwd else tdt
        self.saved, self.saved_act = None, None
        if not recompute:
            buf = torch.empty(M * (P + (hidden if save_act else 0)), dtype=sdt, device=dev)
            self.saved = buf[: M * P].view(M, P)
            if save_act:
                self.saved_act = buf[M * P:].view(M, hidden)
        self.dpreact = self.saved if (dpreact_in_place and not recompute) else torch.empty(M, P, dtype=tdt, device=dev)
        self.dx = torch.empty(M, d_in, dtype=tdt, device=dev)
        gdt = torch.float32 if grad_accum else tdt
        if grad_accum:
            names = ("dw_gate", "dw_up", "dw_down") if self.gated else ("dw1", "dw2")
            self.grad_init = {k: up[k].clone() for k in names}
            self.dw_gate = up[names[0]]
            self.dw_up = up["dw_up"] if self.gated else None
            self.dw_down = up[names[-1]]
        else:
            self.dw_gate = torch.empty(hidden, d_in, dtype=gdt, device=dev)
            self.dw_up = torch.empty(hidden, d_in, dtype=gdt, device=dev) if self.gated else None
            self.dw_down = torch.empty(d_out, hidden, dtype=gdt, device=dev)
        self.ws_fwd = torch.empty(workspace_bytes(self.desc, "fwd"), dtype=torch.uint8, device=dev)
        self.ws_inf = torch.empty(workspace_bytes(self.desc, "fwd_infer"), dtype=torch.uint8, device=dev)
        self.ws_bwd = torch.empty(workspace_bytes(self.desc, "bwd"), dtype=torch.uint8, device=dev)
        self.fp8_args = None
        if fp8_fwd:
            self.x_q = torch.empty(M, d_in, dtype=torch.uint8, device=dev)
            self.w1_q = torch.empty(hidden, d_in, dtype=torch.uint8, device=dev)
            self.w2_q = torch.empty(d_out, hidden, dtype=torch.uint8, device=dev)
            # one fp32 slot each: s_x, s_w1, s_w2, s_post, post_amax, s_grad, s_dpre, dpre_amax
            self.scales = torch.zeros(8, dtype=torch.float32, device=dev)
            self.scales[3] = 1.0              # bootstrap post scale
            self.scales[5] = GRAD_SCALE
            self.scales[6] = GRAD_SCALE       # bootstrap dpre scale
            self.ws_q = torch.empty(mlp_quantize_workspace_bytes(), dtype=torch.uint8, device=dev)
            # per-tile amax each weight quantize records for the next call's delayed scale
            self.w1_amax = torch.zeros(mlp_weight_amax_slots(hidden, d_in), dtype=torch.float32, device=dev)
            self.w2_amax = torch.zeros(mlp_weight_amax_slots(d_out, hidden), dtype=torch.float32, device=dev)
            self.quantize_calls = 0
            s = self.scales
            sp = [s[i:i + 1].data_ptr() for i in range(8)]
            extra = {}
            if fp8_bwd:   # transposed e4m3 weight caches (the page's column-major copies)
                self.w1t_q = torch.empty(d_in, hidden, dtype=torch.uint8, device=dev)
                self.w2t_q = torch.empty(hidden, d_out, dtype=torch.uint8, device=dev)
                extra = dict(w1t_q=self.w1t_q, w2t_q=self.w2t_q, s_grad=sp[5], s_dpre=sp[6], dpre_amax=sp[7])
            self.fp8_args = make_fp8(self.x_q, self.w1_q, self.w2_q, sp[0], sp[1], sp[2], sp[3], sp[4], **extra)

    # ---- steps
    def quantize(self):
        """Per-tensor e4m3 of x (exact scale every call) and of the weight caches W1, W2 (row-major,
        plus the transposed copies with fp8_bwd): exact scales for the first EXACT_SCALE_CALLS
        calls, then the scale of the amax the previous call recorded."""
        s = self.scales
        exact = self.quantize_calls < EXACT_SCALE_CALLS
        self.quantize_calls += 1
        mlp_quantize_e4m3(self.x, self.x_q, s[0:1], self.ws_q)
        mlp_quantize_weight_e4m3(self.w_gate, exact, s[1:2], self.w1_amax, dst=self.w1_q,
                                 dst_t=self.w1t_q if self.fp8_bwd else None, ld_t=self.w_gate.shape[0])
        mlp_quantize_weight_e4m3(self.w_down, exact, s[2:3], self.w2_amax, dst=self.w2_q,
                                 dst_t=self.w2t_q if self.fp8_bwd else None, ld_t=self.w_down.shape[0])

    def refresh_dpre_scale(self):
        """Host side of the delayed dpre scale: next = max(amax * 1.25/57344, 1e-12), kept when
        amax is 0; amax is cleared. Synchronizes (reads amax)."""
        amax = float(self.scales[7].item())
        prev = float(self.scales[6].item())
        self.scales[6] = mlp_fp8_next_scale(amax, prev, DPRE_HEADROOM / E5M2_MAX, DPRE_FLOOR)
        self.scales[7] = 0.0

    def refresh_post_scale(self):
        """Host side of the delayed post scale: next = max(amax * 1.03/448, 1e-6), kept when
        amax is 0; amax is cleared. Synchronizes (reads amax)."""
        amax = float(self.scales[4].item())
        prev = float(self.scales[3].item())
        self.scales[3] = mlp_fp8_next_scale(amax, prev, POST_HEADROOM / E4M3_MAX, POST_FLOOR)
        self.scales[4] = 0.0

    def forward(self):
        mlp_fwd(self.desc, self.x, self.w_gate, self.w_up, self.w_down, self.out, self.saved,
                self.fp8_args, self.ws_fwd)

    def forward_infer(self):
        mlp_fwd_infer(self.desc, self.x, self.w_gate, self.w_up, self.w_down, self.out_infer,
                      self.fp8_args, self.ws_inf)

    def backward(self, dx=True, dw_gate=True, dw_down=True, dpreact=True):
        mlp_bwd(self.desc, self.dout, self.x, self.w_gate, self.w_up, self.w_down, self.saved,
                self.dpreact if (dpreact and not self.fp8_bwd) else None, self.dx if dx else None,
                self.dw_gate if dw_gate else None, self.dw_up if dw_gate else None,
                self.dw_down if dw_down else None, self.grad_accum, self.fp8_args, self.ws_bwd)

    def reset_grads(self):
        if self.grad_accum:
            for k, v in self.grad_init.items():
                self.t[k].copy_(v)

    def step(self):
        if self.fp8:
            self.quantize()
        self.forward()
        self.backward()

    def grads(self) -> dict:
        g = {"dx": self.dx, "dw_down": self.dw_down}
        if self.gated:
            g.update(dw_gate=self.dw_gate, dw_up=self.dw_up)
        else:
            g.update(dw1=self.dw_gate, dw2=self.dw_down)
            del g["dw_down"]
        return g


def runner_for(w, tensors, device="cuda", **kw) -> MlpRunner:
    """A runner for a workload description with fields act, dtype, M, d_in, hidden, d_out,
    gate_mult, down_mult, recompute, grad_accum, fp8_fwd (and optionally fp8_bwd, save_act)."""
    return MlpRunner(act=w.act, dtype=w.dtype, M=w.M, d_in=w.d_in, hidden=w.hidden, d_out=w.d_out,
                     gate_mult=w.gate_mult, down_mult=w.down_mult, recompute=w.recompute,
                     grad_accum=w.grad_accum, fp8_fwd=w.fp8_fwd, fp8_bwd=getattr(w, "fp8_bwd", False),
                     save_act=getattr(w, "save_act", False), tensors=tensors, device=device, **kw)
