"""Device buffers for one MLP problem and the calls of one training step through the C ABI.

A ``MlpRunner`` holds the inputs, the outputs, the saved pre-activation and the workspaces of a
problem in HBM, so a caller (bench, tests, smoke) can run ``forward()`` / ``backward()`` /
``forward_infer()`` repeatedly without allocating. It only marshals: every step runs in the
library's kernels.
"""
from __future__ import annotations

import torch

from . import (GATED_ACTS, make_desc, make_fp8, mlp_bwd, mlp_fp8_next_scale, mlp_fwd, mlp_fwd_infer,
               mlp_quantize_e4m3, workspace_bytes)

E4M3_MAX = 448.0
POST_HEADROOM = 1.03   # delayed post scale = amax * 1.03 / 448, floor 1e-6
POST_FLOOR = 1e-6


class MlpRunner:
    def __init__(self, *, act, dtype, M, d_in, hidden, d_out, gate_mult=1.0, down_mult=1.0,
                 gate_mode="outside", recompute=False, grad_accum=False, fp8_fwd=False,
                 tensors: dict, device="cuda", dpreact_in_place=False):
        self.gated = act in GATED_ACTS
        self.grad_accum = grad_accum
        self.fp8 = fp8_fwd
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}.get(dtype, dtype)
        self.desc = make_desc(M, d_in, hidden, d_out, act, tdt, gate_mult, down_mult, gate_mode,
                              recompute, fp8_fwd)
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
        self.saved = None if recompute else torch.empty(M, P, dtype=tdt, device=dev)
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
            # one fp32 slot each: s_x, s_w1, s_w2, s_post, post_amax
            self.scales = torch.zeros(5, dtype=torch.float32, device=dev)
            self.scales[3] = 1.0              # bootstrap post scale
            self.ws_q = torch.empty(256, dtype=torch.uint8, device=dev)
            s = self.scales
            self.fp8_args = make_fp8(self.x_q, self.w1_q, self.w2_q, s[0:1].data_ptr(), s[1:2].data_ptr(),
                                     s[2:3].data_ptr(), s[3:4].data_ptr(), s[4:5].data_ptr())

    # ---- steps
    def quantize(self):
        """Per-tensor e4m3 of x, W1, W2 (exact scales)."""
        s = self.scales
        mlp_quantize_e4m3(self.x, self.x_q, s[0:1], self.ws_q)
        mlp_quantize_e4m3(self.w_gate, self.w1_q, s[1:2], self.ws_q)
        mlp_quantize_e4m3(self.w_down, self.w2_q, s[2:3], self.ws_q)

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
                self.dpreact if dpreact else None, self.dx if dx else None,
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
    gate_mult, down_mult, recompute, grad_accum, fp8_fwd."""
    return MlpRunner(act=w.act, dtype=w.dtype, M=w.M, d_in=w.d_in, hidden=w.hidden, d_out=w.d_out,
                     gate_mult=w.gate_mult, down_mult=w.down_mult, recompute=w.recompute,
                     grad_accum=w.grad_accum, fp8_fwd=w.fp8_fwd, tensors=tensors, device=device, **kw)
