"""Seeded synthetic inputs for the MLP forward/backward, shared by the tests, the bench and smoke().

This module holds the input recipe and nothing of the MLP's arithmetic: it draws random numbers
and rounds them to a storage dtype. Both the GPU path and the CPU oracle consume the bytes it
returns, so neither depends on the other.

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream per workload, draws in float64,
rounded to float32 by numpy and then to the storage dtype by torch):

* draw order: x, W_gate (or W1), W_up (gated only), W_down (or W2), dout, then the pre-existing
  fp32 weight-gradient buffers when the workload accumulates into them;
* x, dout ~ N(0, 1): the inputs of a transformer MLP are RMS-normalised rows (modded-nanogpt
  ``gpt.py``, ``GPT.forward``, where the MLP input is ``norm(x)``), for which N(0, 1) is the
  stand-in;
* weights ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)), the default ``nn.Linear(bias=False)`` init named
  by flash-swiglu-mlp's README (module usage section); fan_in is d_in for the up/gate
  projections and the intermediate size for the down projection;
* accumulate-into buffers ~ N(0, 0.01^2) in float32.

Shapes follow the pages' examples: LLaMA 4096/11008 on x [2, 1024, 4096] and Falcon-H1
2048/4864 with multipliers 1.125 / 2.0 (flash-swiglu-mlp README, "Falcon H1" section), and the
768-wide GPT MLP with 4 * 768 hidden (modded-nanogpt ``gpt.py``, MLP_HIDDEN_DIM comment).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    act: str            # gated: "swiglu" | "geglu" | "reglu" | "glu"; else "relu_sq" | "relu" | "gelu_tanh"
    dtype: str          # storage dtype of x / weights / outputs: "f32" | "bf16" | "f16"
    batch: tuple        # leading dims of x; M is their product
    d_in: int
    hidden: int
    d_out: int
    gate_mult: float = 1.0
    down_mult: float = 1.0
    recompute: bool = False
    grad_accum: bool = False
    fp8_fwd: bool = False
    seed: int = 0
    fp8_bwd: bool = False   # backward products in fp8 too (e5m2 gradients); needs fp8_fwd
    save_act: bool = False  # the forward keeps the activation next to the pre-activation

    @property
    def M(self) -> int:
        return int(np.prod(self.batch))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def gated(self) -> bool:
        return self.act in ("swiglu", "geglu", "reglu", "glu")

    def model_flops(self) -> float:
        """2*M*N*K summed over the GEMMs of one forward+backward (gated 18*M*d*H, ReLU^2 12*M*d*H,
        for d_in == d_out)."""
        M, d, H, do = self.M, self.d_in, self.hidden, self.d_out
        if self.gated:
            fwd = 2 * M * d * 2 * H + 2 * M * H * do
            bwd = 2 * M * do * H + 2 * do * M * H + 2 * M * 2 * H * d + 2 * 2 * H * M * d
        else:
            fwd = 2 * M * d * H + 2 * M * H * do
            bwd = 2 * M * do * H + 2 * do * M * H + 2 * M * H * d + 2 * H * M * d
        return float(fwd + bwd)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("swiglu_f32_m64_d128_h384", "swiglu", "f32", (64,), 128, 384, 128),
        Workload("llama_swiglu_bf16_m2048_d4096_h11008", "swiglu", "bf16", (2, 1024), 4096, 11008, 4096),
        Workload("falcon_h1_swiglu_bf16_m8192_d2048_h4864", "swiglu", "bf16", (4, 2048), 2048, 4864, 2048,
                 gate_mult=1.125, down_mult=2.0, recompute=True, grad_accum=True),
        Workload("gpt_relu2_bf16_m49152_d768_h3072", "relu_sq", "bf16", (48, 1024), 768, 3072, 768),
        Workload("gpt_relu2_fp8fwd_m49152_d768_h3072", "relu_sq", "bf16", (48, 1024), 768, 3072, 768,
                 fp8_fwd=True),
        # the same with the backward in fp8 too (e5m2 gradients)
        Workload("gpt_relu2_fp8_m49152_d768_h3072", "relu_sq", "bf16", (48, 1024), 768, 3072, 768,
                 fp8_fwd=True, fp8_bwd=True),
        # one GPU's share of the LLaMA step on 8 GPUs: tensor parallel (hidden units split 8 ways,
        # a gate/up pair kept together) and data parallel (tokens split 8 ways)
        Workload("llama_swiglu_bf16_tp8_m2048_d4096_h1376", "swiglu", "bf16", (2, 1024), 4096, 1376, 4096),
        Workload("llama_swiglu_bf16_dp8_m256_d4096_h11008", "swiglu", "bf16", (1, 256), 4096, 11008, 4096),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "llama_swiglu_bf16_m2048_d4096_h11008"

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _to_storage(a: np.ndarray, dtype: str, shape) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a.astype(np.float32))).reshape(shape)
    return t.to(_TORCH_DTYPE[dtype]).contiguous()


def make_inputs(w: Workload) -> dict:
    """All tensors of one forward+backward step of workload ``w``, as CPU torch tensors in their
    storage dtype. Keys: x, w_gate, w_up (gated) or w1, w_down or w2, dout, and dw_* when the
    workload accumulates into existing gradient buffers."""
    rng = np.random.default_rng(w.seed)
    M, d, H, do = w.M, w.d_in, w.hidden, w.d_out
    out = {}
    out["x"] = _to_storage(rng.standard_normal(M * d), w.dtype, (M, d))
    b1 = 1.0 / np.sqrt(d)
    b2 = 1.0 / np.sqrt(H)
    if w.gated:
        out["w_gate"] = _to_storage(rng.uniform(-b1, b1, H * d), w.dtype, (H, d))
        out["w_up"] = _to_storage(rng.uniform(-b1, b1, H * d), w.dtype, (H, d))
        out["w_down"] = _to_storage(rng.uniform(-b2, b2, do * H), w.dtype, (do, H))
    else:
        out["w1"] = _to_storage(rng.uniform(-b1, b1, H * d), w.dtype, (H, d))
        out["w2"] = _to_storage(rng.uniform(-b2, b2, do * H), w.dtype, (do, H))
    out["dout"] = _to_storage(rng.standard_normal(M * do), w.dtype, (M, do))
    if w.grad_accum:
        names = [("dw_gate", (H, d)), ("dw_up", (H, d)), ("dw_down", (do, H))] if w.gated \
            else [("dw1", (H, d)), ("dw2", (do, H))]
        for k, shp in names:
            n = int(np.prod(shp))
            out[k] = _to_storage(0.01 * rng.standard_normal(n), "f32", shp)
    return out


def digest(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's bytes (logged next to results so runs can be matched)."""
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
