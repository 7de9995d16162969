"""Fused transformer-MLP forward/backward for AMD MI355X (gfx950), behind the C ABI of
``include/mlp.h``.

The functions below carry the C entry points' names and only marshal arguments: torch tensors
become device pointers, the current HIP stream is passed along, and a non-OK status raises
``MlpError``. Every step of the MLP runs in the library's HIP kernels; there is no other path.
"""
from __future__ import annotations

import ctypes as C

import torch

from ._lib import (  # noqa: F401
    LIB_PATH, MLP_ACT_GEGLU, MLP_ACT_GELU_TANH, MLP_ACT_GLU, MLP_ACT_REGLU, MLP_ACT_RELU, MLP_ACT_RELU_SQ,
    MLP_ACT_SWIGLU, MLP_BF16, MLP_BWD_DW_DOWN_WITH_DACT, MLP_BWD_GROUPED, MLP_F16, MLP_F32, MLP_FP8_E4M3,
    MLP_FP8_E5M2, MLP_GATE_INSIDE, MLP_GATE_OUTSIDE,
    MLP_NOALLOC_SCRATCH_BYTES, MLP_PHASE_BWD, MLP_PHASE_FWD, MLP_PHASE_FWD_INFER, MlpDesc, MlpError, MlpFp8, check,
    lib,
)

_ACTS = {"swiglu": MLP_ACT_SWIGLU, "relu_sq": MLP_ACT_RELU_SQ, "geglu": MLP_ACT_GEGLU, "reglu": MLP_ACT_REGLU,
         "glu": MLP_ACT_GLU, "gelu_tanh": MLP_ACT_GELU_TANH, "relu": MLP_ACT_RELU}
GATED_ACTS = frozenset({"swiglu", "geglu", "reglu", "glu"})   # a = f(g) * u, weights w_gate and w_up
_DTYPES = {torch.float32: MLP_F32, torch.bfloat16: MLP_BF16, torch.float16: MLP_F16, "f32": MLP_F32,
           "bf16": MLP_BF16, "f16": MLP_F16}
_MODES = {"outside": MLP_GATE_OUTSIDE, "inside": MLP_GATE_INSIDE}
_PHASES = {"fwd": MLP_PHASE_FWD, "fwd_infer": MLP_PHASE_FWD_INFER, "bwd": MLP_PHASE_BWD}


def make_desc(M, d_in, hidden, d_out=None, act="swiglu", dtype=torch.bfloat16, gate_mult=1.0,
              down_mult=1.0, gate_mode="outside", recompute=False, fp8_fwd=False, fp8_bwd=False,
              save_act=False) -> MlpDesc:
    return MlpDesc(int(M), int(d_in), int(hidden), int(d_in if d_out is None else d_out), _ACTS[act],
                   _DTYPES[dtype], float(gate_mult), float(down_mult), _MODES[gate_mode], int(bool(recompute)),
                   int(bool(fp8_fwd)), int(bool(fp8_bwd)), int(bool(save_act)))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_fp8(x_q, w1_q, w2_q, s_x, s_w1, s_w2, s_post=None, post_amax=None, w1t_q=None, w2t_q=None,
             s_grad=None, s_dpre=None, dpre_amax=None) -> MlpFp8:
    return MlpFp8(*[_ptr(t) for t in (x_q, w1_q, w2_q, s_x, s_w1, s_w2, s_post, post_amax, w1t_q, w2t_q,
                                      s_grad, s_dpre, dpre_amax)])


def workspace_bytes(desc: MlpDesc, phase: str) -> int:
    n = lib().mlp_workspace_bytes(C.byref(desc), _PHASES[phase])
    if n == 0:
        raise MlpError(1, "mlp_workspace_bytes")
    return int(n)


def _workspace(desc, phase, workspace, device):
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    n = workspace_bytes(desc, phase)
    return torch.empty(n, dtype=torch.uint8, device=device), n


def mlp_fwd(desc, x, w_gate, w_up, w_down, out, saved_preact=None, fp8=None, workspace=None, stream=None):
    ws, nws = _workspace(desc, "fwd", workspace, out.device)
    st = lib().mlp_fwd(C.byref(desc), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
                       _ptr(saved_preact), C.byref(fp8) if fp8 is not None else None, _ptr(ws), nws,
                       _stream(stream))
    check(st, "mlp_fwd")
    return out


def mlp_fwd_infer(desc, x, w_gate, w_up, w_down, out, fp8=None, workspace=None, stream=None):
    ws, nws = _workspace(desc, "fwd_infer", workspace, out.device)
    st = lib().mlp_fwd_infer(C.byref(desc), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
                             C.byref(fp8) if fp8 is not None else None, _ptr(ws), nws, _stream(stream))
    check(st, "mlp_fwd_infer")
    return out


def mlp_fwd_infer_noalloc(desc, x, w_gate, w_up, w_down, out, fp8=None, stream=None):
    """``mlp_fwd_infer`` on the library's static per-GPU scratch: no workspace argument and no
    allocation (the problem's inference workspace must fit MLP_NOALLOC_SCRATCH_BYTES)."""
    st = lib().mlp_fwd_infer_noalloc(C.byref(desc), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
                                     C.byref(fp8) if fp8 is not None else None, _stream(stream))
    check(st, "mlp_fwd_infer_noalloc")
    return out


def mlp_bwd(desc, dout, x, w_gate, w_up, w_down, saved_preact=None, dpreact=None, dx=None, dw_gate=None,
            dw_up=None, dw_down=None, grad_accum=False, fp8=None, workspace=None, stream=None):
    ws, nws = _workspace(desc, "bwd", workspace, dout.device)
    st = lib().mlp_bwd(C.byref(desc), _ptr(dout), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                       _ptr(saved_preact), _ptr(dpreact), _ptr(dx), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down),
                       int(bool(grad_accum)), C.byref(fp8) if fp8 is not None else None, _ptr(ws), nws,
                       _stream(stream))
    check(st, "mlp_bwd")


def mlp_quantize_workspace_bytes() -> int:
    return int(lib().mlp_quantize_workspace_bytes())


def mlp_quantize_e4m3(src, dst, scale, workspace=None, stream=None):
    """Per-tensor e4m3 quantization of ``src`` (f32/bf16/f16) into ``dst`` (uint8 or float8_e4m3fn)
    and the fp32 device scalar ``scale``."""
    if workspace is None:
        workspace = torch.empty(mlp_quantize_workspace_bytes(), dtype=torch.uint8, device=src.device)
    st = lib().mlp_quantize_e4m3(_ptr(src), _DTYPES[src.dtype], src.numel(), _ptr(dst), _ptr(scale),
                                 _ptr(workspace), workspace.numel(), _stream(stream))
    check(st, "mlp_quantize_e4m3")


def mlp_quantize_fp8(src, fmt, scale, dst=None, dst_t=None, ld_t=None, relu_sq=False, stream=None):
    """fp8 codes of the bf16 matrix ``src`` [rows, cols] with the given scale (a device fp32
    scalar): row-major into ``dst`` and / or transposed into ``dst_t`` [cols, ld_t] (ld_t >= rows,
    a multiple of 16; default rows rounded up to 16; the padding columns are zero). fmt: "e4m3"
    or "e5m2"."""
    rows, cols = src.shape
    if ld_t is None:
        ld_t = (rows + 15) // 16 * 16
    f = {"e4m3": MLP_FP8_E4M3, "e5m2": MLP_FP8_E5M2}[fmt]
    st = lib().mlp_quantize_fp8(_ptr(src), _DTYPES[src.dtype], rows, cols, f, int(bool(relu_sq)), _ptr(scale),
                                _ptr(dst), _ptr(dst_t), int(ld_t), _stream(stream))
    check(st, "mlp_quantize_fp8")


def mlp_weight_amax_slots(rows: int, cols: int) -> int:
    return int(lib().mlp_weight_amax_slots(int(rows), int(cols)))


def mlp_quantize_weight_e4m3(w, exact, scale, tile_amax, dst=None, dst_t=None, ld_t=None, stream=None):
    """The fp8 weight-cache quantizer: e4m3 codes of the [rows, cols] weight ``w`` (bf16 / f32)
    row-major into ``dst`` and / or transposed into ``dst_t`` [cols, ld_t]; the scale (a device fp32
    scalar) is w's exact one when ``exact``, else the one the amax recorded by the previous call in
    ``tile_amax`` gives; this call's per-tile amax is recorded there."""
    rows, cols = w.shape
    if ld_t is None:
        ld_t = (rows + 15) // 16 * 16
    st = lib().mlp_quantize_weight_e4m3(_ptr(w), _DTYPES[w.dtype], rows, cols, int(bool(exact)), _ptr(scale),
                                        _ptr(tile_amax), _ptr(dst), _ptr(dst_t), int(ld_t), _stream(stream))
    check(st, "mlp_quantize_weight_e4m3")


def mlp_bwd_grouped(desc: MlpDesc) -> int:
    """mlp_bwd's schedule flags for this problem: MLP_BWD_GROUPED (dx and the weight gradients
    left after the d-activation GEMM run as one launch) | MLP_BWD_DW_DOWN_WITH_DACT (dW_down runs
    in the d-activation GEMM's launch; save_act only). 0: every product alone."""
    out = C.c_int(0)
    check(lib().mlp_bwd_grouped(C.byref(desc), C.byref(out)), "mlp_bwd_grouped")
    return int(out.value)


def mlp_fp8_next_scale(amax: float, prev_scale: float, gain: float, floor: float) -> float:
    return float(lib().mlp_fp8_next_scale(amax, prev_scale, gain, floor))
