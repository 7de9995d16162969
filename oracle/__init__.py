"""CPU float64 oracle for the fused transformer MLP (test infrastructure only).

This package is the reference the GPU path is checked against. It is plain, slow and written to be
read against the pages it follows:

* quack ``mlp.py`` (``MLPRecomputeFunc``, ``mlp_func`` and the ``MLP`` module's PyTorch
  fallback): what the forward and backward of ``act(x W1^T) W2^T`` compute, and which
  intermediate each backward step consumes and produces;
* flash-swiglu-mlp 0.4.2 README (PyPI description: the computed function, the "Falcon H1 style
  models" section and the "design points" section): the SwiGLU MLP with gate/down multipliers;
* modded-nanogpt ``gpt.py`` (the ``ReLUSqrdMLP`` comment, ``GPT._mlp``, the FP8 MLP constants,
  ``_refresh_delayed_scale`` and ``_quantize_mlp_weights_and_scales``): the ReLU^2 MLP, its
  e4m3 forward and its backward with e5m2 gradients.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import this
package. The product path (``gated_mlp_gemms_amd``) never imports, links or calls it, and this
package never imports the product path: the two share no code.

Every function states the passage it follows. Matrix products use ``numpy.matmul`` in float64 as
a library primitive; nothing else is blocked, fused or reordered.
"""
from .mlp import (  # noqa: F401
    sigmoid, silu, dsilu, relu_sq, drelu_sq, relu, drelu, gelu_tanh, dgelu_tanh, dsigmoid,
    GATED_FNS, PLAIN_FNS,
    gated_forward, gated_backward, gated_sampled,
    act_forward, act_backward, act_sampled,
    relu_sq_forward, relu_sq_backward, relu_sq_sampled,
    accumulate,
)
from .e4m3 import (  # noqa: F401
    E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_grid,
)
from .e5m2 import (  # noqa: F401
    E5M2_MAX, e5m2_decode, e5m2_encode, e5m2_grid,
)
from .fp8 import (  # noqa: F401
    per_tensor_scale, quantize_per_tensor, dequantize, next_delayed_scale, weight_quantize_calls,
    relu_sq_fp8_forward, relu_sq_fp8_backward, quantize_e5m2, relu_sq_fp8_backward_e5m2,
    relu_sq_fp8_backward_e5m2_sampled,
)
