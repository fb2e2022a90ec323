"""CPU oracle for the layer's bandwidth-bound element-wise steps: residual add + RMS
normalisation, and the SiLU-gated product of the MLP.  Plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library and imports nothing from it.

Sources (cited by title and section):
  [guide]  "tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §Llama 3.2 1B架构拆解: every
           sub-layer is wrapped in RMS normalisation and a residual connection; the MLP
           applies SiLU to the gate projection and multiplies it element-wise with the up
           projection.
  [实战]   "Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎", §算子融合: fusing the residual
           add into the normalisation (and the activation into the product) saves a round
           trip of the activations through memory.

What is computed (per token row of H values):
  * h = x + r;  out = h / sqrt(mean(h^2) + eps) * gamma   (residual add + RMSNorm; the sum
    h is also returned, as the next sub-layer's residual);
  * out = silu(g) * u with silu(z) = z / (1 + e^-z)          (the gated MLP activation).

Readings taken where the pages are silent:
  * the residual sum is rounded to bf16 before it is normalised (it is stored as the next
    residual in bf16, and the normalisation reads that stored value);
  * mean(h^2), the scaling and the products run in full precision and each output is
    rounded once to bf16 (nearest even); eps is a caller-given constant (1e-5 for the
    Llama 3 family);
  * without a residual input, h = x.

Parity pins (tests/test_oracle_norm.py): a constant row normalises to gamma * sign; the
result does not change when the row is scaled (eps = 0); the output row has RMS 1 before
gamma (eps = 0); silu against scipy's logistic function; silu(0) = 0 and its limits; the
fused form equals the two steps done apart.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import bf16_to_f64
from .rope import f64_to_bf16


def residual_rmsnorm(x: np.ndarray, r, gamma: np.ndarray, eps: float):
    """bf16 bits x, r (or None) [T, H], gamma [H] -> (out bits [T, H], h bits [T, H])."""
    xf = bf16_to_f64(x)
    h_bits = f64_to_bf16(xf + bf16_to_f64(r)) if r is not None else np.asarray(x, np.uint16)
    h = bf16_to_f64(h_bits)
    inv = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return f64_to_bf16(h * inv * bf16_to_f64(gamma)), h_bits


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """bf16 bits g, u [T, I] -> bf16 bits of silu(g) * u."""
    gf = bf16_to_f64(g)
    return f64_to_bf16(gf / (1.0 + np.exp(-gf)) * bf16_to_f64(u))
