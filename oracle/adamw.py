"""Fused mixed-precision AdamW update of one shard.

[ZF] "Static Memory Allocation": AdamW keeps fp32 master weights, an fp32
first moment m_t and an fp32 second moment v_t; parameters are 16-bit.
[ZF] "Execution Flow for ZeRO-1", step 3: the rank updates its own master
weights and optimizer states from its averaged gradient shard; step 4 gathers
the updated 16-bit parameter shards.
[ZF] "ZeRO-Offload Mechanics": the update is O(1) work per parameter.

The update itself is not written on the pages. Reading taken: AdamW with
decoupled weight decay (Loshchilov & Hutter) and bias correction, in PyTorch's
form (the only code on the page is PyTorch): with t >= 1 counting steps taken,

  g      = fp32(grad) * clip
  m      = beta1 * m + (1 - beta1) * g
  v      = beta2 * v + (1 - beta2) * g * g
  p      = p * (1 - lr * wd)
  denom  = sqrt(v) / sqrt(1 - beta2^t) + eps
  p      = p - (lr / (1 - beta1^t)) * (m / denom)
  param  = bf16(p)

Every per-element operation is one IEEE fp32 operation (no fused multiply-
add), in the order written. The scalars beta1, 1-beta1, beta2, 1-beta2, eps,
lr/(1-beta1^t), sqrt(1-beta2^t) and 1-lr*wd are computed in float64 and rounded
once each to fp32. Decay applies to every element, padding included.
A non-finite clip coefficient skips the update: state and param untouched.
"""
import math
from dataclasses import dataclass

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16

f32 = np.float32


@dataclass(frozen=True)
class AdamWConstants:
    beta1: np.float32
    one_minus_beta1: np.float32
    beta2: np.float32
    one_minus_beta2: np.float32
    eps: np.float32
    step_size: np.float32
    sqrt_bc2: np.float32
    decay: np.float32


def adamw_constants(step: int, lr: float, beta1: float, beta2: float, eps: float,
                    weight_decay: float) -> AdamWConstants:
    if step < 1:
        raise ValueError("step counts from 1")
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    return AdamWConstants(
        beta1=f32(beta1), one_minus_beta1=f32(1.0 - beta1),
        beta2=f32(beta2), one_minus_beta2=f32(1.0 - beta2),
        eps=f32(eps), step_size=f32(lr / bc1), sqrt_bc2=f32(math.sqrt(bc2)),
        decay=f32(1.0 - lr * weight_decay))


def adamw_step(master: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray,
               grad_bits: np.ndarray, step: int, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float, clip: float = 1.0):
    """Returns (master, exp_avg, exp_avg_sq, param_bits) as new arrays.

    param_bits is None when the update is skipped (non-finite clip coefficient).
    """
    c = adamw_constants(step, lr, beta1, beta2, eps, weight_decay)
    clip32 = f32(clip)
    if not np.isfinite(clip32):
        return master.copy(), exp_avg.copy(), exp_avg_sq.copy(), None
    p = np.asarray(master, dtype=np.float32)
    m = np.asarray(exp_avg, dtype=np.float32)
    v = np.asarray(exp_avg_sq, dtype=np.float32)
    g = bf16_to_f32(grad_bits) * clip32
    m = c.beta1 * m + c.one_minus_beta1 * g
    v = c.beta2 * v + c.one_minus_beta2 * (g * g)
    p = p * c.decay
    denom = np.sqrt(v) / c.sqrt_bc2 + c.eps
    p = p - c.step_size * (m / denom)
    return p, m, v, f32_to_bf16(p)

