"""Per-head RMSNorm of q and k, rotary position embedding, then the KV store
(oracle side; test infrastructure only).

Follows "第 0 步：一个能跑的最小推理引擎" (mini-sglang handbook, step 0): its
``rmsnorm`` and ``rope`` operators and its layer function, where q and k each
go through their own RMSNorm over the head dimension (Qwen3's q_norm /
k_norm) and are then rotated at the tokens' absolute positions, while v is
left as it is; and "Mini-SGLang 完整剖析" section 4.6.7 (the attention layer
normalises q and k in place, rotates them, and the backend's first act is
store_kv of k and v through out_loc).

* rmsnorm(x, w) = w * x / sqrt(mean(x^2) + eps), over the head dimension.
* RoPE pairs dimension j with j + D/2 (the first and the second half of the
  head, the Hugging Face / Qwen convention the step-0 page names); pair j at
  position p turns by the angle p * inv_freq[j], inv_freq[j] = 1 / theta^(2j/D):
  (x_j, x_{j+D/2}) -> (x_j cos - x_{j+D/2} sin, x_j sin + x_{j+D/2} cos).

The step-0 page computes inv_freq and the angles in fp32 (``.float()``); the
oracle does the same for these two quantities -- theta^(2j/D) rounded to fp32,
an fp32 division, the angle as one fp32 product -- and everything else in fp64.
"""

import numpy as np


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """fp32 [head_dim / 2]: 1 / theta^(2j / head_dim), the power rounded to
    fp32 and the reciprocal taken in fp32 (as the page's fp32 tensors do)."""
    e = np.arange(0, head_dim, 2, dtype=np.float64) / head_dim
    p = np.power(np.float64(theta), e).astype(np.float32)
    return (np.float32(1.0) / p).astype(np.float32)


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """fp32 [n, head_dim / 2]: position (as fp32) times inv_freq, one fp32 product."""
    pos = np.asarray(positions).astype(np.float32)
    return (pos[:, None] * rope_inv_freq(head_dim, theta)[None, :]).astype(np.float32)


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """fp64: x [..., D], w [D] -> w * x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(w, dtype=np.float64) * (x / np.sqrt(ms + np.float64(eps)))


def rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """fp64: x [n, heads, D] rotated at positions [n] (halves paired)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = rope_angles(positions, D, theta).astype(np.float64)[:, None, :]  # [n, 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def qk_norm_rope(q, k, positions, q_norm_w, k_norm_w, eps: float, theta: float):
    """fp64 (q_out [n, HQ, D], k_out [n, HKV, D]): each head normalised by its
    tensor's norm weight, then rotated at its token's position."""
    return (rope(rmsnorm(q, q_norm_w, eps), positions, theta),
            rope(rmsnorm(k, k_norm_w, eps), positions, theta))
