"""Per-request sampling parameters and the batch argument builder
(oracle side; test infrastructure only).

* is_greedy follows "核心数据结构：Req、Batch、Context", section SamplingParams:
  a request is greedy when (temperature <= 0 or top_k == 1) and top_p == 1.0.
  top_p < 1 is never greedy, even at temperature 0.
* prepare follows "Engine 与采样器", section 采样器 (Sampler.prepare), restated
  in "Mini-SGLang 完整剖析" section 4.8.5: an all-greedy batch gets no
  temperature array at all (argmax fast path). Otherwise every row gets
  T = max(0 if greedy else T, 1e-6); top_k < 1 becomes the vocabulary size;
  top_p is clamped into [1e-6, 1]. The top_k (top_p) array exists only if some
  row actually restricts it.
"""

from dataclasses import dataclass

import numpy as np

MIN_T = 1e-6
MIN_P = 1e-6


@dataclass
class SamplingParams:
    temperature: float = 0.0
    top_k: int = -1
    top_p: float = 1.0


def is_greedy(p: SamplingParams) -> bool:
    return (p.temperature <= 0.0 or p.top_k == 1) and p.top_p == 1.0


def prepare(params, vocab_size: int):
    """-> (temperatures | None, top_k | None, top_p | None) as float32/int32
    numpy arrays, exactly what the device receives."""
    if all(is_greedy(p) for p in params):
        return None, None, None
    ts = [max(0.0 if is_greedy(p) else p.temperature, MIN_T) for p in params]
    ks = [p.top_k if p.top_k >= 1 else vocab_size for p in params]
    ps = [min(max(p.top_p, MIN_P), 1.0) for p in params]
    top_k = np.asarray(ks, dtype=np.int32) if any(k != vocab_size for k in ks) else None
    top_p = np.asarray(ps, dtype=np.float32) if any(q < 1.0 for q in ps) else None
    return np.asarray(ts, dtype=np.float32), top_k, top_p
