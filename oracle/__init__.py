"""Plain, slow, obviously-correct CPU oracle for the paged-KV hot path.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``paged_kv_attention_scatter_amd``) never imports, links or executes anything
here, and nothing here imports the product path: the two share no code. The
only shared module is the seeded input generator (``workloads``), which draws
random numbers and holds none of the method's arithmetic.

Everything is NumPy in float64. bf16 inputs arrive as their uint16 bit
patterns and are widened exactly (bf16 -> fp32 -> fp64 is exact).

Sources (the pages are cited by title and section):

* "Engine 与采样器" (mini-sglang handbook, stage 1) -- sections 显存规划
  (page-count formula), 采样器 (Sampler.prepare / sample / sample_torch) and
  测试 (the sampler test's closed forms).
* "核心数据结构：Req、Batch、Context" (mini-sglang handbook) -- sections
  SamplingParams (is_greedy), Req (length fields), Context (the page table is
  always token-granular).
* "第 0 步：一个能跑的最小推理引擎" (mini-sglang handbook, step 0) -- the
  dense reference ``attention`` function (GQA by repeat_interleave, scale
  1/sqrt(D), causal mask on absolute positions); its ``rmsnorm`` and ``rope``
  operators and the per-head q/k norm before the rotation.
* "Mini-SGLang 完整剖析" -- sections 4.4.3 (KV pool layout, store_kv scatter),
  4.6.4/4.6.5 (page_size > 1 conversion, cu_seqlens), 4.6.7 (q/k norm and
  RoPE in place, then store_kv runs before the attention kernel), 4.8.4-4.8.6
  (greedy rule, sparse argument construction), 4.9.2-4.9.3 (the embedding
  gather), 4.9.4 (store kernel shape contract), 5.2 (worked page counts).
* "Mini-SGLang 源码解析（四）：GPU 计算引擎系统" -- sections 14.3/14.4
  (greedy fast path, top-k renormalisation example).

Every function below is pinned by a ``-m "not gpu"`` test against values the
pages print, closed forms, a textbook library routine on tiny inputs, or
invariants; see ``tests/test_oracle_*.py``.
"""

from .numerics import widen, bf16_bits_to_f64
from .req import Req
from .pages import bytes_per_page, num_pages
from .sampling_params import SamplingParams, is_greedy, prepare
from .store_kv import store_kv
from .attention import gather_kv, attention_request, attention_decode, attention_extend
from .sampler import sample, sample_row, admissible, admissible_row, DELTA
from .qk_norm_rope import rmsnorm, rope, rope_angles, rope_inv_freq, qk_norm_rope
from .embedding import embedding_gather

__all__ = [
    "widen", "bf16_bits_to_f64", "Req", "bytes_per_page", "num_pages",
    "SamplingParams", "is_greedy", "prepare", "store_kv", "gather_kv",
    "attention_request", "attention_decode", "attention_extend", "sample",
    "sample_row", "admissible", "admissible_row", "DELTA", "rmsnorm", "rope", "rope_angles", "rope_inv_freq", "qk_norm_rope",
    "embedding_gather",
]
