"""Seeded synthetic inputs for the paged-KV hot path.

This module is the ONLY code shared by the oracle side (tests) and the GPU
side (tests, bench). It draws random numbers and lays them out; it holds none
of the method's arithmetic (no attention, no softmax, no sampling, no page
count). Shapes follow Qwen3-0.6B's attention (16 query heads, 8 KV heads,
head_dim 128, 28 layers, vocabulary 151936), as printed in
"第 0 步：一个能跑的最小推理引擎".

Recipe (identical for every case):

* ``root = SeedSequence(seed)``; ``root.spawn(7)`` gives, in this order, the
  streams for lengths, pages, q, K/V, logits, params and uniforms.
* K/V of request r come from ``default_rng(kv_stream.spawn(bs)[r])`` as
  [device_len, HKV, D] fp32 N(0, 1) for K then V, so one request can be
  regenerated alone.
* bf16 values are fp32 draws rounded to nearest-even (a dtype conversion).
* page_size 1: a permutation of the pool's pages is consumed request by
  request; page_size 16: a permutation of pages, ceil(S/16) pages per
  request, token t of a request sits at slot page*16 + t % 16. The last page
  of the pool (index num_pages) is the dummy page and is never used.
* Integer ranges are inclusive.
"""

from .configs import (HQ, HKV, HEAD_DIM, VOCAB, LAYERS, CaseConfig, CONFIGS, config,
                      f32_to_bf16_bits, draw_lengths, draw_page_table, draw_case, draw_q,
                      draw_request_kv, draw_logits, draw_sampling_params, draw_uniforms,
                      default_num_pages, table_width)

__all__ = [
    "HQ", "HKV", "HEAD_DIM", "VOCAB", "LAYERS", "CaseConfig", "CONFIGS", "config",
    "f32_to_bf16_bits", "draw_lengths", "draw_page_table", "draw_case", "draw_q", "draw_request_kv",
    "draw_logits", "draw_sampling_params", "draw_uniforms", "default_num_pages", "table_width",
]
