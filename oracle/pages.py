"""KV-pool page count (oracle side; test infrastructure only).

Follows "Engine 与采样器", section 显存规划 (Engine._determine_num_pages), and
the worked budget in "Mini-SGLang 完整剖析" section 5.2:

* bytes per page = 2 (K and V) x head_dim x (KV heads on this rank)
  x page_size x dtype bytes x layers;
* available = int(memory_ratio x free memory before loading the model)
  - model memory;
* num_pages = available // bytes per page, and fewer than two pages is an
  error ("Not enough memory for KV cache").

Under tensor parallelism the KV heads are split evenly across ranks, or
replicated when there are fewer heads than ranks (div_even with replication).
"""


def _kv_heads_per_rank(kv_heads: int, tp_size: int) -> int:
    if kv_heads >= tp_size:
        if kv_heads % tp_size:
            raise ValueError("kv_heads must divide evenly across tp ranks")
        return kv_heads // tp_size
    if tp_size % kv_heads:
        raise ValueError("tp_size must be a multiple of kv_heads to replicate")
    return 1


def bytes_per_page(head_dim: int, kv_heads: int, page_size: int, itemsize: int,
                   num_layers: int, tp_size: int = 1) -> int:
    return 2 * head_dim * _kv_heads_per_rank(kv_heads, tp_size) * page_size * itemsize * num_layers


def num_pages(head_dim: int, kv_heads: int, page_size: int, itemsize: int, num_layers: int,
              free_before: int, model_bytes: int, memory_ratio: float = 0.9,
              tp_size: int = 1) -> int:
    per_page = bytes_per_page(head_dim, kv_heads, page_size, itemsize, num_layers, tp_size)
    available = int(memory_ratio * free_before) - int(model_bytes)
    n = available // per_page
    if n <= 1:
        raise ValueError("Not enough memory for KV cache")
    return n
