"""Embedding row gather of the vocab-parallel embedding (oracle side; test
infrastructure only).

"Mini-SGLang 完整剖析" sections 4.9.2-4.9.3: the first op of forward_batch is
VocabParallelEmbedding's indexing(weights, ids, vocab_range), a gather of one
weight row per token id done by the index kernel as a plain row copy. The
pages do not spell out vocab_range; this follows the plainest reading of a
vocabulary-parallel table: a shard holds the rows of ids in [start, end)
(row id - start of its weight) and writes an all-zero row for any other id,
so adding the shards' outputs gives the full table's gather.
"""

import numpy as np


def embedding_gather(weight: np.ndarray, ids, vocab_start: int, vocab_end: int) -> np.ndarray:
    """weight [rows, hidden] (any element type, bit patterns kept), ids [n]
    -> out [n, hidden]: weight[id - vocab_start] for ids in range, zeros otherwise."""
    ids = np.asarray(ids).astype(np.int64)
    out = np.zeros((ids.shape[0],) + weight.shape[1:], dtype=weight.dtype)
    mask = (ids >= vocab_start) & (ids < vocab_end)
    out[mask] = weight[ids[mask] - vocab_start]
    return out
