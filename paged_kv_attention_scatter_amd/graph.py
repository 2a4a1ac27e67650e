"""Decode steps replayed from HIP graphs over a set of captured batch sizes.

"Mini-SGLang 源码解析（四）：GPU 计算引擎系统", sections 10.4-10.10, and
"Engine 与采样器", section 初始化的顺序, describe the engine's graph runner:
a graph has a fixed batch size, so the engine captures a list of sizes --
1, 2, 4, then every multiple of 8 up to the largest batch -- from the largest
to the smallest, all into one shared memory pool, and at run time pads a
batch to the next captured size with the dummy request, whose page-table row
holds only the dummy page's slot, so everything the padding rows write lands
there.

DecodeGraphRunner does that for one decode step of this library: store_kv of
the new K/V rows and decode attention over the pool (one fused call), then
the sampler. The
graphs replay the library's kernels on static buffers; run() copies a batch
into them (padding rows: the dummy request, one key long, greedy), replays
the graph of the next captured size, and returns views of the outputs. Every
kernel is the library's; this module only stages arguments and replays.
"""

from . import api


def capture_sizes(max_bs: int) -> list:
    """1, 2, 4, then 8, 16, ... up to max_bs (max_bs itself included)."""
    sizes = [b for b in (1, 2, 4) if b <= max_bs] + list(range(8, max_bs + 1, 8))
    if max_bs not in sizes:
        sizes.append(max_bs)
    return sorted(set(sizes))


class DecodeGraphRunner:
    """Captured decode steps over the pool (k_pool, v_pool) and page_table.

    page_table: int32 [rows, width] on the device; its last row is the dummy
    request's and is filled here with dummy_slot (the first slot of the
    dummy page). Requests pick their rows through table_idx at run time.
    max_context bounds every request's device_len (it fixes each graph's
    decode plan bound: bs * max_context keys). T / P / K given to run() are
    the prepared per-row sampling arrays (top_k optional, as in pkv_sample).
    """

    def __init__(self, k_pool, v_pool, page_table, dummy_slot: int, *, max_bs: int, vocab: int,
                 num_q_heads: int, max_context: int, use_top_k: bool = False, logits_dtype=None,
                 page_size: int = 1, sizes=None):
        torch = api._torch()
        dev = k_pool.device
        self.torch = torch
        self.k_pool, self.v_pool, self.page_table = k_pool, v_pool, page_table
        self.page_size = page_size
        self.max_bs, self.vocab, self.max_context = max_bs, vocab, max_context
        self.sizes = sorted(capture_sizes(max_bs) if sizes is None else sizes)
        self.dummy_row = page_table.shape[0] - 1
        self.dummy_slot = dummy_slot
        page_table[self.dummy_row].fill_(dummy_slot)
        hkv, hq, D = k_pool.shape[1], num_q_heads, api.HEAD_DIM
        dt = k_pool.dtype
        ldt = dt if logits_dtype is None else logits_dtype
        i32, f32 = torch.int32, torch.float32
        B = max_bs
        # static inputs and outputs (a batch of n uses rows [0, n))
        self.q = torch.zeros((B, hq, D), dtype=dt, device=dev)
        self.k = torch.zeros((B, hkv, D), dtype=dt, device=dev)
        self.v = torch.zeros((B, hkv, D), dtype=dt, device=dev)
        self.out_loc = torch.full((B,), dummy_slot, dtype=i32, device=dev)
        self.table_idx = torch.full((B,), self.dummy_row, dtype=i32, device=dev)
        self.cached_len = torch.zeros(B, dtype=i32, device=dev)
        self.device_len = torch.ones(B, dtype=i32, device=dev)
        self.logits = torch.zeros((B, vocab), dtype=ldt, device=dev)
        self.T = torch.zeros(B, dtype=f32, device=dev)
        self.P = torch.ones(B, dtype=f32, device=dev)
        self.K = torch.full((B,), vocab, dtype=i32, device=dev) if use_top_k else None
        self.u = torch.zeros(B, dtype=f32, device=dev)
        self.o = torch.zeros((B, hq, D), dtype=dt, device=dev)
        self.tokens = torch.zeros(B, dtype=i32, device=dev)
        self.ws_d = torch.empty(api.decode_workspace_size(B, hq, B * max_context), dtype=torch.uint8, device=dev)
        self.ws_s = api.sample_workspace(B, vocab, dev)
        self.graphs = {}
        # warm up once on a side stream (nothing may be first-touched under
        # capture), then capture from the largest size down into one pool
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self._step(self.sizes[-1])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        pool = torch.cuda.graph_pool_handle()
        for n in reversed(self.sizes):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, pool=pool):
                self._step(n)
            self.graphs[n] = g
        torch.cuda.synchronize()

    def _step(self, n):
        # store_kv and decode attention in one call (the attention kernel
        # writes each request's new row and reads it as its last key)
        api.paged_attention_decode_store(self.q[:n], self.k_pool, self.v_pool, self.page_table, self.cached_len[:n],
                                         self.device_len[:n], self.out_loc[:n], self.k[:n], self.v[:n],
                                         table_idx=self.table_idx[:n], max_total_kv=n * self.max_context,
                                         page_size=self.page_size, out=self.o[:n], workspace=self.ws_d)
        api.sample(self.logits[:n], self.T[:n], None if self.K is None else self.K[:n], self.P[:n], self.u[:n],
                   out=self.tokens[:n], workspace=self.ws_s)

    def size_for(self, bs: int) -> int:
        for n in self.sizes:
            if n >= bs:
                return n
        raise ValueError(f"batch of {bs} exceeds the largest captured size {self.sizes[-1]}")

    def run(self, q, k, v, out_loc, table_idx, cached_len, device_len, logits, T, P, u, K=None, replay=True):
        """One decode step of bs = len(device_len) requests (device tensors).
        Returns (o [bs, num_q_heads, 128], tokens [bs]) -- views of the
        runner's static outputs, valid until the next run(). replay=False
        launches the same padded step eagerly instead of replaying it."""
        bs = device_len.shape[0]
        n = self.size_for(bs)
        for dst, src in ((self.q, q), (self.k, k), (self.v, v), (self.out_loc, out_loc),
                         (self.table_idx, table_idx), (self.cached_len, cached_len),
                         (self.device_len, device_len), (self.logits, logits), (self.T, T), (self.P, P),
                         (self.u, u)):
            dst[:bs].copy_(src)
        if self.K is not None:
            if K is None:
                self.K[:bs].fill_(self.vocab)
            else:
                self.K[:bs].copy_(K)
        if n > bs:  # padding rows: the dummy request, one key on the dummy slot, greedy
            self.out_loc[bs:n].fill_(self.dummy_slot)
            self.table_idx[bs:n].fill_(self.dummy_row)
            self.cached_len[bs:n].fill_(0)
            self.device_len[bs:n].fill_(1)
            self.T[bs:n].fill_(0.0)
            self.P[bs:n].fill_(1.0)
            if self.K is not None:
                self.K[bs:n].fill_(self.vocab)
        if replay:
            self.graphs[n].replay()
        else:
            self._step(n)
        return self.o[:bs], self.tokens[:bs]
