"""A whole decode step (store_kv -> decode attention -> sampler) captured in a
HIP graph and replayed ("Mini-SGLang 源码解析（四）：GPU 计算引擎系统" sections 7
and 10: a captured graph has a fixed batch size, so a smaller batch is padded
with the dummy request, whose page-table row points at the dummy page; the
graph is captured after a warm-up run, with every buffer already allocated,
and replays on the same addresses).

The batch of 5 requests is padded to 8: each padding row is one key long, its
page-table row, out_loc and new K/V point at the dummy slot, and it samples
greedily. Every replay runs after eager work and a synchronisation, with new
inputs copied into the graph's static buffers (a new token per request, the
lengths one longer, new logits), and must equal the same padded step run
eagerly on a twin pool bit for bit (outputs, tokens, pool); the first step's
real rows are also checked against the oracle."""

import numpy as np
import pytest

import oracle
from oracle.attention import attention_request
from gpu_util import check_attention, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
pkv = pytest.importorskip("paged_kv_attention_scatter_amd")

HQ, HKV, D, V = 16, 8, 128, 151936


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.read_faults()


def test_decode_step_graph_replays_match_eager():
    dev = torch.device("cuda")
    rng = np.random.default_rng(2026)
    bs, bs_pad, steps = 5, 8, 4
    num_slots = 60000
    dummy = num_slots - 1
    S0 = rng.integers(300, 2000, bs).astype(np.int32)           # device_len of the first step (new token included)
    width = int(S0.max()) + steps + 31
    slots = rng.permutation(num_slots - 1)                       # the dummy slot is never a real token's
    table = np.full((bs_pad, width), dummy, np.int32)
    off = 0
    for r in range(bs):
        table[r, :S0[r] + steps] = slots[off:off + S0[r] + steps]
        off += S0[r] + steps
    gen = torch.Generator(device=dev).manual_seed(5)
    pool_g = torch.randn((2, num_slots, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
    pool_e = pool_g.clone()

    # static inputs of the captured step
    s_q = torch.zeros((bs_pad, HQ, D), dtype=torch.bfloat16, device=dev)
    s_k = torch.zeros((bs_pad, HKV, D), dtype=torch.bfloat16, device=dev)
    s_v = torch.zeros_like(s_k)
    s_loc = torch.full((bs_pad,), dummy, dtype=torch.int32, device=dev)
    s_table = to_dev(table)
    s_C = torch.zeros(bs_pad, dtype=torch.int32, device=dev)
    s_S = torch.ones(bs_pad, dtype=torch.int32, device=dev)
    s_logits = torch.zeros((bs_pad, V), dtype=torch.bfloat16, device=dev)
    Tp = np.zeros(bs_pad, np.float32)
    Tp[:bs] = [0.0, 0.7, 1.0, 0.7, 1.0]                          # padding rows greedy
    Pp = np.ones(bs_pad, np.float32)
    Pp[:bs] = [1.0, 0.9, 1.0, 0.95, 0.8]
    s_T, s_P = to_dev(Tp), to_dev(Pp)
    s_u = torch.zeros(bs_pad, dtype=torch.float32, device=dev)
    max_kv = bs_pad * width                                       # a bound the graph keeps for every step
    ws_d = torch.empty(pkv.decode_workspace_size(bs_pad, HQ, max_kv), dtype=torch.uint8, device=dev)
    ws_s = pkv.sample_workspace(bs_pad, V, dev)

    def step(pool, o, tok):
        kp, vp = pool[0], pool[1]
        pkv.store_kv(kp, vp, s_loc, s_k, s_v)
        pkv.paged_attention_decode(s_q, kp, vp, s_table, s_C, s_S, max_total_kv=max_kv, out=o, workspace=ws_d)
        pkv.sample(s_logits, s_T, None, s_P, s_u, out=tok, workspace=ws_s)

    def load_inputs(i):
        """Step i's inputs into the static buffers (padding rows unchanged)."""
        Si = S0 + i
        s_S[:bs] = to_dev(Si)
        s_C[:bs] = to_dev(Si - 1)
        s_loc[:bs] = to_dev(table[np.arange(bs), Si - 1])
        s_q[:bs] = torch.randn((bs, HQ, D), generator=gen, device=dev).to(torch.bfloat16)
        s_k[:bs] = torch.randn((bs, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
        s_v[:bs] = torch.randn((bs, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
        s_logits[:bs] = (torch.randn((bs, V), generator=gen, device=dev) * 3).to(torch.bfloat16)
        s_u[:bs] = torch.rand(bs, generator=gen, device=dev)

    o_g = torch.empty_like(s_q)
    t_g = torch.empty(bs_pad, dtype=torch.int32, device=dev)
    o_e, t_e = torch.empty_like(o_g), torch.empty_like(t_g)

    # warm up on a scratch pool, then capture (the capture itself runs nothing)
    load_inputs(0)
    scratch = pool_g.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(scratch, o_g, t_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del scratch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(pool_g, o_g, t_g)
    torch.cuda.synchronize()

    for i in range(steps):
        load_inputs(i)
        torch.cuda.synchronize()
        print(f"graph replay step {i}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        step(pool_e, o_e, t_e)                                    # eager twin, same static inputs
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"step {i}: decode output differs"
        assert torch.equal(t_g, t_e), f"step {i}: tokens differ"
        assert torch.equal(pool_g.view(torch.int16), pool_e.view(torch.int16)), f"step {i}: pools differ"
        assert (to_host(t_g)[bs:] == 0).all()                      # padding rows: argmax of all-zero logits
        if i == 0:  # the real rows against the oracle
            Si, got, q_h = S0, to_host(o_g), to_host(s_q)
            kp_h, vp_h = to_host(pool_g[0]), to_host(pool_g[1])
            refs = []
            for r in range(bs):
                rows = table[r, :Si[r]]
                refs.append(attention_request(oracle.widen(q_h[r:r + 1], "bf16"), oracle.widen(kp_h[rows], "bf16"),
                                              oracle.widen(vp_h[rows], "bf16"), int(Si[r] - 1))[0])
            check_attention(got[:bs], np.stack(refs), "bf16", "graph step 0 decode")
            lg = oracle.widen(to_host(s_logits)[:bs], "bf16")
            T, K, P = oracle.prepare([oracle.SamplingParams(float(Tp[r]), -1, float(Pp[r])) for r in range(bs)], V)
            want, flagged = oracle.sample(lg, T, K, P, to_host(s_u)[:bs].astype(np.float64))
            tok = to_host(t_g)[:bs]
            assert np.array_equal(tok[~flagged], want[~flagged])
    assert pkv.read_faults() == 0


# ---------------------------------------------------------------- the capture set and padded replay

def test_graph_runner_capture_set_and_padding():
    """DecodeGraphRunner with max_bs 24: sizes 1, 2, 4, 8, 16, 24 captured
    largest first into one pool. Batches of 3, 5, 13, 24, 1 and 9 requests
    run padded to 4, 8, 16, 24, 1 and 16 with the dummy request. Every replay
    (after eager work and a synchronisation) must equal the same padded step
    launched eagerly by a twin runner on a twin pool, bit for bit (outputs,
    tokens, the pool outside the dummy slot); the real rows must match the oracle (attention
    bounds; tokens exact on unflagged rows, admissible on flagged ones); only
    the real rows' slots and the dummy slot may change in the pool."""
    from paged_kv_attention_scatter_amd.graph import DecodeGraphRunner, capture_sizes
    assert capture_sizes(256) == [1, 2, 4] + list(range(8, 257, 8))
    dev = torch.device("cuda")
    rng = np.random.default_rng(77)
    n_req, max_ctx = 40, 1536
    num_slots = n_req * max_ctx + 1
    dummy = num_slots - 1
    slots = rng.permutation(num_slots - 1)
    table = np.full((n_req + 1, max_ctx), dummy, np.int32)          # last row: the dummy request
    for r in range(n_req):
        table[r] = slots[r * max_ctx:(r + 1) * max_ctx]
    gen = torch.Generator(device=dev).manual_seed(78)
    pool_g = torch.randn((2, num_slots, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
    pool_e = pool_g.clone()
    tab_g, tab_e = to_dev(table), to_dev(table)
    kw = dict(max_bs=24, vocab=V, num_q_heads=HQ, max_context=max_ctx)
    run_g = DecodeGraphRunner(pool_g[0], pool_g[1], tab_g, dummy, **kw)
    run_e = DecodeGraphRunner(pool_e[0], pool_e[1], tab_e, dummy, **kw)
    assert run_g.sizes == [1, 2, 4, 8, 16, 24]
    lens = rng.integers(200, max_ctx - 10, n_req).astype(np.int32)   # device_len before this run
    for bs, want_n in ((3, 4), (5, 8), (13, 16), (24, 24), (1, 1), (9, 16)):
        reqs = np.sort(rng.choice(n_req, bs, replace=False)).astype(np.int32)
        lens[reqs] += 1                                                # one new token each
        S = lens[reqs].copy()
        C = S - 1
        loc = table[reqs, S - 1]
        q = torch.randn((bs, HQ, D), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((bs, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((bs, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
        lg = (torch.randn((bs, V), generator=gen, device=dev) * 3).to(torch.bfloat16)
        T = np.where(rng.random(bs) < 0.5, 0.0, 0.7).astype(np.float32)
        T = np.maximum(T, np.float32(1e-6)).astype(np.float32)
        P = np.where(T > 1e-6, 0.9, 1.0).astype(np.float32)
        u = rng.random(bs, dtype=np.float32)
        args = (q, k, v, to_dev(loc), to_dev(reqs), to_dev(C), to_dev(S), lg, to_dev(T), to_dev(P), to_dev(u))
        assert run_g.size_for(bs) == want_n
        before = to_host(pool_g[0]).copy() if bs == 5 else None
        torch.cuda.synchronize()
        print(f"graph runner: batch {bs} -> captured size {want_n}", flush=True)
        o_g, t_g = run_g.run(*args)
        torch.cuda.synchronize()
        o_e, t_e = run_e.run(*args, replay=False)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"bs {bs}: decode output differs"
        assert torch.equal(t_g, t_e), f"bs {bs}: tokens differ"
        # the dummy slot takes every padding row's write: its content is unspecified
        assert torch.equal(pool_g[:, :dummy].view(torch.int16), pool_e[:, :dummy].view(torch.int16)), \
            f"bs {bs}: pools differ"
        got, q_h = to_host(o_g), to_host(q)
        kp_h, vp_h = to_host(pool_g[0]), to_host(pool_g[1])
        refs = [attention_request(oracle.widen(q_h[i:i + 1], "bf16"), oracle.widen(kp_h[table[r, :S[i]]], "bf16"),
                                  oracle.widen(vp_h[table[r, :S[i]]], "bf16"), int(C[i]))[0]
                for i, r in enumerate(reqs)]
        check_attention(got, np.stack(refs), "bf16", f"graph runner bs {bs}")
        assert np.array_equal(kp_h[loc], to_host(k)), "the new K rows are at out_loc"
        if before is not None:  # nothing but the real rows' slots and the dummy slot changed
            changed = np.nonzero(np.any(kp_h != before, axis=(1, 2)))[0]
            assert set(changed.tolist()) <= set(loc.tolist()) | {dummy}
        lf = oracle.widen(to_host(lg), "bf16")
        want, flagged = oracle.sample(lf, T, None, P, u.astype(np.float64))
        tok = to_host(t_g)
        assert np.array_equal(tok[~flagged], want[~flagged]), f"bs {bs}: tokens differ from the oracle"
        adm = oracle.admissible(lf, T, None, P, u, np.nonzero(flagged)[0].tolist())
        assert all(int(tok[i]) in adm[i] for i in np.nonzero(flagged)[0])
    assert pkv.read_faults() == 0
