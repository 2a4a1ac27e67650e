"""Benchmark of the paged-KV hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3|2] [--skip-cpu]

A step is one decode step of the whole path over one synthetic batch, on the
current HIP stream: decode attention over the paged pool with the store_kv
of the batch's new K/V rows fused into it (one call), then the sampler over
the batch's logits. The separate store_kv and decode calls are timed beside
it for reference. The default
workload is the 256-request decode batch (device_len ~ U[1024, 8192], bf16,
16 query / 8 KV heads, head_dim 128, page_size 1, pool sized for 28 layers
from 0.9 x free HBM at 114688 bytes per page; logits [256, 151936], 128
greedy rows and 128 at T=0.7, top_p=0.9). The causal extend kernel is timed
on the 8-request prefill case (extend_len ~ U[512, 4096] over a 0-50% cached
prefix) over the same pool. After that pool is freed, the mixed batch (240
decode requests with device_len ~ U[4096, 32768] plus two 2048-token prefill
chunks, page_size 16, sampler at T=1, top_k=50, top_p=0.95) is timed per
launch and as one step; its figures go into the components.

Inputs are resident in HBM before timing. The pool's contents are seeded
N(0, 1) values written by torch on the device; lengths, page tables, q,
logits, sampling parameters and uniforms come from the seeded generators in
workloads/. Rotation defeats the 256 MB Infinity Cache: successive steps use
different layers of the pool and four different logits buffers.

Prints ONE JSON line (see the keys below).
"""

import argparse
import ctypes
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
LAYERS_FILLED = 2               # layers of the pool written with data and rotated through


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=3, choices=[2, 3])
    ap.add_argument("--skip-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--skip-extend", action="store_true")
    ap.add_argument("--skip-mixed", action="store_true",
                    help="skip the mixed chunked-prefill + decode batch (page_size 16) timed after the main step")
    ap.add_argument("--skip-components", action="store_true",
                    help="skip the q/k norm + RoPE + store, embedding and graph-replay timings")
    ap.add_argument("--small-steps", type=str, default=None, metavar="BS[,BS...]",
                    help="only time eager decode steps (decode with its store, sampler) of the first BS requests of "
                         "the 256-request batch over a one-layer pool, for kernel traces; prints per-size times")
    ap.add_argument("--sampler-only", action="store_true",
                    help="only time the sampler: the 256-row mixed batch, then the variants; for kernel traces")
    ap.add_argument("--copy-calib", action="store_true",
                    help="before warm-up, run plain 1 GiB device copies (untimed) whose counter "
                         "readings calibrate FETCH_SIZE/WRITE_SIZE")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode256_traffic.md")
DECODE_SOURCES = ["paged_kv_attention_scatter_amd/csrc/decode.hpp", "paged_kv_attention_scatter_amd/csrc/decode_host.inc",
                  "paged_kv_attention_scatter_amd/csrc/common.hpp"]


def decode_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode call from the committed counter summary, or None
    when that summary was taken on a different version of the decode sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    src = re.search(r"^decode_source_hash:\s*(\S+)", text, re.M)
    val = re.search(r"^traffic_bytes_per_call:\s*(\d+)", text, re.M)
    if not src or not val or src.group(1) != decode_source_hash():
        return None
    return int(val.group(1))


def copy_calibration(torch, dev):
    """Plain device copies of known size (1 GiB read + 1 GiB written each):
    the blit behind Tensor.copy_ and an elementwise kernel."""
    n = 1 << 29
    src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 x (copy_ + neg) of {n * 2} bytes")
    del src, dst


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


SETTLE_MS = 100.0


def settle(torch, fn, ms=SETTLE_MS):
    """Untimed calls of fn for about ms of wall time. The GPU's clocks climb
    over tens of milliseconds of load (an MFMA-bound extend call runs ~20%
    slower straight after an idle second), and the host-side set-up before
    each component leaves the GPU idle, so every timed loop starts from the
    loaded state. The host waits every 8 calls, so wall time is GPU time."""
    t_end = time.perf_counter() + ms / 1e3
    n = 0
    while n < 3 or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; use --gpus 1"}))
        sys.exit(2)
    if args.small_steps:
        return small_steps(args)
    if args.sampler_only:
        return sampler_only(args)
    cpu_pools = None if args.skip_cpu else CpuPools()  # before anything touches the GPU
    import torch
    import paged_kv_attention_scatter_amd as pkv
    from workloads import (HEAD_DIM, HKV, HQ, LAYERS, config, draw_lengths, draw_logits, draw_page_table,
                           draw_q, draw_sampling_params, draw_uniforms)

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = config(args.config)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + cfg.cid)
    if args.copy_calib:
        copy_calibration(torch, dev)

    # ---------------------------------------------------------------- pool sized for 28 layers
    free, total = torch.cuda.mem_get_info()
    num_pages = pkv.num_pages(HEAD_DIM, HKV, 1, 2, LAYERS, free, 0, 0.9)
    num_slots = num_pages + 1
    log(f"free {free / 2**30:.1f} GiB -> {num_pages} pages x 28 layers "
        f"({num_slots * HKV * HEAD_DIM * 2 * 2 * LAYERS / 2**30:.1f} GiB pool)")
    pool = torch.empty((2, LAYERS, num_slots, HKV, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    for layer in range(LAYERS_FILLED):
        pool[0, layer].normal_(generator=gen)
        pool[1, layer].normal_(generator=gen)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- the decode batch
    C, S = draw_lengths(cfg)
    bs = len(S)
    table = draw_page_table(cfg, S, num_pages)
    q = torch.from_numpy(draw_q(cfg, C, S).view(np.int16)).to(dev).view(torch.bfloat16)
    out_loc_h = table[np.arange(bs), S - 1].astype(np.int32)       # slot of each new token
    d_table = torch.from_numpy(table).to(dev)
    d_C, d_S = torch.from_numpy(C).to(dev), torch.from_numpy(S).to(dev)
    d_loc = torch.from_numpy(out_loc_h).to(dev)
    new_k = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
    new_v = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
    total_kv = int(S.sum())
    ws = torch.empty(pkv.decode_workspace_size(bs, HQ, total_kv), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)

    # ---------------------------------------------------------------- sampler inputs
    logits0 = draw_logits(cfg)
    logit_bufs = [torch.from_numpy(logits0.view(np.int16)).to(dev).view(torch.bfloat16)]
    for _ in range(3):
        logit_bufs.append((torch.randn((bs, cfg.vocab), generator=gen, device=dev) * cfg.logit_sigma)
                          .to(torch.bfloat16))
    rows = draw_sampling_params(cfg)
    T, K, P = pkv.prepare_sampling(*zip(*rows), vocab=cfg.vocab)
    d_T = None if T is None else torch.from_numpy(T).to(dev)
    d_K = None if K is None else torch.from_numpy(K).to(dev)
    d_P = None if P is None else torch.from_numpy(P).to(dev)
    d_u = torch.from_numpy(draw_uniforms(cfg)).to(dev)
    tokens = torch.empty(bs, dtype=torch.int32, device=dev)
    s_ws = pkv.sample_workspace(bs, cfg.vocab, dev)

    def attend(kp, vp):  # store_kv of the new rows fused into decode attention
        pkv.paged_attention_decode_store(q, kp, vp, d_table, d_C, d_S, d_loc, new_k, new_v, max_total_kv=total_kv,
                                         out=o, workspace=ws)

    def step(i):
        layer = i % LAYERS_FILLED
        attend(pool[0, layer], pool[1, layer])
        pkv.sample(logit_bufs[i % len(logit_bufs)], d_T, d_K, d_P, d_u, out=tokens, workspace=s_ws)

    # ---------------------------------------------------------------- timed region
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    kv_bytes = total_kv * HKV * HEAD_DIM * 2 * 2           # K and V rows read, bf16
    logit_bytes = bs * cfg.vocab * 2

    # per-op durations with HIP events (same stream as the launches): the
    # step's two calls, then store_kv and decode attention as separate calls
    E = lambda: torch.cuda.Event(enable_timing=True)
    n = args.steps
    ev = [[E() for _ in range(3)] for _ in range(n)]
    for i in range(n):
        layer = i % LAYERS_FILLED
        ev[i][0].record()
        attend(pool[0, layer], pool[1, layer])
        ev[i][1].record()
        pkv.sample(logit_bufs[i % len(logit_bufs)], d_T, d_K, d_P, d_u, out=tokens, workspace=s_ws)
        ev[i][2].record()
    torch.cuda.synchronize()
    ms = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(2)] for i in range(n)])
    decode_ms, sample_ms = (float(np.mean(ms[:, j])) for j in range(2))
    decode_p = np.percentile(ms[:, 0], [10, 50, 90])
    ev = [[E() for _ in range(3)] for _ in range(n)]
    for i in range(n):
        layer = i % LAYERS_FILLED
        kp, vp = pool[0, layer], pool[1, layer]
        ev[i][0].record()
        pkv.store_kv(kp, vp, d_loc, new_k, new_v)
        ev[i][1].record()
        pkv.paged_attention_decode(q, kp, vp, d_table, d_C, d_S, max_total_kv=total_kv, out=o, workspace=ws)
        ev[i][2].record()
    torch.cuda.synchronize()
    ms = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(2)] for i in range(n)])
    store_ms, unfused_ms = (float(np.mean(ms[:, j])) for j in range(2))
    decode_gbs = kv_bytes / (decode_ms * 1e-3) / 1e9
    sample_gbs = logit_bytes / (sample_ms * 1e-3) / 1e9
    log(f"step {ms_per_step:.3f} ms | decode with its store {decode_ms * 1e3:.1f} us ({decode_gbs:.0f} GB/s) | "
        f"sample {sample_ms * 1e3:.1f} us ({sample_gbs:.0f} GB/s) | separate calls: store {store_ms * 1e3:.1f} us, "
        f"decode {unfused_ms * 1e3:.1f} us")

    result = {
        "metric": "decode-attn KV GB/s (% HBM peak) at bs=256; sampler tokens/s; extend TFLOP/s",
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: decode step (store_kv fused into decode attention + sampler), "
                               f"bs={bs}, device_len~U[{int(S.min())}..{int(S.max())}], sum={total_kv}, "
                               "16q/8kv heads, head_dim 128, page_size 1, 28-layer pool, "
                               f"logits [{bs}, {cfg.vocab}] bf16",
                   "bs": bs, "sum_device_len": total_kv, "num_pages": num_pages, "page_size": 1},
        "roofline": {"bound": "hbm", "kernel": "decode attention with its store_kv fused in (split-K + combine, one call)",
                     "achieved": round(decode_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(decode_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": kv_bytes, "avg_launch_us": round(decode_ms * 1e3, 2),
                     "p10_p50_p90_us": [round(x * 1e3, 2) for x in decode_p]},
        "components": {
            "decode_us": round(decode_ms * 1e3, 2),
            "decode_kv_gbs": round(decode_gbs, 1),
            "store_kv_separate_us": round(store_ms * 1e3, 2),
            "decode_separate_us": round(unfused_ms * 1e3, 2),
            "sample_us": round(sample_ms * 1e3, 2),
            "sampler_tokens_per_s": round(bs / (sample_ms * 1e-3), 1),
            "sampler_gbs": round(sample_gbs, 1),
            "sampler_frac_hbm": round(sample_gbs / HBM_PEAK_GBS, 4),
        },
    }

    if args.config == 3:
        result["components"].update(bench_decode64(torch, pkv, pool, num_pages, gen, dev, args))
    if not args.skip_extend:
        result["components"].update(bench_extend(torch, pkv, pool, num_pages, gen, dev, args))
    if not args.skip_components:
        result["components"].update(bench_qk_rope(torch, pkv, pool, num_pages, table, C, S, gen, dev, args))
        result["components"].update(bench_q_prologue(torch, pkv, pool, num_pages, table, C, S, gen, dev, args))
        result["components"].update(bench_embedding(torch, pkv, gen, dev, args))
        result["components"].update(bench_graph(torch, pkv, pool, table, C, S, q, gen, dev, args))
        result["components"].update(bench_sampler_variants(torch, pkv, gen, dev, args))

    if cpu_pools is not None:
        result["cpu_baseline"] = cpu_baseline(cpu_pools)
        cpu_pools.close()
    if not args.skip_mixed:
        del pool, kp, vp, logit_bufs, step
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["components"].update(bench_mixed(torch, pkv, dev, args))
    print(json.dumps(result), flush=True)


def small_steps(args):
    """Eager decode steps of the first bs requests of the 256-request batch
    (decode attention with the store_kv of their new rows fused in, then the
    sampler with their mixed parameters), over one layer's pool with the 28-layer page count, so
    the slots are as scattered as in the full pool. For kernel traces of the
    small-batch path; prints one line per batch size."""
    import torch
    import paged_kv_attention_scatter_amd as pkv
    from workloads import HEAD_DIM, HKV, HQ, LAYERS, config, draw_lengths, draw_page_table, draw_q, \
        draw_sampling_params
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1003)
    cfg = config(3)
    free, _ = torch.cuda.mem_get_info()
    num_pages = pkv.num_pages(HEAD_DIM, HKV, 1, 2, LAYERS, free, 0, 0.9)
    kp = torch.empty((num_pages + 1, HKV, HEAD_DIM), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
    vp = torch.empty_like(kp).normal_(generator=gen)
    C, S = draw_lengths(cfg)
    table = draw_page_table(cfg, S, num_pages)
    q = torch.from_numpy(draw_q(cfg, C, S).view(np.int16)).to(dev).view(torch.bfloat16)
    T_all, _, P_all = pkv.prepare_sampling(*zip(*draw_sampling_params(cfg)), vocab=cfg.vocab)
    res = {}
    for bs in (int(x) for x in args.small_steps.split(",")):
        s_q = q[:bs].clone()
        s_k = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        s_v = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        s_loc = torch.from_numpy(table[np.arange(bs), S[:bs] - 1].astype(np.int32)).to(dev)
        s_table = torch.from_numpy(np.ascontiguousarray(table[:bs])).to(dev)
        s_C, s_S = torch.from_numpy(C[:bs].copy()).to(dev), torch.from_numpy(S[:bs].copy()).to(dev)
        logits = [(torch.randn((bs, cfg.vocab), generator=gen, device=dev) * 3).to(torch.bfloat16)
                  for _ in range(4)]
        T, P = torch.from_numpy(T_all[:bs].copy()).to(dev), torch.from_numpy(P_all[:bs].copy()).to(dev)
        u = torch.rand(bs, generator=gen, device=dev)
        max_kv = int(S[:bs].sum())
        o = torch.empty_like(s_q)
        tok = torch.empty(bs, dtype=torch.int32, device=dev)
        ws_d = torch.empty(pkv.decode_workspace_size(bs, HQ, max_kv), dtype=torch.uint8, device=dev)
        ws_s = pkv.sample_workspace(bs, cfg.vocab, dev)

        def step(i):
            pkv.paged_attention_decode_store(s_q, kp, vp, s_table, s_C, s_S, s_loc, s_k, s_v, max_total_kv=max_kv,
                                             out=o, workspace=ws_d)
            pkv.sample(logits[i % 4], T, None, P, u, out=tok, workspace=ws_s)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        res[f"step_bs{bs}_us"] = round(us, 2)
        log(f"small-batch decode step bs={bs} (sum device_len {max_kv}): {us:.1f} us")
    if pkv.read_faults():
        raise RuntimeError("device fault word set during the small-batch steps")
    print(json.dumps({"small_steps": res}), flush=True)


def sampler_only(args):
    """The sampler alone: the 256-row mixed batch of the decode step (128
    greedy rows, 128 at T = 0.7, top_p = 0.9; four logits buffers rotated),
    then the variants. Prints one JSON line of the times."""
    import torch
    import paged_kv_attention_scatter_amd as pkv
    from workloads import config, draw_logits, draw_sampling_params, draw_uniforms
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1003)
    cfg = config(3)
    bs = cfg.rows
    bufs = [torch.from_numpy(draw_logits(cfg).view(np.int16)).to(dev).view(torch.bfloat16)]
    for _ in range(3):
        bufs.append((torch.randn((bs, cfg.vocab), generator=gen, device=dev) * cfg.logit_sigma).to(torch.bfloat16))
    T, K, P = pkv.prepare_sampling(*zip(*draw_sampling_params(cfg)), vocab=cfg.vocab)
    to = lambda x: None if x is None else torch.from_numpy(x).to(dev)
    d_T, d_K, d_P, d_u = to(T), to(K), to(P), to(draw_uniforms(cfg))
    tokens = torch.empty(bs, dtype=torch.int32, device=dev)
    ws = pkv.sample_workspace(bs, cfg.vocab, dev)
    for i in range(args.warmup):
        pkv.sample(bufs[i % 4], d_T, d_K, d_P, d_u, out=tokens, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        pkv.sample(bufs[i % 4], d_T, d_K, d_P, d_u, out=tokens, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    log(f"sampler decode256 mix: {us:.1f} us ({bs * cfg.vocab * 2 / us / 1e3:.0f} GB/s)")
    res = {"sample_us": round(us, 2)}
    res.update(bench_sampler_variants(torch, pkv, gen, dev, args))
    print(json.dumps(res), flush=True)


def bench_decode64(torch, pkv, pool, num_pages, gen, dev, args):
    """The 64-request decode batch (device_len ~ U[256, 2048], bf16, page_size
    1, same 28-layer pool) with an all-greedy sampler (no temperature array:
    the argmax path) over [64, 151936] logits: store_kv, decode attention,
    decode with the store fused in and the argmax timed apart with HIP events
    on the launch stream, and the step (decode with its store, argmax).
    Calls that read the pool rotate over the filled layers and four
    relabelings of the slots (8 sets of K/V rows, 2.3 GB), so that no call
    finds its rows left in L2 or the MALL by the one before it; the argmax
    rotates over four logits buffers."""
    from workloads import (HEAD_DIM, HKV, HQ, config, draw_lengths, draw_logits, draw_page_table, draw_q,
                           draw_sampling_params)
    cfg = config(2)
    C, S = draw_lengths(cfg)
    bs = len(S)
    table = draw_page_table(cfg, S, num_pages)
    q = torch.from_numpy(draw_q(cfg, C, S).view(np.int16)).to(dev).view(torch.bfloat16)
    sets = []
    for r in range(4):
        t = ((table.astype(np.int64) + r * 600_011) % num_pages).astype(np.int32)
        d_t = torch.from_numpy(t).to(dev)
        d_l = torch.from_numpy(t[np.arange(bs), S - 1].copy()).to(dev)
        sets += [(pool[0, layer], pool[1, layer], d_t, d_l) for layer in range(LAYERS_FILLED)]
    d_C, d_S = torch.from_numpy(C).to(dev), torch.from_numpy(S).to(dev)
    new_k = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
    new_v = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
    total_kv = int(S.sum())
    ws = torch.empty(pkv.decode_workspace_size(bs, HQ, total_kv), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    T, K, P = pkv.prepare_sampling(*zip(*draw_sampling_params(cfg)), vocab=cfg.vocab)
    assert T is None  # all greedy: the argmax path
    bufs = [torch.from_numpy(draw_logits(cfg).view(np.int16)).to(dev).view(torch.bfloat16)]
    for _ in range(3):
        bufs.append((torch.randn((bs, cfg.vocab), generator=gen, device=dev) * cfg.logit_sigma).to(torch.bfloat16))
    tokens = torch.empty(bs, dtype=torch.int32, device=dev)
    s_ws = pkv.sample_workspace(bs, cfg.vocab, dev)
    # Per iteration i: the separate store and decode on set 2i, the fused call
    # on set 2i + 1 (mod 8).
    def sset(i, j):
        return sets[(2 * i + j) % len(sets)]
    ops = [lambda i: pkv.store_kv(sset(i, 0)[0], sset(i, 0)[1], sset(i, 0)[3], new_k, new_v),
           lambda i: pkv.paged_attention_decode(q, sset(i, 0)[0], sset(i, 0)[1], sset(i, 0)[2], d_C, d_S,
                                                max_total_kv=total_kv, out=o, workspace=ws),
           lambda i: pkv.sample(bufs[i % len(bufs)], None, None, None, None, out=tokens, workspace=s_ws),
           lambda i: pkv.paged_attention_decode_store(q, sset(i, 1)[0], sset(i, 1)[1], sset(i, 1)[2], d_C, d_S,
                                                      sset(i, 1)[3], new_k, new_v, max_total_kv=total_kv,
                                                      out=o, workspace=ws)]
    step_ops = (ops[3], ops[2])  # the step: store fused into decode, then the argmax
    it = iter(range(1 << 30))

    def one_step():
        i = next(it)
        for op in ops:
            op(i)
    settle(torch, one_step)
    n = max(20, args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(n)]
    for i in range(n):
        for j, op in enumerate(ops):
            ev[i][j].record()
            op(i)
        ev[i][len(ops)].record()
    torch.cuda.synchronize()
    ms = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(ops))] for i in range(n)])
    st_us, dec_us, am_us, fused_us = (float(np.mean(ms[:, j])) * 1e3 for j in range(len(ops)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        for op in step_ops:
            op(i)
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / n * 1e3
    kv = total_kv * HKV * HEAD_DIM * 2 * 2
    lg = bs * cfg.vocab * 2
    log(f"decode64: store {st_us:.1f} us | decode {dec_us:.1f} us ({kv / dec_us / 1e3:.0f} GB/s) | "
        f"decode with its store {fused_us:.1f} us | argmax {am_us:.1f} us ({lg / am_us / 1e3:.0f} GB/s) | "
        f"step {step_us:.1f} us")
    if pkv.read_faults():
        raise RuntimeError("device fault word set during the decode64 timing")
    return {"decode64_workload": f"bs=64, device_len {int(S.min())}..{int(S.max())}, sum {total_kv}, "
                                 f"page_size 1, all greedy (argmax) over [64, {cfg.vocab}] bf16",
            "decode64_store_us": round(st_us, 2), "decode64_decode_us": round(dec_us, 2),
            "decode64_decode_store_us": round(fused_us, 2),
            "decode64_decode_kv_gbs": round(kv / dec_us / 1e3, 1),
            "decode64_decode_frac_hbm": round(kv / dec_us / 1e3 / HBM_PEAK_GBS, 4),
            "decode64_argmax_us": round(am_us, 2), "decode64_argmax_gbs": round(lg / am_us / 1e3, 1),
            "decode64_argmax_frac_hbm": round(lg / am_us / 1e3 / HBM_PEAK_GBS, 4),
            "decode64_argmax_tokens_per_s": round(bs / (am_us * 1e-6), 1),
            "decode64_step_us": round(step_us, 2)}


def bench_extend(torch, pkv, pool, num_pages, gen, dev, args):
    """Causal extend over a cached prefix: 8 requests, E ~ U[512, 4096],
    prefix 0-50%, page_size 1, over the same pool. Calls rotate over the
    filled layers and four relabelings of the slots (8 sets of K/V rows, about
    1 GB), so that no call finds its rows left in L2 or the MALL by the
    previous calls, as when each layer of a prefill reads its own rows."""
    from workloads import HEAD_DIM, HQ, config, draw_lengths, draw_page_table, draw_q
    cfg = config(4)
    C, S = draw_lengths(cfg)
    E = S - C
    table = draw_page_table(cfg, S, num_pages)
    q = torch.from_numpy(draw_q(cfg, C, S).view(np.int16)).to(dev).view(torch.bfloat16)
    tables = [torch.from_numpy(((table.astype(np.int64) + r * 600_011) % num_pages).astype(np.int32)).to(dev)
              for r in range(4)]
    sets = [(pool[0, layer], pool[1, layer], t) for t in tables for layer in range(LAYERS_FILLED)]
    d_C, d_S = torch.from_numpy(C).to(dev), torch.from_numpy(S).to(dev)
    o = torch.empty_like(q)
    flops = 4.0 * HEAD_DIM * HQ * float(np.sum(E.astype(np.float64) * C + E * (E + 1) / 2.0))
    it = iter(range(1 << 30))

    def call():
        kp, vp, d_table = sets[next(it) % len(sets)]
        pkv.paged_attention_extend(q, kp, vp, d_table, d_C, d_S, max_extend=int(E.max()), out=o)
    try:
        call()
    except pkv.PkvError as e:
        log(f"extend skipped: {e}")
        return {"extend": f"unavailable: {e}"}
    settle(torch, call)
    n = max(16, args.steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    tflops = flops / (us * 1e-6) / 1e12
    log(f"extend {us:.1f} us, {flops / 1e12:.3f} TFLOP -> {tflops:.1f} TFLOP/s")
    return {"extend_us": round(us, 2), "extend_tflop": round(flops / 1e12, 4),
            "extend_tflops": round(tflops, 1), "extend_frac_mfma": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "extend_workload": f"8 requests, extend_len {int(E.min())}..{int(E.max())}, "
                               f"prefix {int(C.min())}..{int(C.max())}, bf16, page_size 1, "
                               f"K/V rows rotated over {len(sets)} sets"}


def bench_qk_rope(torch, pkv, pool, num_pages, table, C, S, gen, dev, args):
    """q/k RMSNorm + rotary embedding + K/V store, fused (the step before
    attention): on the 256 new tokens of the decode batch (positions
    device_len - 1, slots from its page table) and on the 19,892 new tokens
    of the 8-request prefill (positions cached_len + t, slots from its page
    table), over layer 0 of the pool. Bytes per token: q read and written
    (16 heads), k and v read, K and V rows written (8 heads), bf16: 16 KiB."""
    from workloads import HEAD_DIM, HKV, HQ, config, draw_lengths, draw_page_table
    kp, vp = pool[0, 0], pool[1, 0]
    wq = (torch.rand(HEAD_DIM, generator=gen, device=dev) + 0.5).to(torch.bfloat16)
    wk = (torch.rand(HEAD_DIM, generator=gen, device=dev) + 0.5).to(torch.bfloat16)
    cases = {}
    C4, S4 = draw_lengths(config(4))
    t4 = draw_page_table(config(4), S4, num_pages)
    for name, pos, loc in (
            ("decode256", (S - 1).astype(np.int32), table[np.arange(len(S)), S - 1].astype(np.int32)),
            ("prefill8", np.concatenate([np.arange(c, s) for c, s in zip(C4, S4)]).astype(np.int32),
             np.concatenate([t4[r, C4[r]:S4[r]] for r in range(len(S4))]).astype(np.int32))):
        n = len(pos)
        q = torch.randn((n, HQ, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((n, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((n, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        qo = torch.empty_like(q)
        d_pos, d_loc = torch.from_numpy(pos).to(dev), torch.from_numpy(loc).to(dev)
        pkv.qk_norm_rope_store_kv(kp, vp, d_loc, q, k, v, d_pos, wq, wk, q_out=qo)  # checked once
        # the timed loop calls the C ABI with the same arguments marshalled once,
        # so a 256-token call is not timed at the Python wrapper's pace
        pool_desc = pkv.make_pool(kp, vp, 1)
        c_args = (ctypes.byref(pool_desc), d_loc.data_ptr(), 0, n, q.data_ptr(), 0, qo.data_ptr(),
                  0, HQ, k.data_ptr(), HKV * HEAD_DIM, v.data_ptr(), HKV * HEAD_DIM, d_pos.data_ptr(),
                  wq.data_ptr(), wk.data_ptr(), 1e-6, 1_000_000.0, torch.cuda.current_stream().cuda_stream)
        fn = pkv.lib().pkv_qk_norm_rope_store_kv
        run = lambda: fn(*c_args)
        if run() != 0:
            raise RuntimeError(pkv.lib().pkv_last_error().decode())
        settle(torch, run)
        reps = max(20, args.steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        nbytes = n * 2 * (2 * HQ + 4 * HKV) * HEAD_DIM
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"qk norm+rope+store {name}: {n} tokens, {us:.1f} us, {gbs:.0f} GB/s")
        cases[f"qk_rope_store_{name}_us"] = round(us, 2)
        cases[f"qk_rope_store_{name}_gbs"] = round(gbs, 1)
        cases[f"qk_rope_store_{name}_frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
    if pkv.read_faults():
        raise RuntimeError("device fault word set during the qk norm/rope/store timing")
    return cases


def bench_q_prologue(torch, pkv, pool, num_pages, table, C, S, gen, dev, args):
    """q's RMSNorm + RoPE in the attention prologue against the unfused chain,
    over layer 0 of the pool: the 8-request prefill (19,892 new tokens: the
    store call normalises, rotates and stores k; extend normalises and
    rotates q itself) and the 256-request decode step. Unfused: the store
    call also writes q_out (q read, q_out written, read again by attention)."""
    from workloads import HEAD_DIM, HKV, HQ, config, draw_lengths, draw_page_table
    kp, vp = pool[0, 0], pool[1, 0]
    wq = (torch.rand(HEAD_DIM, generator=gen, device=dev) + 0.5).to(torch.bfloat16)
    wk = (torch.rand(HEAD_DIM, generator=gen, device=dev) + 0.5).to(torch.bfloat16)
    C4, S4 = draw_lengths(config(4))
    t4 = draw_page_table(config(4), S4, num_pages)
    out = {}
    for name, Cc, Sc, tab in (("prefill8", C4, S4, t4), ("decode256", C, S, table)):
        pos = np.concatenate([np.arange(c, s) for c, s in zip(Cc, Sc)]).astype(np.int32)
        loc = np.concatenate([tab[r, Cc[r]:Sc[r]] for r in range(len(Sc))]).astype(np.int32)
        n = len(pos)
        q = torch.randn((n, HQ, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((n, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((n, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        qo, o = torch.empty_like(q), torch.empty_like(q)
        d_pos, d_loc = torch.from_numpy(pos).to(dev), torch.from_numpy(loc).to(dev)
        d_tab = torch.from_numpy(tab).to(dev)
        d_C, d_S = torch.from_numpy(Cc).to(dev), torch.from_numpy(Sc).to(dev)
        E = Sc - Cc
        if name == "prefill8":
            attn = lambda qq, **kw: pkv.paged_attention_extend(qq, kp, vp, d_tab, d_C, d_S, max_extend=int(E.max()),
                                                              out=o, **kw)
        else:
            ws = torch.empty(pkv.decode_workspace_size(len(Sc), HQ, int(Sc.sum())), dtype=torch.uint8, device=dev)
            attn = lambda qq, **kw: pkv.paged_attention_decode(qq, kp, vp, d_tab, d_C, d_S,
                                                              max_total_kv=int(Sc.sum()), out=o, workspace=ws, **kw)

        def unfused():
            pkv.qk_norm_rope_store_kv(kp, vp, d_loc, q, k, v, d_pos, wq, wk, q_out=qo)
            attn(qo)

        def fused():
            pkv.qk_norm_rope_store_kv(kp, vp, d_loc, None, k, v, d_pos, None, wk)
            attn(q, q_norm_weight=wq)

        times = {}
        for label, fn in (("unfused", unfused), ("fused", fused)):
            settle(torch, fn)
            reps = max(20, args.steps // 2)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times[label] = e0.elapsed_time(e1) / reps * 1e3
        log(f"q prologue {name}: store + attention unfused {times['unfused']:.1f} us, q norm/rope folded into "
            f"attention {times['fused']:.1f} us (q round trip {n * HQ * HEAD_DIM * 2 * 2 / 1e6:.1f} MB)")
        out[f"q_prologue_{name}_unfused_us"] = round(times["unfused"], 2)
        out[f"q_prologue_{name}_fused_us"] = round(times["fused"], 2)
    if pkv.read_faults():
        raise RuntimeError("device fault word set during the q prologue timing")
    return out


def bench_embedding(torch, pkv, gen, dev, args):
    """Embedding row gather (the first op of forward_batch) from a
    Qwen3-0.6B-shaped table ([151936, 1024] bf16, drawn on the device) for 256
    decode tokens and for the 19,892 tokens of the 8-request prefill (seeded
    random ids). Bytes per token: one 2 KiB row read and one written."""
    V, H = 151936, 1024
    W = torch.empty((V, H), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
    rng = np.random.default_rng(31)
    out = {}
    for name, n in (("decode256", 256), ("prefill8", 19892)):
        ids = torch.from_numpy(rng.integers(0, V, n).astype(np.int32)).to(dev)
        o = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
        pkv.embedding_gather(W, ids, out=o)  # checked once
        fn = pkv.lib().pkv_embedding_gather
        c_args = (W.data_ptr(), 1, V, H, H, ids.data_ptr(), n, 0, V, o.data_ptr(), H,
                  torch.cuda.current_stream().cuda_stream)
        if fn(*c_args) != 0:
            raise RuntimeError(pkv.lib().pkv_last_error().decode())
        settle(torch, lambda: fn(*c_args))
        reps = max(20, args.steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn(*c_args)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        gbs = n * H * 2 * 2 / (us * 1e-6) / 1e9
        log(f"embedding gather {name}: {n} tokens, {us:.1f} us, {gbs:.0f} GB/s")
        out[f"embedding_{name}_us"] = round(us, 2)
        out[f"embedding_{name}_gbs"] = round(gbs, 1)
        out[f"embedding_{name}_frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
    del W
    return out


def bench_sampler_variants(torch, pkv, gen, dev, args):
    """The sampler on [256, 151936] logits, bf16 and fp32 (the dtype of an
    fp32 logits buffer), one parameter mix per batch: all greedy, plain
    (T = 1, no cut), top-k 50, top-p 0.9 (at T = 1 and at T = 0.7), top-k 50
    + top-p 0.95, min_p 0.05, and all three cuts; T = 1 unless stated. Logits ~ N(0, 3^2) drawn on the device, rotated over
    311 MB of buffers so the Infinity Cache does not hold them. Algorithmic
    bytes per call: one read of the logits."""
    bs, V = 256, 151936
    out = {}
    tokens = torch.empty(bs, dtype=torch.int32, device=dev)
    ws = pkv.sample_workspace(bs, V, dev)
    u = torch.rand(bs, generator=gen, device=dev)
    full = lambda v, dt=torch.float32: torch.full((bs,), v, dtype=dt, device=dev)
    mixes = [("greedy", None, None, None, None), ("plain", full(1.0), None, None, None),
             ("topk50", full(1.0), full(50, torch.int32), None, None),
             ("topp09", full(1.0), None, full(0.9), None),
             ("t07_topp09", full(0.7), None, full(0.9), None),
             ("k50_p095", full(1.0), full(50, torch.int32), full(0.95), None),
             ("minp005", full(1.0), None, None, full(0.05)),
             ("k50_p095_minp005", full(1.0), full(50, torch.int32), full(0.95), full(0.05))]
    ptr = lambda t: None if t is None else t.data_ptr()
    fn = pkv.lib().pkv_sample
    stream = torch.cuda.current_stream().cuda_stream
    for dt, code, nbuf in ((torch.bfloat16, 1, 4), (torch.float32, 0, 2)):
        tag = "bf16" if code else "f32"
        bufs = [(torch.randn((bs, V), generator=gen, device=dev) * 3.0).to(dt) for _ in range(nbuf)]
        for name, T, K, P, MP in mixes:
            calls = [(b.data_ptr(), code, bs, V, V, ptr(T), ptr(K), ptr(P), ptr(MP), u.data_ptr(),
                      tokens.data_ptr(), ws.data_ptr(), ws.numel(), stream) for b in bufs]
            for c in calls:
                if fn(*c) != 0:
                    raise RuntimeError(pkv.lib().pkv_last_error().decode())
            it = iter(range(1 << 30))
            settle(torch, lambda: fn(*calls[next(it) % nbuf]), SETTLE_MS / 2)
            reps = max(8, args.steps // 4) * nbuf
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fn(*calls[i % nbuf])
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            gbs = bs * V * bufs[0].element_size() / (us * 1e-6) / 1e9
            key = f"sampler256_{tag}_{name}"
            out[key + "_us"] = round(us, 2)
            out[key + "_frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
        log(f"sampler [256, 151936] {tag}: " + ", ".join(f"{n} {out[f'sampler256_{tag}_{n}_us']:.1f} us"
                                                          for n, *_ in mixes))
        del bufs
    if pkv.read_faults():
        raise RuntimeError("device fault word set during the sampler variants")
    return out


def bench_graph(torch, pkv, pool, table, C, S, q, gen, dev, args):
    """Decode steps (decode attention with the store fused in, sampler) of the first bs
    requests of the 256-request batch over layer 0 of the pool, through the
    graph runner: sizes 1, 2, 4, 8, 16, ..., 256 captured largest first into
    one pool, a batch padded to the next captured size with the dummy
    request. For bs = 1, 5, 8, 60, 64 and 256: the step issued eagerly through
    the Python binding (unpadded), the padded graph replay with its inputs
    already in the runner's buffers, and run() (copying the batch in, then
    the replay). These three repeat one batch over the same K/V rows, which
    for small batches stay in L2 and the MALL from one step to the next; a
    fourth leg issues the eager step over 8 sets of rows in turn (the filled
    layers x four relabelings of the slots), as the layers of a model would."""
    from paged_kv_attention_scatter_amd.graph import DecodeGraphRunner
    from workloads import HEAD_DIM, HKV, HQ, config, draw_sampling_params
    V = config(3).vocab
    rows = draw_sampling_params(config(3))
    T_all, _, P_all = pkv.prepare_sampling(*zip(*rows), vocab=V)
    kp, vp = pool[0, 0], pool[1, 0]
    dummy_slot = kp.shape[0] - 1                         # the dummy page (page_size 1)
    tab = np.full((table.shape[0] + 1, table.shape[1]), dummy_slot, np.int32)
    tab[:-1] = table
    d_tab = torch.from_numpy(tab).to(dev)
    runner = DecodeGraphRunner(kp, vp, d_tab, dummy_slot, max_bs=256, vocab=V, num_q_heads=HQ,
                               max_context=table.shape[1])
    out = {"graph_capture_sizes": len(runner.sizes)}
    reps = max(50, args.steps)

    def timed(fn):
        settle(torch, fn, SETTLE_MS / 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    cold_sets = []
    for r in range(4):
        t = tab.astype(np.int64)
        t[:-1] = (t[:-1] + r * 600_011) % dummy_slot
        d_t = torch.from_numpy(t.astype(np.int32)).to(dev)
        cold_sets += [(pool[0, layer], pool[1, layer], d_t, t) for layer in range(LAYERS_FILLED)]

    for bs in (1, 5, 8, 60, 64, 256):
        n = runner.size_for(bs)
        b_q = q[:bs].clone()
        b_k = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        b_v = torch.randn((bs, HKV, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
        b_loc = torch.from_numpy(table[np.arange(bs), S[:bs] - 1].astype(np.int32)).to(dev)
        b_idx = torch.arange(bs, dtype=torch.int32, device=dev)
        b_C, b_S = torch.from_numpy(C[:bs].copy()).to(dev), torch.from_numpy(S[:bs].copy()).to(dev)
        b_lg = (torch.randn((bs, V), generator=gen, device=dev) * 3).to(torch.bfloat16)
        b_T, b_P = torch.from_numpy(T_all[:bs].copy()).to(dev), torch.from_numpy(P_all[:bs].copy()).to(dev)
        b_u = torch.rand(bs, generator=gen, device=dev)
        max_kv = int(S[:bs].sum())
        o = torch.empty_like(b_q)
        tok = torch.empty(bs, dtype=torch.int32, device=dev)
        ws_d = torch.empty(pkv.decode_workspace_size(bs, HQ, max_kv), dtype=torch.uint8, device=dev)
        ws_s = pkv.sample_workspace(bs, V, dev)

        def eager():
            pkv.paged_attention_decode_store(b_q, kp, vp, d_tab, b_C, b_S, b_loc, b_k, b_v, table_idx=b_idx,
                                             max_total_kv=max_kv, out=o, workspace=ws_d)
            pkv.sample(b_lg, b_T, None, b_P, b_u, out=tok, workspace=ws_s)

        cold_locs = [torch.from_numpy(cs[3][np.arange(bs), S[:bs] - 1].astype(np.int32)).to(dev) for cs in cold_sets]
        it = iter(range(1 << 30))

        def eager_cold():
            i = next(it) % len(cold_sets)
            ck, cv, ct, _ = cold_sets[i]
            pkv.paged_attention_decode_store(b_q, ck, cv, ct, b_C, b_S, cold_locs[i], b_k, b_v, table_idx=b_idx,
                                             max_total_kv=max_kv, out=o, workspace=ws_d)
            pkv.sample(b_lg, b_T, None, b_P, b_u, out=tok, workspace=ws_s)

        args_run = (b_q, b_k, b_v, b_loc, b_idx, b_C, b_S, b_lg, b_T, b_P, b_u)
        runner.run(*args_run)                            # stage this batch (and pad it) once
        t_eager = timed(eager)
        t_replay = timed(runner.graphs[n].replay)
        t_run = timed(lambda: runner.run(*args_run))
        t_cold = timed(eager_cold)
        log(f"decode step bs={bs} (graph size {n}): eager {t_eager:.1f} us, graph replay {t_replay:.1f} us, "
            f"copy-in + replay {t_run:.1f} us; eager over 8 sets of rows {t_cold:.1f} us")
        out[f"step_bs{bs}_eager_us"] = round(t_eager, 2)
        out[f"step_bs{bs}_eager_rotated_us"] = round(t_cold, 2)
        out[f"step_bs{bs}_graph_us"] = round(t_replay, 2)
        out[f"step_bs{bs}_graph_run_us"] = round(t_run, 2)
    del runner
    if pkv.read_faults():
        raise RuntimeError("device fault word set during the graph timing")
    return out


def bench_mixed(torch, pkv, dev, args):
    """The mixed batch: 240 decode requests (device_len ~ U[4096, 32768]) and 2
    prefill chunks of 2048 tokens over cached prefixes of 2048 j tokens, bf16,
    page_size 16, one layer's pool sized 1.25 x the pages the batch uses; the
    sampler over [242, 151936] logits, every row at T=1, top_k=50,
    top_p=0.95. One decode launch, one extend launch and the sampler on one
    stream: timed apart and as one step. Timed alone, the extend rotates over
    four relabelings of the chunks' pages, so that no call finds its K/V rows
    left in L2 or the MALL by the previous ones."""
    from workloads import (HEAD_DIM, HKV, HQ, config, default_num_pages, draw_lengths, draw_page_table,
                           draw_q, draw_sampling_params, draw_uniforms)
    cfg = config(5)
    C, S = draw_lengths(cfg)
    nump = default_num_pages(cfg, S)
    table = draw_page_table(cfg, S, nump)
    E = (S - C).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(E)])
    dec = np.nonzero(E == 1)[0].astype(np.int32)
    ext = np.nonzero(E > 1)[0].astype(np.int32)
    q_all = draw_q(cfg, C, S).view(np.int16)
    q_dec = torch.from_numpy(q_all[cu[dec]]).to(dev).view(torch.bfloat16)
    q_ext = torch.from_numpy(np.concatenate([q_all[cu[r]:cu[r + 1]] for r in ext])).to(dev).view(torch.bfloat16)
    num_slots = (nump + 1) * cfg.page_size
    gen = torch.Generator(device=dev)
    gen.manual_seed(1005)
    kp = torch.empty((num_slots, HKV, HEAD_DIM), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
    vp = torch.empty((num_slots, HKV, HEAD_DIM), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
    d_table = torch.from_numpy(table).to(dev)
    d_C, d_S = torch.from_numpy(C).to(dev), torch.from_numpy(S).to(dev)
    d_dec, d_ext = torch.from_numpy(dec).to(dev), torch.from_numpy(ext).to(dev)
    Cd, Sd = d_C[d_dec].contiguous(), d_S[d_dec].contiguous()
    Ce, Se = d_C[d_ext].contiguous(), d_S[d_ext].contiguous()
    dec_kv = int(S[dec].sum())
    max_ext = int(E[ext].max())
    ws = torch.empty(pkv.decode_workspace_size(len(dec), HQ, dec_kv), dtype=torch.uint8, device=dev)
    o_dec, o_ext = torch.empty_like(q_dec), torch.empty_like(q_ext)
    rows = cfg.rows
    bufs = [(torch.randn((rows, cfg.vocab), generator=gen, device=dev) * cfg.logit_sigma).to(torch.bfloat16)
            for _ in range(4)]
    T, K, P = pkv.prepare_sampling(*zip(*draw_sampling_params(cfg)), vocab=cfg.vocab)
    to = lambda x: None if x is None else torch.from_numpy(x).to(dev)
    d_T, d_K, d_P, d_u = to(T), to(K), to(P), to(draw_uniforms(cfg))
    tokens = torch.empty(rows, dtype=torch.int32, device=dev)
    s_ws = pkv.sample_workspace(rows, cfg.vocab, dev)
    ps = cfg.page_size

    def decode():
        pkv.paged_attention_decode(q_dec, kp, vp, d_table, Cd, Sd, table_idx=d_dec, max_total_kv=dec_kv,
                                   page_size=ps, out=o_dec, workspace=ws)

    ext_tables = []
    for r in range(4):
        t = table.astype(np.int64)
        t[ext] = (t[ext] + r * 100_003 * cfg.page_size) % (nump * cfg.page_size)
        ext_tables.append(torch.from_numpy(t.astype(np.int32)).to(dev))

    def extend(i=0):
        pkv.paged_attention_extend(q_ext, kp, vp, ext_tables[i % len(ext_tables)], Ce, Se, table_idx=d_ext,
                                   max_extend=max_ext, page_size=ps, out=o_ext)

    def sample(i):
        pkv.sample(bufs[i % len(bufs)], d_T, d_K, d_P, d_u, out=tokens, workspace=s_ws)

    d_mp = torch.full((rows,), 0.05, dtype=torch.float32, device=dev)

    def sample_min_p(i):  # the same rows with min_p = 0.05 on top
        pkv.sample(bufs[i % len(bufs)], d_T, d_K, d_P, d_u, min_p=d_mp, out=tokens, workspace=s_ws)

    def timed(fn, n):
        it = iter(range(1 << 30))
        settle(torch, lambda: fn(next(it)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    n = max(10, args.steps // 4)
    dec_us = timed(lambda i: decode(), n)
    ext_us = timed(extend, n)
    smp_us = timed(sample, 4 * n)
    smp_mp_us = timed(sample_min_p, 4 * n)
    step_us = timed(lambda i: (decode(), extend(), sample(i)), n)
    kv_bytes = dec_kv * HKV * HEAD_DIM * 2 * 2
    flops = 4.0 * HEAD_DIM * HQ * float(np.sum(E[ext] * C[ext] + E[ext] * (E[ext] + 1) / 2.0))
    dec_gbs = kv_bytes / (dec_us * 1e-6) / 1e9
    ext_tf = flops / (ext_us * 1e-6) / 1e12
    smp_gbs = rows * cfg.vocab * 2 / (smp_us * 1e-6) / 1e9
    log(f"mixed242: decode {dec_us:.1f} us ({dec_gbs:.0f} GB/s) | extend {ext_us:.1f} us ({ext_tf:.0f} TFLOP/s) "
        f"| sample {smp_us:.1f} us ({smp_gbs:.0f} GB/s; {smp_mp_us:.1f} us with min_p 0.05) | step {step_us:.1f} us")
    if pkv.read_faults():
        raise RuntimeError("device fault word set during the mixed batch")
    return {"mixed242_workload": f"240 decode rows (device_len {int(S[dec].min())}..{int(S[dec].max())}, "
                                 f"sum {dec_kv}) + 2 prefill chunks of 2048 over prefixes {C[ext].tolist()}, "
                                 f"page_size 16, {num_slots} slots; sampler [242, {cfg.vocab}] T=1 k=50 p=0.95",
            "mixed242_decode_us": round(dec_us, 2), "mixed242_decode_kv_gbs": round(dec_gbs, 1),
            "mixed242_decode_frac_hbm": round(dec_gbs / HBM_PEAK_GBS, 4),
            "mixed242_extend_us": round(ext_us, 2), "mixed242_extend_tflops": round(ext_tf, 1),
            "mixed242_extend_frac_mfma": round(ext_tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "mixed242_sample_us": round(smp_us, 2), "mixed242_sampler_gbs": round(smp_gbs, 1),
            "mixed242_sampler_tokens_per_s": round(rows / (smp_us * 1e-6), 1),
            "mixed242_sample_min_p_us": round(smp_mp_us, 2),
            "mixed242_step_us": round(step_us, 2)}


# ---------------------------------------------------------------- CPU baseline (the oracle on the host cores)
#
# Worker processes are started with the "spawn" method before the GPU is
# initialised and import only NumPy, the seeded generators and the oracle.
# Each worker draws its share of the inputs with the workloads generators
# (untimed), waits at a barrier, then runs the oracle on them; the time is
# from the first worker's start to the last worker's end.

_CPU_BARRIER = None


def _cpu_worker_init(barrier, cpu):
    global _CPU_BARRIER
    _CPU_BARRIER = barrier
    if cpu is not None:
        os.sched_setaffinity(0, {cpu.get()})


def _cpu_worker_task(job):
    import oracle
    from workloads import config, draw_logits, draw_lengths, draw_q, draw_request_kv, draw_sampling_params, \
        draw_uniforms, f32_to_bf16_bits
    kind, items = job
    if kind == "decode":  # items: request ids of the 256-request decode batch
        cfg = config(3)
        C, S = draw_lengths(cfg)
        q = draw_q(cfg, C, S)
        data = []
        for r in items:
            K, V = draw_request_kv(cfg, r, int(S[r]))
            data.append((r, f32_to_bf16_bits(K), f32_to_bf16_bits(V)))
        _CPU_BARRIER.wait(timeout=300)
        t0 = time.perf_counter()
        nbytes = 0
        for r, K, V in data:
            tab = np.arange(int(S[r]), dtype=np.int64)[None, :]
            oracle.attention_decode(q[r:r + 1], K, V, tab, C[r:r + 1], S[r:r + 1], "bf16")
            nbytes += int(S[r]) * 8 * 128 * 2 * 2
        return t0, time.perf_counter(), nbytes
    if kind == "extend":  # items: (request, t0, t1) query-row spans of the 8-request prefill
        cfg = config(4)
        C, S = draw_lengths(cfg)
        q = draw_q(cfg, C, S)
        cu = np.concatenate([[0], np.cumsum(S - C)])
        data = []
        for r, a, b in items:
            K, V = draw_request_kv(cfg, r, int(S[r]))
            n = int(C[r]) + b
            data.append((r, a, b, f32_to_bf16_bits(K[:n]), f32_to_bf16_bits(V[:n])))
        _CPU_BARRIER.wait(timeout=300)
        t0 = time.perf_counter()
        flops = 0.0
        for r, a, b, K, V in data:
            c = int(C[r])
            tab = np.arange(c + b, dtype=np.int64)[None, :]
            oracle.attention_extend(q[cu[r] + a:cu[r] + b], K, V, tab, np.array([c + a], np.int32),
                                    np.array([c + b], np.int32), "bf16")
            flops += 4.0 * 128 * 16 * float(sum(c + t + 1 for t in range(a, b)))
        return t0, time.perf_counter(), flops
    if kind == "sample":  # items: row ids of the 256-row mixed sampler batch
        cfg = config(3)
        lf = oracle.widen(draw_logits(cfg)[list(items)], "bf16")
        T, K, P = oracle.prepare([oracle.SamplingParams(*p) for p in draw_sampling_params(cfg)], cfg.vocab)
        u = draw_uniforms(cfg)
        sel = lambda x: None if x is None else x[list(items)]
        _CPU_BARRIER.wait(timeout=300)
        t0 = time.perf_counter()
        oracle.sample(lf, sel(T), sel(K), sel(P), sel(u))
        return t0, time.perf_counter(), len(items)
    raise ValueError(kind)


def host_cpus():
    """(logical CPUs this process may use, one logical CPU per physical core
    among them, CPU model name)."""
    cpus = sorted(os.sched_getaffinity(0))
    cores = {}
    for c in cpus:
        try:
            with open(f"/sys/devices/system/cpu/cpu{c}/topology/core_id") as f:
                core = f.read().strip()
            with open(f"/sys/devices/system/cpu/cpu{c}/topology/physical_package_id") as f:
                pkg = f.read().strip()
        except OSError:
            core, pkg = str(c), "0"
        cores.setdefault((pkg, core), c)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cpus, sorted(cores.values()), model


class CpuPools:
    """Two oracle pools: every logical CPU of this process's share (at most
    16, the host share of one GPU), and one logical CPU per physical core.
    Created before the GPU is initialised."""

    def __init__(self):
        import multiprocessing as mp
        self.ctx = mp.get_context("spawn")
        cpus, phys, self.model = host_cpus()
        self.sets = {"logical": cpus[:16]}
        if len(phys) < len(cpus):
            self.sets["physical"] = phys[:16]
        self.pools = {}
        for name, cs in self.sets.items():
            barrier = self.ctx.Barrier(len(cs))
            q = self.ctx.Queue()
            for c in cs:
                q.put(c)
            self.pools[name] = (self.ctx.Pool(len(cs), initializer=_cpu_worker_init, initargs=(barrier, q)), len(cs))

    def run(self, name, kind, items):
        """Splits items into one job per worker; returns (seconds, summed result)."""
        pool, n = self.pools[name]
        jobs = [(kind, items[i::n]) for i in range(n)]
        res = pool.map(_cpu_worker_task, jobs, chunksize=1)
        return max(r[1] for r in res) - min(r[0] for r in res), sum(r[2] for r in res)

    def close(self):
        for pool, _ in self.pools.values():
            pool.terminate()


def cpu_baseline(pools):
    """The oracle, as it stands (fp64 NumPy, one process per core), on the GPU
    box's host cores, with all logical CPUs and with physical cores only (the
    faster is reported): decode attention of the whole 256-request batch (KV
    GB/s, the unit of the GPU figure), the last 64 query rows of every request
    of the 8-request prefill (causal TFLOP/s) and the 256-row mixed sampler
    batch (tokens/s)."""
    from workloads import config, draw_lengths
    C4, S4 = draw_lengths(config(4))
    ext_items = []
    for r in range(len(S4)):
        E = int(S4[r] - C4[r])
        ext_items += [(r, E - 64, E - 32), (r, E - 32, E)]
    runs = {}
    for name in pools.sets:
        d_s, d_bytes = pools.run(name, "decode", list(range(256)))
        e_s, e_flops = pools.run(name, "extend", ext_items)
        s_s, s_rows = pools.run(name, "sample", list(range(256)))
        runs[name] = {"cores": len(pools.sets[name]), "decode_s": round(d_s, 3),
                      "decode_kv_gbs": round(d_bytes / d_s / 1e9, 4), "extend_s": round(e_s, 3),
                      "extend_tflops": round(e_flops / e_s / 1e12, 6), "sample_s": round(s_s, 3),
                      "sampler_tokens_per_s": round(s_rows / s_s, 2)}
        log(f"cpu baseline ({name}, {len(pools.sets[name])} processes): decode {runs[name]['decode_kv_gbs']:.3f} GB/s, "
            f"extend {runs[name]['extend_tflops'] * 1e3:.3f} GFLOP/s, sampler {runs[name]['sampler_tokens_per_s']:.1f} tokens/s")
    best = max(runs, key=lambda n: runs[n]["decode_kv_gbs"])
    b = runs[best]
    return {"value": b["decode_kv_gbs"], "unit": "GB/s", "cores": b["cores"], "kind": "oracle",
            "sample": f"decode attention of all 256 requests of the decode batch ({b['decode_s']:.1f} s), plus "
                      f"the last 64 query rows of each of the 8 prefill requests ({b['extend_s']:.1f} s) and the "
                      f"256-row mixed sampler batch ({b['sample_s']:.1f} s); fp64 NumPy, one process per core, "
                      f"{best} cores (the faster of {', '.join(runs)})",
            "extend_tflops": b["extend_tflops"], "sampler_tokens_per_s": b["sampler_tokens_per_s"],
            "cpu_model": pools.model, "runs": runs}


if __name__ == "__main__":
    main()
