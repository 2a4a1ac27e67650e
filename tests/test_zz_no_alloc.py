"""The decode entry point that allocates nothing
(pkv_paged_attention_decode_noalloc), called through the C ABI: on two calls
in a row -- the second with a smaller batch -- its output equals
pkv_paged_attention_decode's bit for bit (same kernels, same split plan) and
meets the attention bounds against the oracle; a size beyond its scratch is
refused before anything runs."""

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits
from gpu_util import check_attention, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
pkv = pytest.importorskip("paged_kv_attention_scatter_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.read_faults()  # clear


def _batch(seed, lens, slots_extra=100):
    rng = np.random.default_rng(seed)
    S = np.asarray(lens, np.int32)
    bs, total = len(S), int(S.sum())
    n_slots = total + slots_extra
    perm = rng.permutation(n_slots)
    width = (int(S.max()) + 31) // 32 * 32
    table = np.full((bs, width), n_slots - 1, np.int32)
    off = 0
    for r in range(bs):
        table[r, :S[r]] = perm[off:off + S[r]]
        off += S[r]
    kv = f32_to_bf16_bits(rng.standard_normal((2, n_slots, 8, 128), dtype=np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((bs, 16, 128), dtype=np.float32))
    return S, table, kv, q


def test_noalloc_decode_matches_workspace_decode_twice():
    rng = np.random.default_rng(11)
    first = rng.integers(1, 3000, 96)
    second = rng.integers(1, 700, 9)
    for call, lens in enumerate((first, second)):
        S, table, kv, q = _batch(100 + call, lens)
        print(f"noalloc decode call {call}: bs={len(S)} sum S={int(S.sum())}", flush=True)
        dk, dv, dq = to_dev(kv[0], "bf16"), to_dev(kv[1], "bf16"), to_dev(q, "bf16")
        dt, dC, dS = to_dev(table), to_dev(S - 1), to_dev(S)
        out_ws = pkv.paged_attention_decode(dq, dk, dv, dt, dC, dS, max_total_kv=int(S.sum()))
        out_na = torch.full_like(out_ws, float("nan"))
        pkv.paged_attention_decode_noalloc(dq, dk, dv, dt, dC, dS, max_total_kv=int(S.sum()), out=out_na)
        torch.cuda.synchronize()
        a, b = to_host(out_ws), to_host(out_na)
        assert np.array_equal(a, b), f"call {call}: noalloc output differs from the workspace entry point"
        ref = oracle.attention_decode(q, kv[0], kv[1], table, S - 1, S, "bf16")
        mx, rel = check_attention(b, ref, "bf16", f"noalloc call {call}")
        print(f"  bit-equal to the workspace call; max|d|={mx:.3e} relL2={rel:.3e}", flush=True)
        assert pkv.read_faults() == 0


def test_noalloc_decode_refuses_oversized_call():
    bs = 4000                                   # partials of 4000 + 1024 slots exceed the scratch
    assert pkv.decode_workspace_size(bs, 16, 1 << 30) > pkv._lib.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((bs, 16, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((64, 8, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((bs, 32), dtype=torch.int32, device="cuda")
    lens = torch.ones(bs, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_noalloc(q, pool, pool, table, lens - 1, lens, max_total_kv=1 << 30, out=out)
    assert e.value.status == -6 and "scratch" in str(e.value)
