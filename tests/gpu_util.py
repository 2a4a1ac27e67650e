"""Helpers shared by the GPU parity tests: host <-> device transfer of the
generator's arrays and the acceptance bounds."""

import numpy as np

import oracle

# Attention acceptance bounds (fp32: max-abs 1e-5; bf16: max-abs 2e-2 AND
# relative L2 1e-2 over the output tensor).
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2


def torch_mod():
    import torch
    return torch


def to_dev(x: np.ndarray, dtype: str | None = None, device="cuda"):
    """numpy -> GPU tensor; dtype "bf16" means x holds bf16 bit patterns."""
    torch = torch_mod()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_host(t):
    """GPU tensor -> numpy (bf16 as uint16 bit patterns)."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_attention(got, ref: np.ndarray, dtype: str, what: str = ""):
    """got: kernel output (numpy, kernel dtype); ref: fp64 oracle output.
    Returns (max_abs, rel_l2)."""
    g = oracle.widen(got, dtype)
    assert np.all(np.isfinite(g)), f"{what}: non-finite kernel output"
    d = g - ref
    max_abs = float(np.max(np.abs(d)))
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: max|d| {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max|d| {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{what}: rel L2 {rel:.3e} > {BF16_REL_L2}"
    return max_abs, rel
