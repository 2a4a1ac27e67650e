"""Shared pytest configuration: markers and repo-root import path."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # GPU runs start the oracle's worker pool now, before any test initialises
    # the GPU in this process (the full-size parity tests use it)
    expr = (config.option.markexpr or "").replace(" ", "")
    if "gpu" in expr and "notgpu" not in expr:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import oracle_pool
        oracle_pool.start()
