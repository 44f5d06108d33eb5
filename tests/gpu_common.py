"""Shared set-up for the GPU parity tests."""

import sys

import pytest
import torch

import paged_kv_cache_heads_amd as pa


def announce(msg: str) -> None:
    """Name the case before any GPU work, so a crash can be traced to it."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="session")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa._lib.load()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")
