"""Helpers for the GPU parity tests (imported by tests/test_gpu_*.py)."""
import sys

import numpy as np
import pytest
import torch

from verify_pass_rejection_amd import native as nat

BF16_ATOL = 2e-2      # max-abs tolerance for bf16 K/V attention outputs
F32_ATOL = 1e-4       # max-abs tolerance for fp32 attention outputs


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    nat.load()                       # fails loudly if the library is missing
    return torch.device("cuda:0")


def say(*msg):
    print("[gpu]", *msg, flush=True)
    sys.stdout.flush()


def f64(t):
    """Exact widening of a (bf16 / fp32) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def i64(t):
    return t.detach().to("cpu").to(torch.int64).numpy()
