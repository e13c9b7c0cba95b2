"""Helpers shared by the GPU parity tests (inputs to the device, tolerances)."""

import sys

import numpy as np
import torch

from conftest import rel_frobenius  # noqa: F401  (re-exported)

# Tolerances fixed for the build: bf16 paths rel. Frobenius <= 5e-3, fp32
# paths <= 1e-5, cross-entropy loss absolute <= 1e-3; masks and permutation
# indices bit-exact.
TOL = {"bf16": 5e-3, "f32": 1e-5}
XENT_ABS = 1e-3


def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    return torch.device("cuda:0")


def cu(t):
    return t.to(dev()).contiguous()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def sync():
    torch.cuda.synchronize()


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def randn(gen_seed, shape, dtype, std=1.0):
    rng = np.random.default_rng(gen_seed)
    a = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return torch.from_numpy(a).to(tdtype(dtype))


def mask_bits(n):
    """Device buffer for n dropout keep flags saved as bits."""
    return torch.empty((n + 7) // 8, dtype=torch.uint8, device="cuda")


def unpack_bits(t, n):
    """Keep flags (bool [n]) from a bit buffer: bit i & 7 of byte i >> 3."""
    return np.unpackbits(t.cpu().numpy(), bitorder="little")[:n].astype(bool)
