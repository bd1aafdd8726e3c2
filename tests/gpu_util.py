"""Helpers for the GPU parity tests: host <-> device copies of the seeded
inputs and outputs.  No arithmetic of the method lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

FMT_NAME = {oracle.E4M3: "e4m3", oracle.E5M2: "e5m2"}
FMAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}


def say(*a):
    """Name the case before each GPU step, flushed, so a fault names it."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_u8(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def dev_input(x: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) or float32 -> device tensor of that dtype."""
    if x.dtype == np.uint16:
        return dev_bf16(x)
    return dev_f32(x)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def crafted_history(window_amax: float, length: int = 16, device="cuda") -> torch.Tensor:
    """A history whose window max is `window_amax` (one entry): the next
    delayed call then scales by fmax / window_amax."""
    w = torch.zeros(32, dtype=torch.int32)
    f = w.view(torch.float32)
    f[0] = window_amax
    w[16] = length     # len
    w[17] = 1          # pos
    w[18] = 1          # count
    return w.to(device)


def random_codes(rng, shape, fmt):
    t = oracle.decode_table(fmt)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)
    return rng.choice(finite, size=shape)
