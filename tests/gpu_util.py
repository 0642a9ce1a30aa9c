"""Helpers for the GPU tests: host <-> device copies of the synthetic arrays."""

from __future__ import annotations

import os

import numpy as np
import torch

ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def to_dev(a: np.ndarray, device="cuda:0") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def say(*args) -> None:
    print(*args, flush=True)
