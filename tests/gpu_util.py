"""Helpers shared by the GPU parity tests: host<->device marshalling only."""

from __future__ import annotations

import os
import sys

import numpy as np
import torch


def log(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8_dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def i64_dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(device)


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def first_mismatch(got: np.ndarray, want: np.ndarray, row: int | None = None) -> str:
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    if bad.size == 0:
        return "identical"
    i = int(bad[0])
    where = f"byte {i}" if row is None else f"row {i // row} byte {i % row}"
    return f"{bad.size} bytes differ; first at {where}: got {got.reshape(-1)[i]:#x} want {want.reshape(-1)[i]:#x}"
