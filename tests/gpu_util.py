"""Helpers for the GPU parity tests (host side only)."""

from __future__ import annotations

import sys

import numpy as np
import torch

ATOL = 1e-3
RTOL = 1e-2


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash log says what ran."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_fp16_close(gpu: torch.Tensor, ref: np.ndarray, what: str = "out") -> None:
    """|gpu - oracle| <= 1e-3 + 1e-2 * |oracle| element by element."""
    g = host(gpu).astype(np.float64)
    r = np.asarray(ref).astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    err = np.abs(g - r)
    tol = ATOL + RTOL * np.abs(r)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)}: gpu {g[tuple(i)]!r} oracle {r[tuple(i)]!r}")


def assert_equal(gpu: torch.Tensor, ref: np.ndarray, what: str) -> None:
    g = host(gpu)
    r = np.asarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if not np.array_equal(g, r):
        bad = np.argwhere(g != r)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {g.size} differ; first at {i}: gpu {g[i]!r} oracle {r[i]!r}")
