"""Shared pieces of the GPU parity tests (imported only by tests marked gpu)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    """Name the case on stdout before a GPU step (flushed, so a crash still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u16(bits: np.ndarray, act: str):
    """uint16 bit patterns -> device tensor of the 16-bit float type."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.float16 if act == "f16" else torch.bfloat16)


def host_f32(t) -> np.ndarray:
    return t.float().cpu().numpy()


def act_round(a: np.ndarray, act: str) -> np.ndarray:
    """float64 -> nearest value of the activation type, as float32 (via torch's RNE casts)."""
    tt = torch.from_numpy(np.asarray(a, dtype=np.float32))
    return tt.to(torch.float16 if act == "f16" else torch.bfloat16).float().numpy()


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)
