"""Helpers for the GPU tests: device placement and a flushed progress line that
names the case before each GPU step."""
import sys

import numpy as np
import torch


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def dev(X: np.ndarray, ld: int = None) -> torch.Tensor:
    """Feature-major float32 [d, n] on cuda:0; with ``ld`` > n the columns sit
    in a wider buffer (leading dimension ld)."""
    X = np.ascontiguousarray(X, np.float32)
    if ld is None or ld == X.shape[1]:
        return torch.from_numpy(X).to("cuda:0")
    buf = np.full((X.shape[0], ld), np.nan, np.float32)
    buf[:, : X.shape[1]] = X
    t = torch.from_numpy(buf).to("cuda:0")
    return t[:, : X.shape[1]]


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()
