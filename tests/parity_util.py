"""Helpers shared by the GPU parity tests: host copies, the row-max relative
error metric, lazy per-expert host views for the oracle."""
import threading

import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16, torch.float32, torch.float64):
        return t.detach().float().cpu().numpy()
    return t.detach().cpu().numpy()


def row_rel_err(y, ref) -> float:
    """max over rows of max|y - ref| / max|ref| (row-max-normalized)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(y - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def mat_rel_err(y, ref) -> float:
    """max|y - ref| / max|ref| over a whole matrix. Used for weight gradients:
    each entry is a sum over tokens whose terms cancel, so a row of one can be
    small next to its terms and the row-normalized metric would measure the
    cancellation rather than the arithmetic."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-30))


class LazyHost:
    """Indexable host view of a device tensor [E, ...]: expert e is copied to
    the host (as fp32) when the oracle asks for it, and not kept. With a
    label, every 32nd copy prints a progress line."""

    def __init__(self, t: torch.Tensor, label: str | None = None):
        self.t = t
        self.label = label
        self.n = 0
        self.lock = threading.Lock()

    def __getitem__(self, e):
        if self.label:
            with self.lock:
                self.n += 1
                if self.n % 32 == 0:
                    print(f"    oracle: {self.n} {self.label} copies", flush=True)
        return host(self.t[int(e)])


def route_args(wl):
    return dict(top_k=wl.K, n_groups=wl.G, topk_groups=wl.M, group_topn=wl.topn)
