"""Shared helpers for the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

import oracle
from int4_weight_streaming_q4_amd import inputs

DEV = "cuda"


def u16(t: torch.Tensor) -> np.ndarray:
    """binary16 bit patterns held in an int16 tensor -> numpy uint16."""
    return inputs.to_numpy_u16(t)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy()


def assert_within(y_gpu, y_ref, mag, what="", rel=2e-3, abs_=1e-6):
    """The per-output acceptance rule |y - y_ref| <= rel * mag + abs."""
    y = np.asarray(y_gpu, np.float64)
    ok = oracle.within_bound(y, y_ref, mag, rel, abs_)
    if not ok.all():
        bad = np.flatnonzero(~ok)[:8]
        raise AssertionError(
            f"{what}: {int((~ok).sum())} of {ok.size} outputs outside the bound; "
            f"first {bad.tolist()}: gpu={y[bad]} ref={np.asarray(y_ref)[bad]} "
            f"mag={np.asarray(mag)[bad]}")


def rel_err_stats(y_gpu, y_ref, mag):
    y = np.asarray(y_gpu, np.float64)
    r = np.abs(y - y_ref) / (np.asarray(mag) + 1e-30)
    return float(r.max()), float(np.median(r))


def sync():
    torch.cuda.synchronize()
