"""Helpers shared by the tests: tolerance metric and host/device moves."""
import numpy as np

LAYER_TOL = 1e-3     # max relative error of fp32 layer outputs
LOGIT_TOL = 1e-2     # max absolute error of logits


def rel_err(got, want) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o)): elementwise relative error with
    an RMS floor, so that entries near zero do not dominate."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if want.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(want ** 2))
    den = np.maximum(np.abs(want), rms if rms > 0 else 1e-30)
    return float(np.max(np.abs(got - want) / den))


def dev(a, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed so a fault still shows it)."""
    print(msg, flush=True)
