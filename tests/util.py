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


def ulp_diff(got, want) -> np.ndarray:
    """Distance in fp32 units in the last place (same-sign finite values)."""
    g = np.asarray(got, np.float32).view(np.int32).astype(np.int64)
    w = np.asarray(want, np.float32).view(np.int32).astype(np.int64)
    g = np.where(g < 0, np.int64(-2**31) - g, g)
    w = np.where(w < 0, np.int64(-2**31) - w, w)
    return np.abs(g - w)


def assert_same_fp32(got, want, min_equal=0.999, max_ulp=2):
    """The GPU carries its sums in fp64 and rounds once, so its fp32 values
    should equal the oracle's except for rare rounding-midpoint cases."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    eq = float(np.mean(got == want)) if want.size else 1.0
    worst = int(ulp_diff(got, want).max()) if want.size else 0
    assert eq >= min_equal and worst <= max_ulp, f"equal fraction {eq:.6f}, worst {worst} ulp"
    return eq


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
