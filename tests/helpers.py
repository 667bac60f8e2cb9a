"""Shared test helpers (comparison metrics, conversions)."""
import numpy as np
import torch

TOL = 2e-3          # max-rel-err (normwise, infinity norm) on fp32 outputs


def f64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_err(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i| (0 when both are zero)."""
    got = f64(got)
    ref = f64(ref)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def bits_to_bool(bits, n):
    b = bits.detach().cpu().numpy().astype(np.uint64)
    b = np.atleast_2d(b)
    out = np.zeros((b.shape[0], b.shape[1] * 64), dtype=bool)
    for k in range(64):
        out[:, k::64] = ((b >> np.uint64(k)) & np.uint64(1)).astype(bool)
    return out[:, :n]


def announce(name):
    print(f"[case] {name}", flush=True)
