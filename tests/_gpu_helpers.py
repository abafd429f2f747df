"""Shared helpers for the GPU parity tests (not collected by pytest)."""

import sys

import numpy as np
import torch

# Tolerances stated for bf16 inputs with fp32 accumulation: max-abs error of
# the output and of the natural-log LSE against the fp64 oracle.
OUT_TOL = 1e-2
LSE_TOL = 1e-3


def announce(*parts):
    """Name the case before a GPU step, flushed, so a crash still says which."""
    print("[gpu-case]", *parts, file=sys.stderr, flush=True)


def dev(x, dtype=None):
    t = x if isinstance(x, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def host(x):
    return x.detach().to("cpu", torch.float64).numpy()


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at |x| (8 significant bits): the
    rounding error that storing an exact result as bf16 may add by itself."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def assert_close(name, got, ref, tol, bf16_output=False):
    """max |got - ref| <= tol elementwise (fp64 oracle as ref). For a bf16
    output tensor the bound is tol plus the output's own storage rounding
    (half a bf16 ulp of the exact value), which no bf16-output kernel avoids."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    fin_g, fin_r = np.isfinite(got), np.isfinite(ref)
    if not np.array_equal(fin_g, fin_r):
        raise AssertionError(f"{name}: finite mask differs at {np.argwhere(fin_g != fin_r)[:5].tolist()}")
    assert np.array_equal(got[~fin_r], ref[~fin_r]), f"{name}: infinities differ"
    if not fin_r.any():
        return 0.0
    diff = np.zeros_like(ref)
    diff[fin_r] = np.abs(got[fin_r] - ref[fin_r])
    err = float(diff.max())
    allowed = tol + (bf16_half_ulp(np.where(fin_r, ref, 0.0)) if bf16_output else 0.0)
    bad = diff > allowed
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: error {diff[i]:.3e} > allowed {allowed[i] if np.ndim(allowed) else allowed:.3e} "
                             f"at {i} (got {got[i]!r}, ref {ref[i]!r}); max-abs {err:.3e}, "
                             f"{int(bad.sum())} of {bad.size} elements over")
    print(f"[parity] {name}: max-abs {err:.3e} (tol {tol:.0e}{' + bf16 half-ulp' if bf16_output else ''})",
          flush=True)
    return err


def guarded_empty(shape, dtype, guard=4096, fill=None):
    """A tensor view with `guard` poisoned elements after it, to catch overruns."""
    n = int(np.prod(shape))
    buf = torch.empty(n + guard, dtype=dtype, device="cuda")
    if fill is None:
        fill = float("nan")
    buf.fill_(fill)
    return buf[:n].view(shape), buf[n:]


def guard_intact(guard, fill=None):
    g = guard.float().cpu()
    if fill is None:
        return bool(torch.isnan(g).all())
    return bool((g == fill).all())
