"""Shared helpers for the GPU parity tests (not collected by pytest)."""

import os
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


# Above this magnitude half a bf16 ulp (2**-6) exceeds OUT_TOL by itself, so a
# bf16 output cannot hold the flat bound there whatever the kernel does; below
# it the rounding of the stored result takes at most 2**-7 and the flat bound
# stands.
BF16_FLAT_LIMIT = 4.0

# Every assert_close result of the session: the plain max-abs error, the same
# over the elements the flat bound covers, and the test that produced it. The
# session writes them out as JSON lines when ATTN_PARITY_RECORD names a file.
RECORDS = []


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at |x| (8 significant bits): the
    rounding error that storing an exact result as bf16 may add by itself."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def assert_close(name, got, ref, tol, bf16_output=False, few_keys=False):
    """max |got - ref| <= tol elementwise against the fp64 oracle (ref). For a
    bf16 output the bound stays flat wherever |ref| < BF16_FLAT_LIMIT; only
    elements of larger magnitude, where the output's own storage rounding (half
    a bf16 ulp of the exact value) passes tol by itself, get that rounding added.

    few_keys: edge cases whose rows see only a handful of keys (documents of a
    few tokens, the first rows under a causal mask, contexts of 1-33 tokens).
    Their outputs reach 2.5-4.5 (a weighted mean of a few N(0, 1) values), where
    storing the result as bf16 takes up to 2**-7 and rounding each probability
    to bf16 for the P V product adds up to 2**-9 of sum_j w_j |v_j| on top, so
    such tests add half a bf16 ulp of the exact value at every magnitude."""
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
    aref = np.abs(np.where(fin_r, ref, 0.0))
    flat = aref < (0.0 if few_keys else BF16_FLAT_LIMIT) if bf16_output else np.ones(ref.shape, dtype=bool)
    err_flat = float(diff[flat].max()) if flat.any() else 0.0
    allowed = tol + (np.where(flat, 0.0, bf16_half_ulp(aref)) if bf16_output else 0.0)
    bad = diff > allowed
    RECORDS.append({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "name": name,
                    "max_abs": err, "max_abs_flat_region": err_flat, "tol": tol, "elements": int(ref.size),
                    "over_tol": int(bad.sum()), "max_abs_ref": float(aref.max()), "few_keys": bool(few_keys),
                    "max_abs_below_flat_limit": float(diff[aref < BF16_FLAT_LIMIT].max()) if (aref < BF16_FLAT_LIMIT).any() else 0.0})
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: error {diff[i]:.3e} > allowed {allowed[i] if np.ndim(allowed) else allowed:.3e} "
                             f"at {i} (got {got[i]!r}, ref {ref[i]!r}); max-abs {err:.3e}, "
                             f"{int(bad.sum())} of {bad.size} elements over")
    rule = ""
    if bf16_output:
        rule = ", + bf16 half-ulp" + ("" if few_keys else f" where |ref| >= {BF16_FLAT_LIMIT:g}")
    print(f"[parity] {name}: max-abs {err:.3e} (tol {tol:.0e}{rule})", flush=True)
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
