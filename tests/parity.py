"""Helpers shared by the GPU parity tests: tolerance checks and the oracle
evaluated on a sample of rows of a large problem."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# |gpu - ref| <= ATOL + RTOL * |ref| against the unrounded fp64 oracle
TOL_F32 = (1e-4, 1e-4)
TOL_BF16 = (2e-3, 2e-3)


# a bf16-rounded output adds up to half a bf16 ulp (<= 2^-8 |ref|) on top
BF16_HALF_ULP = 2.0 ** -8


def tol_for(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def tol_out_bf16(tol):
    """The tolerance widened by the rounding of a bf16 output."""
    return (tol[0], tol[1] + BF16_HALF_ULP)


def check_close(got, ref, tol, what="y"):
    """Elementwise |got - ref| <= atol + rtol |ref|; reports the worst index."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    atol, rtol = tol
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)  # NaN counts as bad unless both are NaN
    both_nan = np.isnan(got) & np.isnan(ref)
    bad &= ~both_nan
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), got.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
            f"(atol={atol}, rtol={rtol}); worst at {idx}: got {got[idx]!r}, ref {ref[idx]!r}; "
            f"max abs err {float(np.nanmax(err)):.3e}")
    return float(np.nanmax(err)) if err.size else 0.0


def host(t):
    return None if t is None else t.detach().to("cpu")


def oracle_m1_rows(inp, rows, softplus=True):
    """fp64 oracle for rows [(b, d), ...] of a Mamba-1 problem whose inputs
    live on any device; returns (y [R, L], last [R, N])."""
    ys, lasts = [], []
    by_b = {}
    for i, (b, d) in enumerate(rows):
        by_b.setdefault(b, []).append((i, d))
    out_y = [None] * len(rows)
    out_l = [None] * len(rows)
    for b, lst in by_b.items():
        ds = torch.tensor([d for _, d in lst], dtype=torch.long)
        sel = lambda t: None if t is None else host(t[b:b + 1].index_select(1, ds.to(t.device)))
        vec = lambda t: None if t is None else host(t.index_select(0, ds.to(t.device)))
        y, last = oracle.m1(sel(inp["u"]), sel(inp["delta"]), vec(inp["A"]), host(inp["B"][b:b + 1]),
                            host(inp["C"][b:b + 1]), vec(inp.get("D")), sel(inp.get("z")),
                            vec(inp.get("delta_bias")), softplus=softplus)
        for j, (i, _) in enumerate(lst):
            out_y[i] = y[0, j]
            out_l[i] = last[0, j]
    del ys, lasts
    return np.stack(out_y), np.stack(out_l)


def oracle_m2_units(inp, units, softplus=True):
    """fp64 oracle for (b, h) pairs of a Mamba-2 problem: returns
    y [U, L, P] and last [U, P, N]."""
    ys, lasts = [], []
    for b, h in units:
        sl = slice(b, b + 1)
        hs = slice(h, h + 1)
        G = inp["B"].shape[2]
        H = inp["x"].shape[2]
        g = h // (H // G)
        v = lambda t: None if t is None else host(t[hs])
        y, last = oracle.m2(host(inp["x"][sl, :, hs]), host(inp["dt"][sl, :, hs]), v(inp["A"]),
                            host(inp["B"][sl, :, g:g + 1]), host(inp["C"][sl, :, g:g + 1]), v(inp.get("D")),
                            None if inp.get("z") is None else host(inp["z"][sl, :, hs]), v(inp.get("dt_bias")),
                            softplus=softplus)
        ys.append(y[0, :, 0])
        lasts.append(last[0, 0])
    return np.stack(ys), np.stack(lasts)
