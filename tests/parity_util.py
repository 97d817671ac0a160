"""Helpers shared by the GPU parity tests: host/device copies of the stored inputs
and the comparison against the fp64 oracle with the stated bounds.

Bounds (stated for the fused forward): bf16/fp16 inputs — max |dO| <= 1e-2,
mean |dO| <= 1e-3, max |dL| <= 1e-3; fp32 inputs — max |dO| <= 1e-4 (and
|dL| <= 1e-3).  dO is the GPU output widened to fp64 minus the oracle's fp64 O.
Where |O_ref| >= 4 an element passes the max bound if it is one of the two bf16
neighbours of O_ref (faithful rounding): there one bf16 step is 2^-5 or more, so
correct rounding of the output alone can miss O_ref by more than 1e-2.  Below 4 the
literal bound holds for every element.
"""
import json
import os
import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def record(w, **figures):
    """Append one JSON line of parity figures to $FA_PARITY_LOG (when set)."""
    path = os.environ.get("FA_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    row = {"test": test, "workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
           "dtype": w.dtype, "causal": bool(w.causal), "sigma_qk": w.sigma_q}
    row.update({k: (float(v) if isinstance(v, (float, np.floating)) else v)
                for k, v in figures.items()})
    with open(path, "a") as f:
        f.write(json.dumps(row) + "\n")


def bf16_neighbours_ok(o_gpu64, o_ref):
    """True where o_gpu is the bf16 value just below or just above o_ref in magnitude."""
    e = np.frexp(np.abs(o_ref))[1].astype(np.int32)    # |o_ref| in [2^(e-1), 2^e)
    quantum = np.ldexp(1.0, e - 1 - 7)                  # bf16 spacing there
    lo = np.trunc(o_ref / quantum) * quantum
    hi = lo + np.sign(o_ref) * quantum
    return (o_gpu64 == lo) | (o_gpu64 == hi)


def compare(w, o_gpu_np, lse_gpu, sel_bh, sel_row, o64, l64):
    d = w.d
    o_sel = oracle.widen(o_gpu_np.reshape(-1, d)[sel_bh * w.Nq + sel_row], w.dtype)
    l_sel = lse_gpu.reshape(-1)[sel_bh * w.Nq + sel_row].astype(np.float64)
    assert np.isfinite(o_sel).all() and np.isfinite(l_sel).all()
    err = np.abs(o_sel - o64)
    derr_l = np.abs(l_sel - l64)
    if w.dtype == "f32":
        say(f"  {w.name}: max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} "
            f"max|dL|={derr_l.max():.3e}")
        record(w, rows=len(sel_row), max_do=err.max(), mean_do=err.mean(), max_dl=derr_l.max())
        assert err.max() <= 1e-4
        assert derr_l.max() <= 1e-3
        return
    big = np.abs(o64) >= 4.0
    over = err > 1e-2
    faithful = over & big & (bf16_neighbours_ok(o_sel, o64) if w.dtype == "bf16" else False)
    band = (np.abs(o64) >= 2.0) & ~big
    say(f"  {w.name}: max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} "
        f"max|dL|={derr_l.max():.3e} faithful-rounding exceptions={int(faithful.sum())}")
    record(w, rows=len(sel_row), max_do=err.max(), mean_do=err.mean(), max_dl=derr_l.max(),
           over_lt2=int((over & (np.abs(o64) < 2.0)).sum()), over_2_4=int((over & band).sum()),
           over_ge4=int((over & big).sum()), faithful_ge4=int(faithful.sum()),
           max_abs_oref=float(np.abs(o64).max()))
    assert not (over & ~faithful).any(), f"max|dO| {err[over & ~faithful].max():.3e} > 1e-2"
    assert err.mean() <= 1e-3
    assert derr_l.max() <= 1e-3


