"""Helpers for the GPU parity tests: tolerances and comparisons."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances of the method's statement: bf16 K/V with fp32 accumulation
# max abs <= 2e-2 and max rel <= 1e-2; fp32 inputs <= 1e-5.  "rel" is taken per
# output row (one query head of one sequence): ||gpu - ref||_inf / ||ref||_inf,
# because an element-wise relative error is undefined where the reference
# crosses zero.
TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-5, 1e-5)}


def errors(gpu: torch.Tensor, ref: np.ndarray):
    g = gpu.detach().float().cpu().double().numpy().reshape(-1, ref.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    diff = np.abs(g - r)
    abs_err = float(diff.max()) if diff.size else 0.0
    row_ref = np.abs(r).max(axis=1)
    row_err = diff.max(axis=1)
    nz = row_ref > 0
    rel = float((row_err[nz] / row_ref[nz]).max()) if nz.any() else 0.0
    # rows whose reference is exactly zero must be exactly zero
    if (~nz).any():
        abs_zero_rows = float(row_err[~nz].max())
        rel = max(rel, abs_zero_rows * 1e30 if abs_zero_rows > 0 else 0.0)
    return abs_err, rel


def assert_parity(gpu: torch.Tensor, ref: np.ndarray, dtype, what: str):
    assert torch.isfinite(gpu.float()).all(), f"{what}: non-finite output"
    abs_tol, rel_tol = TOL[dtype]
    abs_err, rel = errors(gpu, ref)
    print(f"[parity] {what}: max_abs={abs_err:.3e} max_row_rel={rel:.3e}", flush=True)
    assert abs_err <= abs_tol, f"{what}: max abs error {abs_err} > {abs_tol}"
    assert rel <= rel_tol, f"{what}: max row-relative error {rel} > {rel_tol}"


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()
