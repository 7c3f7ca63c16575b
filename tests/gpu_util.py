"""Shared helpers of the GPU parity tests: device copies of synthgen inputs and
error metrics.  Expected values always come from the fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

import synthgen as sg

# Tolerances.  End to end: max abs error 1e-4 for fp32 tensors, 2e-2 with bf16
# inputs and fp32 accumulation.  Per branch, relative to the branch's largest
# magnitude (the compressed branch is ~0.01 in size, so the absolute bound alone
# could not see it break): 1e-5 fp32, 1e-2 bf16.
ABS_TOL = {"f32": 1e-4, "bf16": 2e-2}
REL_TOL = {"f32": 1e-5, "bf16": 1e-2}
# log-sum-exp of the scaled logits.  With bf16 operands each probability is
# rounded to bf16 (relative error <= 2^-9) before it enters both the PV
# product and the normaliser, so the normaliser, and hence its log, may be off
# by up to 2^-9; the bound allows twice that.
LSE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}


def tdtype(w: sg.Workload) -> torch.dtype:
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def dev(x, dtype=None):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def problem(pk, w: sg.Workload, **kw):
    kw.setdefault("summary_mode", w.summary_mode)
    return pk.make_problem(w.grid, w.n_q_heads, w.n_kv_heads, w.window, w.block, tdtype(w),
                           w.rope_pairs, w.rope_base, **kw)


def device_inputs(inp: sg.Inputs) -> dict:
    dt = tdtype(inp.workload)
    return dict(q=dev(inp.q, dt), k_loc=dev(inp.k_loc, dt), v_loc=dev(inp.v_loc, dt),
                k_cmp=dev(inp.k_cmp, dt), v_cmp=dev(inp.v_cmp, dt), a=dev(inp.a),
                coords=dev(inp.coords), cell_to_pos=dev(inp.cell_to_pos), gate=dev(inp.gate))


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def round_like(x: np.ndarray, w: sg.Workload) -> np.ndarray:
    """Oracle values rounded to the workload's storage dtype (as the GPU stores them)."""
    x32 = np.asarray(x, dtype=np.float32)
    return (sg.round_to_bf16(x32) if w.dtype == "bf16" else x32).astype(np.float64)


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def max_rel(got, ref) -> float:
    ref = np.asarray(ref, np.float64)
    return max_abs(got, ref) / float(np.abs(ref).max())
