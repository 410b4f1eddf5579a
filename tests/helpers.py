"""Shared test utilities: device transfer of seeded inputs and the agreement metric."""

from __future__ import annotations

import numpy as np
import torch

import workloads as W

# Agreement bars: max|H - H_ref| / mean(diag(H_ref)).  The float64 oracle is
# the reference; the bars are the ones the target states for bf16 and float32
# inputs (the pages measure 2.8e-5 for bf16 in / fp32 out at 32K tokens per
# batch and 4.7e-6 for a float32 GEMM).
TOL = {W.BF16: 5e-5, W.F32: 1e-5}


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == W.F16:
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def torch_dtype(dtype: str):
    return {W.BF16: torch.bfloat16, W.F32: torch.float32, W.F16: torch.float16}[dtype]


def agreement(H: np.ndarray, H_ref: np.ndarray) -> float:
    md = float(np.mean(np.diag(H_ref)))
    return float(np.max(np.abs(H.astype(np.float64) - H_ref))) / md


def block_agreement(B: np.ndarray, B_ref: np.ndarray) -> float:
    """Max over blocks of max|B_b - B_ref_b| / mean(diag(B_ref_b)); all-zero blocks must be exact."""
    worst = 0.0
    for b in range(B_ref.shape[0]):
        md = float(np.mean(np.diag(B_ref[b])))
        diff = float(np.max(np.abs(B[b].astype(np.float64) - B_ref[b])))
        if md == 0.0:
            assert diff == 0.0
            continue
        worst = max(worst, diff / md)
    return worst


# Relative distance from a half-integer below which w / step is a rounding tie: both neighbour
# codes are correct there (the float64 additions of the propagated errors come in another order
# on the GPU, about 1e-16 relative, which can tip such a tie either way).
TIE_TOL = 1e-12


def quantize_against_gpu_ties(Wr, U, group, gpu_codes, **kw):
    """The oracle's block quantize with the GPU's choice taken at rounding ties.

    The oracle reports every tie and its two neighbour codes; this checker takes
    the GPU's code there when it is one of them (and the oracle's own choice
    otherwise, which then fails the code comparison).  Returns the oracle's
    ``(Q, codes, scales, loss)`` and ``(ties, taken)``: how many tie positions
    there were and at how many the GPU's code differed from the oracle's own.
    """
    import oracle as O
    count = {"ties": 0, "taken": 0}
    gpu_codes = np.asarray(gpu_codes)

    def pick(i, rows, lo, hi, dflt):
        g = gpu_codes[rows, i].astype(np.float64)
        ok = (g == lo) | (g == hi)
        out = np.where(ok, g, dflt)
        count["ties"] += int(rows.size)
        count["taken"] += int(np.sum(out != dflt))
        return out

    res = O.gptq_quantize(Wr, U, group_size=group, tie_tol=TIE_TOL, tie_break=pick, **kw)
    assert count["taken"] <= count["ties"]
    return res, (count["ties"], count["taken"])
