"""Shared helpers of the GPU parity tests: moving seeded cases to the device,
running the library, and the acceptance check against the fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

import oracle

# Acceptance bar.  fp32 inputs: max abs error <= 1e-5.  16-bit inputs: the
# (atol, rtol) = (2e-3, 1e-2) pair applied per element as |err| <= atol + rtol*|ref|
# (a bf16 output above 0.5 in magnitude cannot be stored within 2e-3 of the exact
# value: half a bf16 ulp is 2^-9 |o|), and per output row (one query head of one
# token) max |err| / max |ref| <= 1e-2.
TOL_F32_ABS = 1e-5
TOL_16_ABS = 2e-3
TOL_16_REL = 1e-2
TOL_16_ROW_REL = 1e-2
# Tighter check of the arithmetic: outputs are the fp32 result rounded to the
# 16-bit type, so they may sit at most half an ulp of that type (plus the fp32
# accumulation error) from the exact value.
ULP_SLACK = 0.5
FP32_REL = 3e-5
# The chunked-prefill kernel rounds its softmax weights to the 16-bit type before the
# P.V product (and sums the rounded weights), so an output is a convex combination of
# V rows under weights w'_i = w_i (1 + e_i) / sum_j w_j (1 + e_j), |e_i| <= u (unit
# roundoff of the type).  Then |o' - o| <= u sum_i w_i |v_i - o| / (1 - u) <= 2 u max|v| / (1 - u):
# its half-ulp check takes that term on top.
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def ulp16(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit type at |ref| (normal range; subnormal floor)."""
    mant = 7 if dtype == "bf16" else 10
    floor = 2.0 ** -133 if dtype == "bf16" else 2.0 ** -24
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-300)))
    return np.maximum(2.0 ** (e - mant), floor)


def dev(x, device="cuda"):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(device).contiguous()


def check_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "", weights_vmax: float = None) -> dict:
    """Assert the acceptance bar and the half-ulp check; returns error statistics.
    weights_vmax: for outputs of the chunked-prefill kernel (weights rounded to the
    16-bit type), the largest |V| element the rows attend to; the half-ulp check then
    allows the rounding of the weights on top (see UNIT_ROUNDOFF)."""
    g = gpu.detach().to("cpu").to(torch.float64).numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    stats = {"max_abs": float(err.max()) if err.size else 0.0}
    if dtype == "f32":
        assert stats["max_abs"] <= TOL_F32_ABS, f"{what}: max abs err {stats['max_abs']:.3e}"
        return stats
    bound = TOL_16_ABS + TOL_16_REL * np.abs(ref)
    worst = float((err / bound).max()) if err.size else 0.0
    stats["tol_used"] = worst
    rows_ref = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    rows_err = err.reshape(-1, ref.shape[-1]).max(axis=1)
    live = rows_ref > 0
    rel = rows_err[live] / rows_ref[live]
    stats["max_row_rel"] = float(rel.max()) if rel.size else 0.0
    rowmax = np.repeat(rows_ref, ref.shape[-1]).reshape(ref.shape)
    weights = 0.0 if weights_vmax is None else 2 * UNIT_ROUNDOFF[dtype] * weights_vmax / (1 - UNIT_ROUNDOFF[dtype])
    ulps = err / (ulp16(ref, dtype) * ULP_SLACK + FP32_REL * rowmax + weights + 1e-30)
    stats["ulp_check"] = float(ulps.max()) if ulps.size else 0.0
    assert worst <= 1.0, f"{what}: error beyond atol+rtol*|ref| by factor {worst:.3f} (max abs {stats['max_abs']:.3e})"
    assert stats["max_row_rel"] <= TOL_16_ROW_REL, f"{what}: max row rel err {stats['max_row_rel']:.3e}"
    assert np.all(rows_err[~live] == 0), f"{what}: zero reference rows must give exact zeros"
    assert stats["ulp_check"] <= 1.0, f"{what}: beyond half an ulp plus fp32 error (x{stats['ulp_check']:.2f})"
    if weights_vmax is not None:
        stats["weights_bound"] = weights
    return stats


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view of a tensor's storage, for bit-exact comparisons."""
    t = t.detach().contiguous()
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def oracle_decode_case(case, query=None, pool=None, bt=None, ctx=None):
    pool = case.pool if pool is None else pool
    return oracle.decode(case.query if query is None else query, pool.key_cache, pool.value_cache,
                         case.block_tables if bt is None else bt, case.context_lens if ctx is None else ctx,
                         case.num_kv_heads, case.block_size, case.scale, case.dtype)


def vmax_of(t) -> float:
    """Largest |element| of a logical V tensor (the bound of the weights-rounding term)."""
    t = t if isinstance(t, torch.Tensor) else torch.from_numpy(np.asarray(t))
    return float(t.detach().to("cpu").float().abs().max()) if t.numel() else 0.0
