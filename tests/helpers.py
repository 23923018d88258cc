"""Shared helpers of the GPU parity tests: moving seeded cases to the device,
running the library, and the acceptance check against the fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

import oracle

# acceptance bar: fp32 inputs max abs error <= 1e-5; 16-bit inputs max abs error
# <= 2e-3 and, per output row (one query head of one token), max |err| / max |ref|
# <= 1e-2 (a relative error per element is not used as a gate: outputs cross zero)
TOL_F32_ABS = 1e-5
TOL_16_ABS = 2e-3
TOL_16_ROW_REL = 1e-2


def dev(x, device="cuda"):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(device).contiguous()


def check_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """Assert the acceptance bar; returns the error statistics."""
    g = gpu.detach().to("cpu").to(torch.float64).numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    stats = {"max_abs": float(err.max()) if err.size else 0.0}
    if dtype == "f32":
        assert stats["max_abs"] <= TOL_F32_ABS, f"{what}: max abs err {stats['max_abs']:.3e}"
        return stats
    rows_ref = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    rows_err = err.reshape(-1, ref.shape[-1]).max(axis=1)
    live = rows_ref > 0
    rel = rows_err[live] / rows_ref[live]
    stats["max_row_rel"] = float(rel.max()) if rel.size else 0.0
    assert stats["max_abs"] <= TOL_16_ABS, f"{what}: max abs err {stats['max_abs']:.3e}"
    assert stats["max_row_rel"] <= TOL_16_ROW_REL, f"{what}: max row rel err {stats['max_row_rel']:.3e}"
    assert np.all(rows_err[~live] == 0), f"{what}: zero reference rows must give exact zeros"
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
