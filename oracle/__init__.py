"""fp64 CPU oracle for paged attention, reshape_and_cache and copy_blocks.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path never does.  It shares no
code with the GPU library: ``oracle.c`` is compiled by gcc on its own, and
``brute.py`` holds a NumPy dense-attention reference on logical (never paged)
K/V used to pin the C oracle.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(brute force, placement invariance, closed forms, worked byte counts); no
function is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# a different build of oracle.c (e.g. a deliberately broken copy in the
# self-test that shows the pins catch mistakes) can be pointed to here
LIB_PATH = os.environ.get("PKV_ORACLE_LIB", os.path.join(HERE, "liboracle.so"))

_DT = {"f32": 0, "f16": 1, "bf16": 2}
_ESZ = {"f32": 4, "f16": 2, "bf16": 2}
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I, D, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_longlong
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, D, I]
    lib.oracle_chunked.argtypes = [P, P, P, I, P, P, P, P, I, I, I, I, I, I, D, I]
    lib.oracle_reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
    lib.oracle_copy_blocks.argtypes = [P, P, I, P, I, I, I, I, I, I]
    lib.oracle_kv_bytes_per_token.argtypes = [I, I, I, I]
    lib.oracle_kv_bytes_per_token.restype = LL
    lib.oracle_kv_bytes_per_block.argtypes = [I, I, I, I]
    lib.oracle_kv_bytes_per_block.restype = LL
    lib.oracle_decode_element.argtypes = [P, LL, I]
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    lib.oracle_decode_element.restype = D
    for f in (lib.oracle_decode, lib.oracle_chunked, lib.oracle_reshape_and_cache, lib.oracle_copy_blocks):
        f.restype = I
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _arr(x, dtype=None):
    """Host array view (numpy) of a numpy array or CPU torch tensor, contiguous."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            assert x.device.type == "cpu", "the oracle reads host memory only"
            x = x.contiguous()
            if x.dtype in (torch.bfloat16, torch.float16):
                x = x.view(torch.int16)
            x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x if dtype is None else np.asarray(x, dtype=dtype))
    return x


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def decode(query, key_cache, value_cache, block_tables, context_lens, num_kv_heads, block_size, scale,
           dtype: str) -> np.ndarray:
    """fp64 output [S, Hq, D] of paged decode attention (see oracle.c)."""
    q = _arr(query)
    S, Hq, D = q.shape
    kc, vc = _arr(key_cache), _arr(value_cache)
    bt = _arr(block_tables, np.int32)
    cl = _arr(context_lens, np.int32)
    NB = kc.shape[0]
    MB = bt.shape[1] if bt.ndim == 2 and bt.shape[1] > 0 else 1
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode(_p(out), _p(q), _p(kc), _p(vc), _p(bt), _p(cl), S, Hq, num_kv_heads, D,
                               block_size, NB, MB, float(scale), _DT[dtype])
    _check(rc, "oracle_decode")
    return out


def chunked(query, cu_q_lens, key_cache, value_cache, block_tables, context_lens, num_kv_heads, block_size,
            scale, dtype: str) -> np.ndarray:
    """fp64 output [total_q, Hq, D] of causal chunked-prefill attention."""
    q = _arr(query)
    T, Hq, D = q.shape
    cu = _arr(cu_q_lens, np.int32)
    kc, vc = _arr(key_cache), _arr(value_cache)
    bt = _arr(block_tables, np.int32)
    cl = _arr(context_lens, np.int32)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    rc = _load().oracle_chunked(_p(out), _p(q), _p(cu), len(cu) - 1, _p(kc), _p(vc), _p(bt), _p(cl), Hq,
                                num_kv_heads, D, block_size, kc.shape[0], bt.shape[1], float(scale), _DT[dtype])
    _check(rc, "oracle_chunked")
    return out


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, dtype: str) -> None:
    """Write tokens into the caches in place (caches must be numpy arrays or
    contiguous CPU tensors; they are modified)."""
    k, v = _arr(key), _arr(value)
    kc, vc = _arr(key_cache), _arr(value_cache)
    sm = _arr(slot_mapping, np.int64)
    n = sm.shape[0]
    H, D = (k.shape[1], k.shape[2]) if k.ndim == 3 else (kc.shape[1], kc.shape[3])
    rc = _load().oracle_reshape_and_cache(_p(k), _p(v), _p(kc), _p(vc), _p(sm), n, H, D, kc.shape[2],
                                          kc.shape[0], _DT[dtype])
    _check(rc, "oracle_reshape_and_cache")
    _writeback(key_cache, kc)
    _writeback(value_cache, vc)


def copy_blocks(key_caches, value_caches, block_mapping, dtype: str) -> None:
    """Copy whole blocks (src -> dst) in every layer, in place."""
    ks = [_arr(x) for x in key_caches]
    vs = [_arr(x) for x in value_caches]
    bm = _arr(block_mapping, np.int64).reshape(-1, 2)
    L = len(ks)
    kp = (ctypes.c_void_p * max(L, 1))(*[a.ctypes.data for a in ks])
    vp = (ctypes.c_void_p * max(L, 1))(*[a.ctypes.data for a in vs])
    shape = ks[0].shape if L else (1, 1, 1, 1)
    rc = _load().oracle_copy_blocks(kp, vp, L, _p(bm), bm.shape[0], shape[1], shape[3], shape[2], shape[0],
                                    _DT[dtype])
    _check(rc, "oracle_copy_blocks")
    for a, b in zip(key_caches, ks):
        _writeback(a, b)
    for a, b in zip(value_caches, vs):
        _writeback(a, b)


def _writeback(orig, arr):
    """If _arr had to copy, write results back into the caller's object."""
    try:
        import torch
        if isinstance(orig, torch.Tensor):
            view = orig.view(torch.int16) if orig.dtype in (torch.bfloat16, torch.float16) else orig
            if view.numpy().ctypes.data != arr.ctypes.data:
                view.copy_(torch.from_numpy(arr))
            return
    except ImportError:  # pragma: no cover
        pass
    if isinstance(orig, np.ndarray) and orig.ctypes.data != arr.ctypes.data:
        orig[...] = arr


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes) -> int:
    return int(_load().oracle_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes))


def kv_bytes_per_block(block_size, num_kv_heads, head_dim, elem_bytes) -> int:
    return int(_load().oracle_kv_bytes_per_block(block_size, num_kv_heads, head_dim, elem_bytes))


def decode_elements(raw, dtype: str) -> np.ndarray:
    """Decode every element of a raw array with the oracle's own decoders."""
    a = _arr(raw)
    flat = a.reshape(-1)
    lib = _load()
    return np.array([lib.oracle_decode_element(_p(flat), i, _DT[dtype]) for i in range(flat.size)])


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())
