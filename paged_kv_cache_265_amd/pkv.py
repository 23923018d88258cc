"""Thin Python binding of libpkv.so (include/pkv.h).

Argument marshalling only: shapes are read from torch tensors, pointers and the
current HIP stream are handed to the C entry points, and a non-zero status is
raised as PkvError.  Every step of the computation runs in the library's HIP
kernels; there is no fallback of any kind, so without the built library every
call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

F32, F16, BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_CONTRACT = 0, -1, -2, -3, -4, -6

# device-side contract (include/pkv.h): verdict words and violation codes
CONTRACT_OK = (1 << 64) - 1
(BAD_CONTEXT_LEN, BAD_BLOCK_ID, BAD_QUERY_LENS, BAD_SLOT, DUPLICATE_SLOT, BAD_COPY_BLOCK, DUPLICATE_COPY_DST,
 COPY_DST_IS_SRC) = range(1, 9)

# every function include/pkv.h declares
SYMBOLS = (
    "pkv_version",
    "pkv_decode_partition_size",
    "pkv_decode_workspace_size",
    "paged_attention_decode",
    "paged_attention_decode_static",
    "pkv_decode_variant",
    "pkv_decode_variant_workspace_size",
    "paged_attention_chunked",
    "paged_attention_mixed",
    "pkv_mixed_workspace_size",
    "reshape_and_cache",
    "copy_blocks",
    "pkv_read_probe",
    "pkv_check_tables",
    "pkv_check_slots",
    "pkv_check_copies",
    "pkv_check_tables_host",
    "pkv_check_slots_host",
    "pkv_check_copies_host",
    "pkv_error_string",
    "pkv_last_error",
)

_lib = None


class PkvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first (python -c "
                           f"'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = I
    lib.pkv_decode_partition_size.argtypes = [I] * 7
    lib.pkv_decode_partition_size.restype = I
    lib.pkv_decode_workspace_size.argtypes = [I] * 7
    lib.pkv_decode_workspace_size.restype = Z
    lib.paged_attention_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, Z, P]
    lib.paged_attention_decode.restype = I
    lib.paged_attention_decode_static.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P]
    lib.paged_attention_decode_static.restype = I
    lib.pkv_decode_variant.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, Z, I, I, P]
    lib.pkv_decode_variant.restype = I
    lib.pkv_decode_variant_workspace_size.argtypes = [I] * 10
    lib.pkv_decode_variant_workspace_size.restype = Z
    lib.paged_attention_chunked.argtypes = [P, P, P, I, I, I, P, P, P, P, I, I, I, I, I, I, F, I, P]
    lib.paged_attention_chunked.restype = I
    lib.paged_attention_mixed.argtypes = [P, P, P, I, I, I, P, P, P, P, I, I, I, I, I, I, F, I, P, Z, P]
    lib.paged_attention_mixed.restype = I
    lib.pkv_mixed_workspace_size.argtypes = [I] * 5
    lib.pkv_mixed_workspace_size.restype = Z
    lib.reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
    lib.reshape_and_cache.restype = I
    lib.copy_blocks.argtypes = [P, P, I, P, I, I, I, I, I, I, P]
    lib.copy_blocks.restype = I
    lib.pkv_read_probe.argtypes = [P, Z, P, P]
    lib.pkv_read_probe.restype = I
    U64 = ctypes.c_uint64
    lib.pkv_check_tables.argtypes = [P, P, P, I, I, I, I, I, I, P, P]
    lib.pkv_check_slots.argtypes = [P, I, I, I, P, P]
    lib.pkv_check_copies.argtypes = [P, I, I, P, P]
    for f in (lib.pkv_check_tables, lib.pkv_check_slots, lib.pkv_check_copies):
        f.restype = I
    lib.pkv_check_tables_host.argtypes = [P, P, P, I, I, I, I, I, I]
    lib.pkv_check_slots_host.argtypes = [P, I, I, I]
    lib.pkv_check_copies_host.argtypes = [P, I, I]
    for f in (lib.pkv_check_tables_host, lib.pkv_check_slots_host, lib.pkv_check_copies_host):
        f.restype = U64
    lib.pkv_error_string.argtypes = [I]
    lib.pkv_error_string.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != OK:
        lib = load_library()
        raise PkvError(rc, f"{lib.pkv_error_string(rc).decode()}: {lib.pkv_last_error().decode()}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype(*ts: torch.Tensor) -> int:
    d = ts[0].dtype
    for t in ts[1:]:
        if t.dtype != d:
            raise TypeError(f"dtype mismatch: {d} vs {t.dtype}")
    if d not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {d}")
    return DTYPE_CODE[d]


def _contig(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def version() -> int:
    return load_library().pkv_version()


def decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                          partition_size: int = 0) -> int:
    rc = load_library().pkv_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                  max_blocks_per_seq, partition_size)
    if rc < 0:
        _check(rc)
    return rc


SIZE_INVALID = (1 << 64) - 1  # PKV_SIZE_INVALID


def _size(n: int) -> int:
    if n == SIZE_INVALID:
        raise PkvError(ERR_INVALID, load_library().pkv_last_error().decode())
    return int(n)


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                          partition_size: int = 0) -> int:
    return _size(load_library().pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                          max_blocks_per_seq, partition_size))


def paged_attention_decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                           value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                           scale: float, partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """out[s, h] = softmax over the sequence's cached tokens (see include/pkv.h).

    query/out [S, Hq, D]; key_cache [NB, Hkv, BS, D]; value_cache [NB, Hkv, D, BS];
    block_tables int32 [S, MB]; context_lens int32 [S].  A workspace is allocated
    here when none is given and one is needed."""
    _contig(out, query, key_cache, value_cache, block_tables, context_lens)
    S, Hq, D = query.shape
    NB, Hkv, BS, _ = key_cache.shape
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    dt = _dtype(out, query, key_cache, value_cache)
    need = decode_workspace_size(S, Hq, Hkv, D, BS, max(MB, 1), partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().paged_attention_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), _ptr(context_lens), S, Hq,
        Hkv, D, BS, NB, MB, float(scale), dt, int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc)
    return out


INNER_LOOP = {"auto": 0, "valu": 1, "mfma": 2}


def decode_variant(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, partition_size: int = 0,
                   inner_loop: str = "auto", ring: int = 0, stream=None) -> torch.Tensor:
    """Test and measurement hook (pkv_decode_variant): paged_attention_decode with the
    inner loop ("auto", "valu" or "mfma") and the prefetch ring (0: the loop's own, 2:
    two tiles) forced.  The workspace is allocated here."""
    _contig(out, query, key_cache, value_cache, block_tables, context_lens)
    S, Hq, D = query.shape
    NB, Hkv, BS, _ = key_cache.shape
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    dt = _dtype(out, query, key_cache, value_cache)
    lib = load_library()
    loop = INNER_LOOP[inner_loop]
    need = _size(lib.pkv_decode_variant_workspace_size(S, Hq, Hkv, D, BS, max(MB, 1), partition_size, dt, loop,
                                                       ring))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=query.device)
    rc = lib.pkv_decode_variant(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                                _ptr(context_lens), S, Hq, Hkv, D, BS, NB, MB, float(scale), dt, int(partition_size),
                                _ptr(ws), need, loop, int(ring), _stream(stream))
    _check(rc)
    return out


STATIC_SCRATCH_BYTES = 64 << 20  # PKV_STATIC_SCRATCH_BYTES


def paged_attention_decode_static(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                                  value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                                  scale: float, partition_size: int = 0, stream=None) -> torch.Tensor:
    """paged_attention_decode without a workspace: the library's static per-device
    scratch holds the partial records, so nothing is allocated (see include/pkv.h)."""
    _contig(out, query, key_cache, value_cache, block_tables, context_lens)
    S, Hq, D = query.shape
    NB, Hkv, BS, _ = key_cache.shape
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    dt = _dtype(out, query, key_cache, value_cache)
    rc = load_library().paged_attention_decode_static(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), _ptr(context_lens), S, Hq,
        Hkv, D, BS, NB, MB, float(scale), dt, int(partition_size), _stream(stream))
    _check(rc)
    return out


def paged_attention_chunked(out: torch.Tensor, query: torch.Tensor, cu_q_lens: torch.Tensor, max_q_len: int,
                            key_cache: torch.Tensor, value_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, scale: float, stream=None) -> torch.Tensor:
    """Causal attention of chunked-prefill segments (see include/pkv.h).

    query/out [total_q, Hq, D]; cu_q_lens int32 [num_segs + 1]; context_lens
    int32 [num_segs] counts each segment's cached tokens including its chunk."""
    _contig(out, query, cu_q_lens, key_cache, value_cache, block_tables, context_lens)
    T, Hq, D = query.shape
    NB, Hkv, BS, _ = key_cache.shape
    MB = block_tables.shape[1]
    dt = _dtype(out, query, key_cache, value_cache)
    rc = load_library().paged_attention_chunked(
        _ptr(out), _ptr(query), _ptr(cu_q_lens), cu_q_lens.shape[0] - 1, T, int(max_q_len), _ptr(key_cache),
        _ptr(value_cache), _ptr(block_tables), _ptr(context_lens), Hq, Hkv, D, BS, NB, MB, float(scale), dt,
        _stream(stream))
    _check(rc)
    return out


def mixed_workspace_size(num_segs, num_q_heads, num_kv_heads, head_dim, block_size) -> int:
    return _size(load_library().pkv_mixed_workspace_size(num_segs, num_q_heads, num_kv_heads, head_dim, block_size))


def paged_attention_mixed(out: torch.Tensor, query: torch.Tensor, cu_q_lens: torch.Tensor, max_q_len: int,
                          key_cache: torch.Tensor, value_cache: torch.Tensor, block_tables: torch.Tensor,
                          context_lens: torch.Tensor, scale: float, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """A flattened batch of decode tokens (one-row segments) and prefill chunks in one
    attention launch; same arguments and result as paged_attention_chunked (see
    include/pkv.h).  A workspace is allocated here when none is given."""
    _contig(out, query, cu_q_lens, key_cache, value_cache, block_tables, context_lens)
    T, Hq, D = query.shape
    NB, Hkv, BS, _ = key_cache.shape
    MB = block_tables.shape[1]
    S = cu_q_lens.shape[0] - 1
    dt = _dtype(out, query, key_cache, value_cache)
    need = mixed_workspace_size(S, Hq, Hkv, D, BS) if S > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load_library().paged_attention_mixed(
        _ptr(out), _ptr(query), _ptr(cu_q_lens), S, T, int(max_q_len), _ptr(key_cache), _ptr(value_cache),
        _ptr(block_tables), _ptr(context_lens), Hq, Hkv, D, BS, NB, MB, float(scale), dt, _ptr(workspace), ws_bytes,
        _stream(stream))
    _check(rc)
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                      slot_mapping: torch.Tensor, stream=None) -> None:
    """Write key/value [Ntok, Hkv, D] into the slots slot_mapping (int64) names."""
    _contig(key, value, key_cache, value_cache, slot_mapping)
    n = slot_mapping.shape[0]
    NB, Hkv, BS, D = key_cache.shape
    dt = _dtype(key, value, key_cache, value_cache)
    rc = load_library().reshape_and_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                          _ptr(slot_mapping), n, Hkv, D, BS, NB, dt, _stream(stream))
    _check(rc)


def copy_blocks(key_caches: Sequence[torch.Tensor], value_caches: Sequence[torch.Tensor],
                block_mapping: torch.Tensor, stream=None) -> None:
    """Copy whole blocks src -> dst (block_mapping int64 [Npairs, 2]) in every layer."""
    L = len(key_caches)
    if L != len(value_caches):
        raise ValueError("key_caches and value_caches differ in length")
    _contig(block_mapping, *key_caches, *value_caches)
    NB, Hkv, BS, D = key_caches[0].shape if L else (1, 1, 16, 64)
    dt = _dtype(*key_caches, *value_caches) if L else F16
    kp = (ctypes.c_void_p * max(L, 1))(*[t.data_ptr() for t in key_caches])
    vp = (ctypes.c_void_p * max(L, 1))(*[t.data_ptr() for t in value_caches])
    npairs = block_mapping.shape[0] if block_mapping.dim() == 2 else block_mapping.numel() // 2
    rc = load_library().copy_blocks(kp, vp, L, _ptr(block_mapping), npairs, Hkv, D, BS, NB, dt, _stream(stream))
    _check(rc)


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream every byte of `buf` with the decode kernels' load shape (a measurement
    utility for the practical read ceiling; see include/pkv.h)."""
    _contig(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    rc = load_library().pkv_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream))
    _check(rc)


# ---- the device-side contract --------------------------------------------------------

def violation(index: int, sub: int, code: int) -> int:
    """The verdict word of one violation: (index << 32) | (sub-index << 8) | code."""
    return (index << 32) | (min(max(sub, 0), 0xFFFFFF) << 8) | code


def unpack_verdict(v: int):
    """(index, sub-index, code) of a verdict word other than CONTRACT_OK."""
    return v >> 32, (v >> 8) & 0xFFFFFF, v & 0xFF


def _verdict_call(fn, *args, stream=None) -> int:
    out = ctypes.c_uint64(CONTRACT_OK)
    _check(fn(*args, ctypes.byref(out), _stream(stream)))
    return out.value


def check_tables(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int, num_blocks: int,
                 cu_q_lens: Optional[torch.Tensor] = None, total_q: int = 0, max_q_len: int = 0, stream=None) -> int:
    """Verdict of the contract pre-pass over device block tables / context lengths
    (and query lengths when cu_q_lens is given)."""
    _contig(block_tables, context_lens)
    rows, MB = block_tables.shape
    return _verdict_call(load_library().pkv_check_tables, _ptr(block_tables), _ptr(context_lens), _ptr(cu_q_lens),
                         rows, MB, block_size, num_blocks, total_q, max_q_len, stream=stream)


def check_slots(slot_mapping: torch.Tensor, block_size: int, num_blocks: int, stream=None) -> int:
    _contig(slot_mapping)
    return _verdict_call(load_library().pkv_check_slots, _ptr(slot_mapping), slot_mapping.shape[0], block_size,
                         num_blocks, stream=stream)


def check_copies(block_mapping: torch.Tensor, num_blocks: int, stream=None) -> int:
    _contig(block_mapping)
    return _verdict_call(load_library().pkv_check_copies, _ptr(block_mapping), block_mapping.shape[0], num_blocks,
                         stream=stream)


def _host(a, dtype):
    import numpy as np
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def check_tables_host(block_tables, context_lens, block_size: int, num_blocks: int, cu_q_lens=None, total_q: int = 0,
                      max_q_len: int = 0) -> int:
    """The same verdict from the same item checks run on the CPU over host arrays."""
    import numpy as np
    bt, cl = _host(block_tables, np.int32), _host(context_lens, np.int32)
    cu = None if cu_q_lens is None else _host(cu_q_lens, np.int32)
    rows, MB = bt.shape
    return int(load_library().pkv_check_tables_host(bt.ctypes.data, cl.ctypes.data,
                                                    None if cu is None else cu.ctypes.data, rows, MB, block_size,
                                                    num_blocks, total_q, max_q_len))


def check_slots_host(slot_mapping, block_size: int, num_blocks: int) -> int:
    import numpy as np
    sm = _host(slot_mapping, np.int64)
    return int(load_library().pkv_check_slots_host(sm.ctypes.data, sm.shape[0], block_size, num_blocks))


def check_copies_host(block_mapping, num_blocks: int) -> int:
    import numpy as np
    bm = _host(block_mapping, np.int64).reshape(-1, 2)
    return int(load_library().pkv_check_copies_host(bm.ctypes.data, bm.shape[0], num_blocks))
