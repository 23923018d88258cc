"""Seeded generators for paged KV pools, block tables and queries.

Pool layout (the library's ABI layout, stated here so inputs can be built):
  key_cache   [num_blocks, num_kv_heads, block_size, head_dim]   token-major tile
  value_cache [num_blocks, num_kv_heads, head_dim, block_size]   head_dim-major tile
  block_tables int32 [num_seqs, max_blocks_per_seq]; padding entries are INT32_MAX
  slot = physical_block * block_size + offset_in_block (int64)

Every slot and block that holds no token is filled with NaN, so a reader that
touches one is caught.  Random numbers come from numpy's PCG64 generator seeded
with a list ``[265, config]``; values are drawn in float32 from N(0, 1) and
rounded to the storage type by torch (round to nearest even).

Draw order inside ``build_paged``: placement permutation, then K of all tokens in
logical order, then V.  Callers draw context lengths before and queries after.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

INT32_MAX = np.iinfo(np.int32).max

# name -> (torch dtype, ABI code, bytes per element)
DTYPES = {
    "f32": (torch.float32, 0, 4),
    "f16": (torch.float16, 1, 2),
    "bf16": (torch.bfloat16, 2, 2),
}


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of K plus V that one token occupies across all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DTYPES[dtype][0])


@dataclass
class Pool:
    dtype: str
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    key_cache: torch.Tensor    # [NB, Hkv, BS, D]
    value_cache: torch.Tensor  # [NB, Hkv, D, BS]

    @property
    def block_bytes(self) -> int:
        """Bytes of one block of K (or of V) over all kv heads."""
        return self.num_kv_heads * self.block_size * self.head_dim * DTYPES[self.dtype][2]

    def clone(self) -> "Pool":
        return Pool(self.dtype, self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size,
                    self.key_cache.clone(), self.value_cache.clone())


def new_pool(dtype: str, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int) -> Pool:
    tdt = DTYPES[dtype][0]
    k = torch.full((num_blocks, num_kv_heads, block_size, head_dim), float("nan"), dtype=tdt)
    v = torch.full((num_blocks, num_kv_heads, head_dim, block_size), float("nan"), dtype=tdt)
    return Pool(dtype, num_blocks, num_kv_heads, head_dim, block_size, k, v)


def write_tokens(pool: Pool, slots: np.ndarray, k: torch.Tensor, v: torch.Tensor) -> None:
    """Place tokens (rows of k, v: [n, Hkv, D]) at the given slots of the pool."""
    if len(slots) == 0:
        return
    slots = np.asarray(slots, dtype=np.int64)
    blk = torch.from_numpy(slots // pool.block_size)
    off = torch.from_numpy(slots % pool.block_size)
    pool.key_cache[blk, :, off, :] = k
    pool.value_cache[blk, :, :, off] = v


@dataclass
class Paged:
    """Sequences placed in a shuffled pool."""
    pool: Pool
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, MB]
    cu_tokens: np.ndarray             # int64 [S+1], logical token offsets
    logical_k: torch.Tensor           # [T, Hkv, D] storage dtype
    logical_v: torch.Tensor
    token_slots: np.ndarray           # int64 [T], slot of each logical token
    pending: np.ndarray               # bool [T], tokens left for reshape_and_cache

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]


def build_paged(rng: np.random.Generator, dtype: str, num_kv_heads: int, head_dim: int,
                block_size: int, context_lens: Sequence[int], resident_lens: Optional[Sequence[int]] = None,
                max_blocks_per_seq: Optional[int] = None, num_blocks: Optional[int] = None,
                pool_factor: float = 1.25) -> Paged:
    """Scatter seeded logical K/V of each sequence into a randomly placed pool.

    Sequence s has context_lens[s] tokens; the first resident_lens[s] are written
    now, the rest are marked pending (their slots stay NaN)."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    res = ctx if resident_lens is None else np.asarray(resident_lens, dtype=np.int64)
    NB, bt, cu, slots = _place(rng, ctx, block_size, max_blocks_per_seq, num_blocks, pool_factor)
    T = int(cu[-1])
    pend = np.zeros(T, dtype=bool)
    for s in range(len(ctx)):
        pend[cu[s]:cu[s + 1]] = np.arange(int(ctx[s])) >= res[s]
    k = _cast(rng.standard_normal((T, num_kv_heads, head_dim), dtype=np.float32), dtype)
    v = _cast(rng.standard_normal((T, num_kv_heads, head_dim), dtype=np.float32), dtype)
    pool = new_pool(dtype, NB, num_kv_heads, head_dim, block_size)
    keep = ~pend
    write_tokens(pool, slots[keep], k[torch.from_numpy(keep)], v[torch.from_numpy(keep)])
    return Paged(pool, ctx.astype(np.int32), bt, cu, k, v, slots, pend)


def _place(rng, ctx, block_size, max_blocks_per_seq, num_blocks, pool_factor):
    """Random block placement: (pool blocks, block tables, token offsets, token slots)."""
    S = len(ctx)
    nblk = (ctx + block_size - 1) // block_size
    need = int(nblk.sum())
    MB = int(max(1, nblk.max() if S else 1)) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    assert (nblk <= MB).all()
    NB = int(math.ceil(pool_factor * need)) if num_blocks is None else int(num_blocks)
    NB = max(NB, need, 1)
    perm = rng.permutation(NB)[:need]
    bt = np.full((S, MB), INT32_MAX, dtype=np.int32)
    cu = np.zeros(S + 1, dtype=np.int64)
    cu[1:] = np.cumsum(ctx)
    slots = np.empty(int(cu[-1]), dtype=np.int64)
    pos = 0
    for s in range(S):
        n = int(ctx[s])
        b = int(nblk[s])
        phys = perm[pos:pos + b]
        pos += b
        bt[s, :b] = phys
        t = np.arange(n, dtype=np.int64)
        slots[cu[s]:cu[s + 1]] = phys[t // block_size].astype(np.int64) * block_size + t % block_size
    return NB, bt, cu, slots


def reblock(p: Paged, block_size: int, rng: np.random.Generator, pool_factor: float = 1.25) -> Paged:
    """The same logical K/V (pending tokens stay unwritten) in a new pool of another
    block size, with a fresh random placement."""
    ctx = p.context_lens.astype(np.int64)
    nblk = (ctx + block_size - 1) // block_size
    NB, bt, cu, slots = _place(rng, ctx, block_size, None, None, pool_factor)
    pool = new_pool(p.pool.dtype, NB, p.pool.num_kv_heads, p.pool.head_dim, block_size)
    keep = ~p.pending
    write_tokens(pool, slots[keep], p.logical_k[torch.from_numpy(keep)], p.logical_v[torch.from_numpy(keep)])
    assert bt.shape[1] == max(1, int(nblk.max() if len(ctx) else 1))
    return Paged(pool, p.context_lens.copy(), bt, cu, p.logical_k, p.logical_v, slots, p.pending.copy())


@dataclass
class DecodeCase:
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    paged: Paged
    query: torch.Tensor                         # [S, Hq, D]
    new_key: Optional[torch.Tensor] = None      # [Ntok, Hkv, D] tokens to write first
    new_value: Optional[torch.Tensor] = None
    slot_mapping: Optional[np.ndarray] = None   # int64 [Ntok]
    label: str = ""

    @property
    def pool(self) -> Pool:
        return self.paged.pool

    @property
    def context_lens(self) -> np.ndarray:
        return self.paged.context_lens

    @property
    def block_tables(self) -> np.ndarray:
        return self.paged.block_tables

    @property
    def num_blocks(self) -> int:
        return self.paged.pool.num_blocks

    @property
    def max_blocks_per_seq(self) -> int:
        return self.paged.max_blocks_per_seq


def _pending_writes(p: Paged):
    idx = np.nonzero(p.pending)[0]
    ti = torch.from_numpy(idx)
    return p.logical_k[ti].contiguous(), p.logical_v[ti].contiguous(), p.token_slots[idx].copy()


def make_decode_case(seed, dtype: str, context_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                     head_dim: int, block_size: int = 16, scale: Optional[float] = None,
                     append_last: bool = False, max_blocks_per_seq: Optional[int] = None,
                     num_blocks: Optional[int] = None, rng: Optional[np.random.Generator] = None,
                     label: str = "") -> DecodeCase:
    """Decode batch; with append_last the newest token of each sequence is left
    for reshape_and_cache (context_lens already count it)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    ctx = np.asarray(context_lens, dtype=np.int64)
    res = np.maximum(ctx - 1, 0) if append_last else ctx
    p = build_paged(rng, dtype, num_kv_heads, head_dim, block_size, ctx, res, max_blocks_per_seq, num_blocks)
    q = _cast(rng.standard_normal((len(ctx), num_q_heads, head_dim), dtype=np.float32), dtype)
    sc = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    c = DecodeCase(dtype, len(ctx), num_q_heads, num_kv_heads, head_dim, block_size, sc, p, q, label=label)
    if append_last:
        c.new_key, c.new_value, c.slot_mapping = _pending_writes(p)
    return c


@dataclass
class ChunkedCase:
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    paged: Paged
    query: torch.Tensor            # [total_q, Hq, D]
    cu_q_lens: np.ndarray          # int32 [nseg+1]
    new_key: torch.Tensor          # chunk tokens, written before attention
    new_value: torch.Tensor
    slot_mapping: np.ndarray
    label: str = ""

    @property
    def num_segs(self) -> int:
        return len(self.cu_q_lens) - 1

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.cu_q_lens).max()) if self.num_segs else 0


def make_chunked_case(seed, dtype: str, cached_lens: Sequence[int], q_lens: Sequence[int], num_q_heads: int,
                      num_kv_heads: int, head_dim: int, block_size: int = 16, scale: Optional[float] = None,
                      max_blocks_per_seq: Optional[int] = None, rng: Optional[np.random.Generator] = None,
                      label: str = "") -> ChunkedCase:
    """Chunked-prefill segments: cached_lens[i] tokens already in the pool, then a
    chunk of q_lens[i] new tokens whose K/V are written before attention."""
    rng = np.random.default_rng(seed) if rng is None else rng
    cached = np.asarray(cached_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    ctx = cached + ql
    p = build_paged(rng, dtype, num_kv_heads, head_dim, block_size, ctx, cached, max_blocks_per_seq)
    cu = np.zeros(len(ql) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    q = _cast(rng.standard_normal((int(cu[-1]), num_q_heads, head_dim), dtype=np.float32), dtype)
    sc = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    nk, nv, sm = _pending_writes(p)
    return ChunkedCase(dtype, num_q_heads, num_kv_heads, head_dim, block_size, sc, p, q, cu, nk, nv, sm, label)


# ----------------------------------------------------------------------------
# Prefix-shared parallel sampling with copy-on-write of the shared last block.
# ----------------------------------------------------------------------------

@dataclass
class CowCase:
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    pool: Pool                    # state before copy_blocks / reshape_and_cache
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S, MB] after copy-on-write planning
    query: torch.Tensor           # [S, Hq, D]
    block_mapping: np.ndarray     # int64 [Npairs, 2] (src, dst)
    new_key: torch.Tensor         # private tokens of every sample, sample order
    new_value: torch.Tensor
    slot_mapping: np.ndarray      # int64
    prompt_of: np.ndarray         # int32 [S] prompt index of each sample
    prompt_lens: np.ndarray       # int64 [P]
    private_lens: np.ndarray      # int64 [S]
    prompt_k: List[torch.Tensor]  # per prompt [len, Hkv, D]
    prompt_v: List[torch.Tensor]
    private_k: List[torch.Tensor]  # per sample [n, Hkv, D]
    private_v: List[torch.Tensor]
    refcount: np.ndarray          # int32 [NB] references after planning
    shared_blocks: np.ndarray     # physical ids of prompt blocks still shared

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)

    @property
    def num_blocks(self) -> int:
        return self.pool.num_blocks

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]

    def logical(self, s: int):
        """Logical K/V of sample s: its prompt followed by its own tokens."""
        p = int(self.prompt_of[s])
        return (torch.cat([self.prompt_k[p], self.private_k[s]]), torch.cat([self.prompt_v[p], self.private_v[s]]))


class _BlockManager:
    """Minimal host bookkeeping: free list, refcounts, copy-on-write planning."""

    def __init__(self, order: np.ndarray):
        self.free = list(order[::-1])
        self.ref = {}

    def alloc(self) -> int:
        b = int(self.free.pop())
        self.ref[b] = 1
        return b


def make_cow_case(seed, dtype: str = "bf16", num_prompts: int = 16, samples_per_prompt: int = 8,
                  prompt_blocks: int = 64, max_private: int = 256, num_q_heads: int = 32, num_kv_heads: int = 8,
                  head_dim: int = 128, block_size: int = 16, prompt_short: Optional[Sequence[int]] = None,
                  private_lens: Optional[Sequence[int]] = None, max_blocks_per_seq: Optional[int] = None,
                  pool_factor: float = 1.25) -> CowCase:
    """Parallel sampling: each prompt's blocks are shared by its samples with a
    refcount; a sample that appends into a block still shared copies it first
    (the count drops by one per copy) and the last sharer writes in place."""
    rng = np.random.default_rng(seed)
    P, G = num_prompts, samples_per_prompt
    S = P * G
    BS = block_size
    r = (rng.integers(1, BS, size=P, endpoint=False) if prompt_short is None
         else np.asarray(prompt_short, dtype=np.int64))
    plen = prompt_blocks * BS - r
    npriv = (rng.integers(0, max_private, size=S, endpoint=True) if private_lens is None
             else np.asarray(private_lens, dtype=np.int64))
    prompt_of = np.repeat(np.arange(P, dtype=np.int32), G)
    ctx = plen[prompt_of] + npriv
    nblk = (ctx + BS - 1) // BS
    MB = int(nblk.max()) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    # blocks needed: shared prompt blocks, plus per sample its copy and fresh blocks
    need = P * prompt_blocks + int(np.sum(np.maximum(nblk - prompt_blocks, 0))) + S
    NB = int(math.ceil(pool_factor * need))
    order = rng.permutation(NB)
    bm = _BlockManager(order)
    bt = np.full((S, MB), INT32_MAX, dtype=np.int32)
    pool = new_pool(dtype, NB, num_kv_heads, head_dim, BS)
    prompt_k, prompt_v, shared = [], [], []
    for p in range(P):
        blocks = [bm.alloc() for _ in range(prompt_blocks)]
        for b in blocks:
            bm.ref[b] = G
        shared.extend(blocks)
        n = int(plen[p])
        k = _cast(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)
        v = _cast(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)
        t = np.arange(n, dtype=np.int64)
        write_tokens(pool, np.asarray(blocks, dtype=np.int64)[t // BS] * BS + t % BS, k, v)
        prompt_k.append(k)
        prompt_v.append(v)
        for j in range(G):
            bt[p * G + j, :prompt_blocks] = blocks
    pairs, slots, priv_k, priv_v = [], [], [], []
    for s in range(S):
        n = int(npriv[s])
        k = _cast(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)
        v = _cast(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)
        priv_k.append(k)
        priv_v.append(v)
        base = int(plen[prompt_of[s]])
        for i in range(n):
            pos = base + i
            lb = pos // BS
            if lb < prompt_blocks:
                cur = int(bt[s, lb])
                if bm.ref[cur] > 1:  # still shared: copy, drop the count, write the copy
                    new = bm.alloc()
                    pairs.append((cur, new))
                    bm.ref[cur] -= 1
                    bt[s, lb] = new
            elif bt[s, lb] == INT32_MAX:
                bt[s, lb] = bm.alloc()
            slots.append(int(bt[s, lb]) * BS + pos % BS)
    query = _cast(rng.standard_normal((S, num_q_heads, head_dim), dtype=np.float32), dtype)
    ref = np.zeros(NB, dtype=np.int32)
    for b, c in bm.ref.items():
        ref[b] = c
    nk = torch.cat(priv_k) if S else torch.empty(0)
    nv = torch.cat(priv_v) if S else torch.empty(0)
    still = np.asarray([b for b in shared if ref[b] > 0], dtype=np.int64)
    return CowCase(dtype, num_q_heads, num_kv_heads, head_dim, BS, 1.0 / math.sqrt(head_dim), pool,
                   ctx.astype(np.int32), bt, query,
                   np.asarray(pairs, dtype=np.int64).reshape(-1, 2), nk.contiguous(), nv.contiguous(),
                   np.asarray(slots, dtype=np.int64), prompt_of, plen, npriv, prompt_k, prompt_v,
                   priv_k, priv_v, ref, still)


def append_tokens(pool: Pool, block_tables: np.ndarray, context_lens: np.ndarray, seqs: Sequence[int]) -> np.ndarray:
    """Slots at which each listed sequence's next token goes (no allocation: the
    slot must lie in a block the table already holds)."""
    out = []
    for s in seqs:
        pos = int(context_lens[s])
        out.append(int(block_tables[s, pos // pool.block_size]) * pool.block_size + pos % pool.block_size)
    return np.asarray(out, dtype=np.int64)


# ----------------------------------------------------------------------------
# The five workloads.
# ----------------------------------------------------------------------------

def config_decode(cfg: int) -> DecodeCase:
    """Decode workloads 1-3 (tiny MHA fp32, OPT-13B-shaped MHA fp16, GQA bf16)."""
    rng = np.random.default_rng([265, cfg])
    if cfg == 1:
        return make_decode_case(None, "f32", [1, 7, 16, 33], 4, 4, 64, 16, scale=1.0 / 8.0,
                                max_blocks_per_seq=3, num_blocks=32, rng=rng, label="tiny MHA f32")
    if cfg == 2:
        ctx = rng.integers(128, 2048, size=64, endpoint=True)
        return make_decode_case(None, "f16", ctx, 40, 40, 128, 16, scale=1.0 / math.sqrt(128),
                                max_blocks_per_seq=128, rng=rng, label="OPT-13B layer MHA f16")
    if cfg == 3:
        z = rng.standard_normal(256)
        ctx = np.clip(np.rint(np.exp(math.log(1024.0) + 1.0 * z)), 16, 8192).astype(np.int64)
        return make_decode_case(None, "bf16", ctx, 32, 8, 128, 16, append_last=True,
                                max_blocks_per_seq=512, rng=rng, label="GQA 32/8 bf16")
    raise ValueError(cfg)


def config_cow(seed=(265, 4)) -> CowCase:
    """Workload 4: 16 prompts x 8 samples sharing prompt blocks, GQA 32/8 bf16."""
    return make_cow_case(list(seed), max_blocks_per_seq=80)


def config_long_mixed(decode_seqs: int = 32, segs: int = 8):
    """Workload 5: MQA 32/1 bf16 long-context decode plus chunked-prefill segments,
    both in one pool (one Paged object; decode sequences first)."""
    rng = np.random.default_rng([265, 5])
    dctx = rng.integers(16384, 131072, size=decode_seqs, endpoint=True)
    cached = np.full(segs, 4096, dtype=np.int64)
    ql = np.full(segs, 512, dtype=np.int64)
    ctx = np.concatenate([dctx, cached + ql])
    res = np.concatenate([dctx, cached])
    p = build_paged(rng, "bf16", 1, 128, 16, ctx, res, max_blocks_per_seq=8192)
    qd = _cast(rng.standard_normal((decode_seqs, 32, 128), dtype=np.float32), "bf16")
    cu = np.zeros(segs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    qc = _cast(rng.standard_normal((int(cu[-1]), 32, 128), dtype=np.float32), "bf16")
    return p, qd, qc, cu


def algorithmic_decode_bytes(context_lens: np.ndarray, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             elem_bytes: int) -> int:
    """K and V of every logical token for every kv head, read once, plus the query."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    return int(ctx.sum()) * num_kv_heads * head_dim * 2 * elem_bytes + len(ctx) * num_q_heads * head_dim * elem_bytes


def algorithmic_chunked_flops(context_lens: np.ndarray, q_lens: np.ndarray, num_q_heads: int, head_dim: int) -> int:
    """Multiply-adds of QK^T and PV over the causal key ranges, two flops each."""
    pairs = 0
    for n, L in zip(np.asarray(context_lens, dtype=np.int64), np.asarray(q_lens, dtype=np.int64)):
        first = n - L + 1  # keys seen by row 0
        pairs += int(L * first + L * (L - 1) // 2)
    return pairs * num_q_heads * head_dim * 2 * 2
