"""Plain model of the paged KV-cache block manager -- TEST INFRASTRUCTURE.

Only the tests (and the benchmark's CPU leg) may use this module; the product
path never does.  It shares no code with the native manager in
paged_kv_cache_265_amd/csrc/block_manager.cpp: both are written from the pages.

What it models ("现代 LLM 推理引擎剖析", sections 1.3 and 2.2; "每生成一个字都要把全部
权重读一遍：从 vLLM 看 LLM 推理提速", paging section and its copy-on-write paragraph):
- a pool of fixed-size blocks; the free ones wait in a free-block queue;
- a block table per sequence maps its logical blocks to physical ones, filled
  on demand as the sequence grows (only the last block can be partial);
- every physical block has a reference count; a fork shares all of the parent's
  blocks (count + 1 each); a write into a shared last block first copies it to a
  fresh block (copy-on-write), lowering the old block's count by one;
- prefix caching: each full block of a prompt gets a hash chained from the
  previous block's hash and the block's token ids; a new prompt reuses the
  longest run of leading blocks whose hashes are cached (count + 1);
- freeing (or preempting) a sequence lowers its blocks' counts; blocks that
  reach zero go back to the free queue, keeping their hash until they are
  handed out again.

Readings where the pages leave the policy open (the native manager follows the
same ones):
1. The free queue is first-in first-out: blocks are handed out from its head,
   freed blocks join its tail; at creation it holds 0 .. num_blocks-1 in order.
2. A freed sequence releases its blocks from the last logical block to the
   first, so a prompt's leading blocks stay longest in the queue (and cached).
3. The hash of block i is FNV-1a (64-bit) over the little-endian bytes of the
   previous hash (block 0: the FNV offset basis) followed by the block's token
   ids as little-endian int32.  A lookup hit also requires the cached block's
   token ids to equal the chunk's (no reliance on hash uniqueness).
4. A cached block is only ever a full prompt block; a block handed out again
   from the free queue loses its hash.  When two blocks would carry the same
   hash, the first one registered keeps it.
5. The copy-on-write count update is "decrement by one per copy" (the page
   says the count goes back to 1 for the two-sharer case).

Parity status: pinned by tests/test_block_manager.py against invariants that
hold for any correct manager (reference counts equal the table references, the
free queue holds exactly the unreferenced blocks, every sequence reads back its
own token history through its table from a simulated pool, copies only on
shared blocks) and by published FNV-1a test vectors.
"""

from __future__ import annotations

from collections import OrderedDict
from typing import Dict, List, Optional, Sequence, Tuple

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the FNV prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(prev: int, tokens: Sequence[int]) -> int:
    data = prev.to_bytes(8, "little") + b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


def chunk_hashes(tokens: Sequence[int], block_size: int) -> List[int]:
    """Chained hashes of the full block_size-token chunks of a prompt."""
    out, prev = [], FNV_OFFSET
    for i in range(len(tokens) // block_size):
        prev = block_hash(prev, tokens[i * block_size:(i + 1) * block_size])
        out.append(prev)
    return out


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.free: "OrderedDict[int, None]" = OrderedDict((b, None) for b in range(num_blocks))
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.hash_of: Dict[int, int] = {}            # block -> its cached hash
        self.tokens_of: Dict[int, Tuple[int, ...]] = {}
        self.block_of: Dict[int, int] = {}           # hash -> block

    # -- pool ----------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def _allocate(self) -> int:
        if not self.free:
            raise MemoryError("no free block")
        b, _ = self.free.popitem(last=False)
        if b in self.hash_of:  # handed out again: its cached content goes away
            h = self.hash_of.pop(b)
            self.tokens_of.pop(b)
            if self.block_of.get(h) == b:
                del self.block_of[h]
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free[b] = None

    # -- sequences -------------------------------------------------------------------
    def add_sequence(self, seq: int, prompt: Optional[Sequence[int]] = None) -> int:
        """New sequence; with a prompt, reuse its longest cached prefix of full blocks.
        Returns the number of prompt tokens already in the cache."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        table: List[int] = []
        if prompt is not None:
            bs = self.block_size
            for i, h in enumerate(chunk_hashes(prompt, bs)):
                b = self.block_of.get(h)
                if b is None or self.tokens_of[b] != tuple(int(t) for t in prompt[i * bs:(i + 1) * bs]):
                    break
                if self.ref[b] == 0:
                    del self.free[b]
                self.ref[b] += 1
                table.append(b)
        self.tables[seq] = table
        self.lens[seq] = len(table) * self.block_size
        return self.lens[seq]

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Room for n more tokens: returns their slots (block * block_size + offset)
        and the (src, dst) block copies to run before writing them."""
        table, bs = self.tables[seq], self.block_size
        length = self.lens[seq]
        cow = n > 0 and length % bs != 0 and self.ref[table[-1]] > 1
        fresh = -(-(length + n) // bs) - (-(-length // bs)) + (1 if cow else 0)
        if fresh > len(self.free):  # nothing changes when the pool cannot hold the tokens
            raise MemoryError(f"{fresh} blocks needed, {len(self.free)} free")
        slots, copies = [], []
        for _ in range(n):
            off = self.lens[seq] % bs
            if off == 0:
                table.append(self._allocate())
            elif self.ref[table[-1]] > 1:  # writing into a shared block: copy it first
                old = table[-1]
                new = self._allocate()
                copies.append((old, new))
                self.ref[old] -= 1
                table[-1] = new
            slots.append(table[-1] * bs + off)
            self.lens[seq] += 1
        return slots, copies

    def commit_prompt(self, seq: int, prompt: Sequence[int]) -> int:
        """Register the hashes of the sequence's full prompt blocks (after their
        K/V were written).  Returns how many blocks got a hash."""
        bs, table, added = self.block_size, self.tables[seq], 0
        full = min(len(prompt), self.lens[seq]) // bs
        for i, h in enumerate(chunk_hashes(prompt[:full * bs], bs)):
            b = table[i]
            if b in self.hash_of or h in self.block_of:
                continue
            self.hash_of[b] = h
            self.tokens_of[b] = tuple(int(t) for t in prompt[i * bs:(i + 1) * bs])
            self.block_of[h] = b
            added += 1
        return added

    def free_sequence(self, seq: int) -> None:
        for b in reversed(self.tables.pop(seq)):
            self._release(b)
        del self.lens[seq]

    # -- queries ----------------------------------------------------------------------
    def block_table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def context_len(self, seq: int) -> int:
        return self.lens[seq]

    def refcount(self, b: int) -> int:
        return self.ref[b]

    def free_order(self) -> List[int]:
        return list(self.free)
