"""Seeded beam-search workload: an operation script for a paged-KV block manager
plus the K/V each token writes.  Input generation only: no attention arithmetic
and no block management here -- the script says what happens to which sequence,
a manager decides where it goes.

Shape ("每生成一个字都要把全部权重读一遍：从 vLLM 看 LLM 推理提速", paging section:
beam-search branches share a prefix and copy a block only where they fork;
"现代 LLM 推理引擎剖析", section 2.2: prompts with a long common prefix share its
cached blocks): P prompts with a common system prefix and their own tails; each
starts one beam; every step each live beam appends one token; then beams fork
(a copy of a beam, forked at its current length -- arbitrary positions, since
beams have different histories) and the weakest are dropped, keeping at most
`width` beams per prompt and at least one.

K and V of a token depend on its position and its token id only, so sequences
with equal prefixes hold equal K/V there (what makes sharing and prefix caching
exact): kv[layer][0 or 1][position][token id] -> [Hkv, D].
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np
import torch


@dataclass
class BeamScript:
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    scale: float
    vocab: int
    prompts: List[List[int]]
    ops: List[tuple]            # ("add", seq, prompt index), ("append", seq, [token ids]),
                                # ("fork", parent, child), ("free", seq), ("commit", seq),
                                # ("decode", checkpoint index)
    k_table: torch.Tensor       # [layers, max_pos, vocab, Hkv, D], storage dtype
    v_table: torch.Tensor
    queries: List[torch.Tensor]  # per decode checkpoint: [max_live, Hq, D]


def make_beam_script(seed=(265, 6), num_prompts: int = 4, system_len: int = 70, tail_len=(20, 90),
                     steps: int = 40, width: int = 4, fork_p: float = 0.35, num_layers: int = 4,
                     num_q_heads: int = 8, num_kv_heads: int = 2, head_dim: int = 128, dtype: str = "bf16",
                     vocab: int = 32, decode_every: int = 10) -> BeamScript:
    rng = np.random.default_rng(list(seed))
    system = rng.integers(0, vocab, size=system_len).tolist()
    prompts = [system + rng.integers(0, vocab, size=int(rng.integers(tail_len[0], tail_len[1] + 1))).tolist()
               for _ in range(num_prompts)]
    max_pos = max(len(p) for p in prompts) + steps + 1
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    shape = (num_layers, max_pos, vocab, num_kv_heads, head_dim)
    k_table = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(tdt)
    v_table = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(tdt)

    ops: List[tuple] = []
    beams: List[List[int]] = []   # per prompt: live sequence ids
    next_id = 0
    for pi in range(num_prompts):
        ops.append(("add", next_id, pi))
        ops.append(("commit", next_id))
        beams.append([next_id])
        next_id += 1
    queries = []
    for step in range(steps):
        for group in beams:
            for s in group:
                ops.append(("append", s, [int(rng.integers(0, vocab))]))
        for group in beams:
            for s in list(group):
                if len(group) < width and rng.random() < fork_p:
                    ops.append(("fork", s, next_id))
                    group.append(next_id)
                    next_id += 1
            while len(group) > 1 and rng.random() < 0.25:
                s = group.pop(int(rng.integers(0, len(group))))
                ops.append(("free", s))
        if (step + 1) % decode_every == 0:
            live = sum(len(g) for g in beams)
            queries.append(torch.from_numpy(
                rng.standard_normal((live, num_q_heads, head_dim), dtype=np.float32)).to(tdt))
            ops.append(("decode", len(queries) - 1))
    return BeamScript(num_layers, num_q_heads, num_kv_heads, head_dim, dtype, 1.0 / np.sqrt(head_dim), vocab,
                      prompts, ops, k_table, v_table, queries)
