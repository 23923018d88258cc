"""GPU parity of paged_attention_mixed: one launch over a flattened batch of decode
tokens (one-row segments) and prefill chunks, through the C ABI.

Every row is compared with the oracle's chunked attention (a decode token is a
chunk of one row); prefill rows must equal paged_attention_chunked's bit for bit
(the same tile code runs them), decode rows agree with paged_attention_decode to
the tolerance.  Every case prints what it runs before it launches anything."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_265_amd as pkv
from workloads.gen import make_chunked_case, reblock

from helpers import bits, check_close, dev, vmax_of

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def write_chunks(case, paged=None):
    paged = case.paged if paged is None else paged
    kc, vc = dev(paged.pool.key_cache), dev(paged.pool.value_cache)
    pend = np.nonzero(paged.pending)[0]
    ti = torch.from_numpy(pend)
    pkv.reshape_and_cache(dev(paged.logical_k[ti].contiguous()), dev(paged.logical_v[ti].contiguous()), kc, vc,
                          dev(paged.token_slots[pend].copy()))
    return kc, vc


def oracle_rows(case, paged=None):
    paged = case.paged if paged is None else paged
    pool = paged.pool.clone()
    pend = np.nonzero(paged.pending)[0]
    ti = torch.from_numpy(pend)
    oracle.reshape_and_cache(paged.logical_k[ti], paged.logical_v[ti], pool.key_cache, pool.value_cache,
                             paged.token_slots[pend], case.dtype)
    return oracle.chunked(case.query, case.cu_q_lens, pool.key_cache, pool.value_cache, paged.block_tables,
                          paged.context_lens, case.num_kv_heads, pool.block_size, case.scale, case.dtype)


def run(case, fn, paged=None):
    paged = case.paged if paged is None else paged
    q_lens = np.diff(case.cu_q_lens)
    say(f"{fn.__name__} {case.dtype} bs={paged.pool.block_size} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} q_lens={q_lens.tolist()} ctx={paged.context_lens.tolist()}")
    kc, vc = write_chunks(case, paged)
    q = dev(case.query)
    out = torch.full_like(q, float("nan"))
    fn(out, q, dev(case.cu_q_lens), case.max_q_len, kc, vc, dev(paged.block_tables), dev(paged.context_lens),
       case.scale)
    torch.cuda.synchronize()
    return out


def decode_rows(case):
    """Query rows of the one-row segments."""
    q_lens = np.diff(case.cu_q_lens)
    return np.asarray(case.cu_q_lens[:-1])[q_lens == 1]


# (dtype, G, Hkv, D, cached tokens, query rows per segment): decode segments (one
# row) with short and long contexts, prefill chunks with and without cached
# prefixes, every decode inner loop (G 1, 2: vector ALU; 4-16: 16-head matrix
# cores; 17-32: 32-head matrix cores) and both head dims
CASES = [
    ("bf16", 4, 2, 128, [0, 700, 40, 2999, 15, 100], [1, 1, 64, 1, 33, 1]),
    ("f16", 1, 4, 128, [16, 5, 1200], [1, 40, 1]),
    ("bf16", 2, 2, 64, [300, 0, 77], [1, 20, 1]),
    ("bf16", 32, 1, 128, [4095, 200, 16383, 31], [1, 40, 1, 17]),
    ("f16", 8, 1, 64, [513, 1000], [1, 130]),
    ("bf16", 20, 2, 128, [1, 900, 60], [1, 1, 9]),
    ("bf16", 4, 8, 128, [5000, 3000, 1, 800, 50], [1, 1, 1, 1, 1]),      # decode only
    ("f16", 4, 2, 128, [0, 100], [50, 7]),                                 # prefill only
    # more segments than one round of in-wave loads: the decode start units come from
    # the prologue's scan
    ("bf16", 8, 1, 128, [40 + (i * 53) % 900 for i in range(300)] + [700, 0], [1] * 300 + [33, 64]),
    # at least eight (chunk, kv head) pairs for sure (the launch then gives each XCD whole
    # pairs; the cases above have fewer and take the tiles in launch order): eight kv
    # heads with one chunk, one kv head with eight chunks
    ("bf16", 4, 8, 128, [30, 200, 1000], [1, 40, 1]),
    ("bf16", 32, 1, 128, [100, 3000] + [50 + 37 * i for i in range(8)], [1, 1] + [9] * 8),
]


@pytest.mark.parametrize("dtype,G,Hkv,D,cached,q_lens", CASES)
def test_mixed_matches_oracle_and_the_separate_calls(dtype, G, Hkv, D, cached, q_lens):
    case = make_chunked_case([71, G, D, len(q_lens)], dtype, cached, q_lens, G * Hkv, Hkv, D)
    ref = oracle_rows(case)
    out = run(case, pkv.paged_attention_mixed)
    check_close(out, ref, dtype, f"mixed {dtype} G={G}", weights_vmax=vmax_of(case.paged.logical_v))
    sep = run(case, pkv.paged_attention_chunked)
    rows = decode_rows(case)
    pre = np.setdiff1d(np.arange(out.shape[0]), rows)
    if len(pre):
        assert torch.equal(bits(out[torch.from_numpy(pre)]), bits(sep[torch.from_numpy(pre)])), "prefill rows"
    # decode rows against the decode call on the same sequences
    if len(rows):
        seg = np.nonzero(np.diff(case.cu_q_lens) == 1)[0]
        kc, vc = write_chunks(case)
        q = dev(case.query[torch.from_numpy(rows)].contiguous())
        od = torch.full_like(q, float("nan"))
        pkv.paged_attention_decode(od, q, kc, vc, dev(case.paged.block_tables[seg].copy()),
                                   dev(case.paged.context_lens[seg].copy()), case.scale)
        torch.cuda.synchronize()
        check_close(out[torch.from_numpy(rows)], ref[rows], dtype, "decode rows of mixed")
        check_close(od, ref[rows], dtype, "decode call")


@pytest.mark.parametrize("bs", [8, 32])
def test_mixed_block_sizes(bs):
    case = make_chunked_case([72, bs], "bf16", [0, 700, 40, 2999], [1, 1, 64, 1], 8, 2, 128)
    p = reblock(case.paged, bs, np.random.default_rng(bs))
    ref = oracle_rows(case, p)
    out = run(case, pkv.paged_attention_mixed, p)
    check_close(out, ref, "bf16", f"mixed bs={bs}", weights_vmax=vmax_of(p.logical_v))
    # block size changes nothing: same bits as at 16
    out16 = run(case, pkv.paged_attention_mixed)
    assert torch.equal(bits(out), bits(out16))


def test_mixed_repeated_runs_are_bitwise_identical():
    case = make_chunked_case([73], "bf16", [4000, 300, 10, 2000], [1, 100, 1, 1], 32, 1, 128)
    first = bits(run(case, pkv.paged_attention_mixed)).clone()
    for _ in range(4):
        assert torch.equal(bits(run(case, pkv.paged_attention_mixed)), first)


def test_mixed_nan_slots_never_leak():
    """Slots past each context and unused blocks hold NaN; outputs stay finite."""
    case = make_chunked_case([74], "bf16", [3, 18, 45, 77, 0], [1, 1, 9, 1, 30], 16, 4, 128)
    assert torch.isnan(case.paged.pool.key_cache).any()
    out = run(case, pkv.paged_attention_mixed)
    assert torch.isfinite(out).all()
    check_close(out, oracle_rows(case), "bf16", "nan slots", weights_vmax=vmax_of(case.paged.logical_v))
