"""GPU parity of paged_attention_decode against the fp64 oracle, through the C ABI.

Sizes span several blocks, several partitions and ragged tails; every case
prints what it runs before it launches anything."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_265_amd as pkv
from workloads.gen import INT32_MAX, make_decode_case, write_tokens

from helpers import bits, check_close, dev, oracle_decode_case

pytestmark = pytest.mark.gpu


def run_decode(case, partition_size=0, bt=None, kc=None, vc=None, query=None, inner_loop=None, ring=0):
    """paged_attention_decode, or with inner_loop / ring given the test hook that forces
    the inner loop ("valu" / "mfma") or a two-tile prefetch ring."""
    say(f"decode {case.label or ''} S={case.num_seqs} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} {case.dtype} part={partition_size} max_ctx={int(case.context_lens.max(initial=0))} "
        f"loop={inner_loop or 'auto'} ring={ring}")
    q = dev(case.query if query is None else query)
    kc = dev(case.pool.key_cache) if kc is None else kc
    vc = dev(case.pool.value_cache) if vc is None else vc
    out = torch.full_like(q, float("nan"))
    bt_d, cl_d = dev(case.block_tables if bt is None else bt), dev(case.context_lens)
    if inner_loop is None and ring == 0:
        pkv.paged_attention_decode(out, q, kc, vc, bt_d, cl_d, case.scale, partition_size=partition_size)
    else:
        pkv.decode_variant(out, q, kc, vc, bt_d, cl_d, case.scale, partition_size=partition_size,
                           inner_loop=inner_loop or "auto", ring=ring)
    torch.cuda.synchronize()
    return out


def say(msg):
    print(msg, flush=True)


CASES = [
    # (dtype, G, Hkv, D, context lengths)
    ("f32", 1, 4, 64, [1, 7, 16, 33]),
    ("f32", 1, 2, 128, [17, 200, 513, 1]),
    ("f32", 4, 2, 64, [100, 31, 600]),
    ("f16", 1, 4, 128, [130, 16, 1000, 515]),
    ("f16", 2, 3, 64, [45, 300, 700]),
    ("bf16", 3, 2, 128, [33, 520, 1100]),
    ("bf16", 4, 8, 128, [1, 15, 16, 17, 512, 513, 1024, 1500]),
    ("f16", 4, 2, 64, [77, 1030, 9]),
    ("bf16", 5, 2, 128, [250, 700]),
    ("bf16", 8, 2, 64, [64, 900]),
    ("f16", 16, 1, 128, [640, 19]),
    ("bf16", 32, 1, 128, [2000, 511, 3]),
    ("bf16", 40, 1, 64, [300, 1200]),
    ("f16", 20, 2, 128, [1, 33, 4000, 250]),    # 32-head P.V loop with the second head tile partly used
    ("bf16", 17, 1, 64, [16, 47, 2100]),
    ("f16", 32, 2, 64, [5000, 3, 600]),
]


@pytest.mark.parametrize("dtype,G,Hkv,D,ctx", CASES)
def test_decode_matches_oracle(dtype, G, Hkv, D, ctx):
    case = make_decode_case([21, G, D, len(ctx)], dtype, ctx, G * Hkv, Hkv, D)
    ref = oracle_decode_case(case)
    out = run_decode(case)
    check_close(out, ref, dtype, f"{dtype} G={G}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 1), ("bf16", 2), ("f16", 32)])
def test_both_inner_loops_match_oracle(path, dtype, G):
    Hkv = 2 if G < 32 else 1
    case = make_decode_case([22, G], dtype, [3, 700, 1025, 64], G * Hkv, Hkv, 128)
    check_close(run_decode(case, inner_loop=path), oracle_decode_case(case), dtype, f"{path} {dtype} G={G}")


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 1), ("f32", 2), ("bf16", 32)])
def test_partition_size_invariance(dtype, G):
    """Partitions of 1 to 7, 32 or 128 blocks, or the balanced split, agree with the oracle
    (every remainder of the fixed-partition prefetch ring)."""
    Hkv = 2 if G < 32 else 1
    case = make_decode_case([23, G], dtype, [1, 40, 333, 1200, 2048], G * Hkv, Hkv, 128,
                            max_blocks_per_seq=128)
    ref = oracle_decode_case(case)
    outs = []
    for part in (16, 32, 48, 64, 80, 96, 112, 512, 2048, 0):
        out = run_decode(case, partition_size=part)
        check_close(out, ref, dtype, f"partition {part}")
        outs.append(out)


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 1), ("bf16", 32), ("f32", 1)])
def test_placement_invariance_and_determinism_bitwise(dtype, G):
    """Moving blocks to other physical places changes nothing, bit for bit; so does running again."""
    Hkv = 2 if G < 32 else 1
    case = make_decode_case([24, G], dtype, [5, 300, 1000, 17], G * Hkv, Hkv, 64)
    a = run_decode(case)
    b = run_decode(case)
    assert torch.equal(bits(a), bits(b))
    rng = np.random.default_rng(5)
    perm = rng.permutation(case.num_blocks)
    k = torch.empty_like(case.pool.key_cache)
    v = torch.empty_like(case.pool.value_cache)
    k[torch.from_numpy(perm)] = case.pool.key_cache
    v[torch.from_numpy(perm)] = case.pool.value_cache
    bt = case.block_tables.copy()
    used = bt != INT32_MAX
    bt[used] = perm[bt[used]]
    c = run_decode(case, bt=bt, kc=dev(k), vc=dev(v))
    assert torch.equal(bits(a), bits(c))


@pytest.mark.parametrize("part", [0, 64])
@pytest.mark.parametrize("dtype,G,Hkv", [("bf16", 4, 8), ("f16", 8, 2), ("bf16", 32, 1), ("f16", 1, 4)])
def test_repeated_runs_are_bitwise_identical(part, dtype, G, Hkv):
    """Eight runs on the same buffers give the same bits.  Outputs near a rounding
    midpoint expose any run-to-run wobble in the fp32 sums (a build of the 16-head
    matrix-core loop once showed a few such flips per run while staying within the
    parity tolerance)."""
    case = make_decode_case([32, G], dtype, [1, 8, 15, 16, 17, 24, 32, 512, 520, 1500], G * Hkv, Hkv, 128)
    q = dev(case.query)
    kc, vc = dev(case.pool.key_cache), dev(case.pool.value_cache)
    bt, cl = dev(case.block_tables), dev(case.context_lens)
    say(f"repeat {dtype} G={G} Hkv={Hkv} part={part}")
    first = None
    for _ in range(8):
        out = torch.full_like(q, float("nan"))
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, case.scale, partition_size=part)
        torch.cuda.synchronize()
        if first is None:
            first = bits(out).clone()
        else:
            assert torch.equal(bits(out), first)


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 1), ("bf16", 32), ("f32", 1), ("bf16", 2)])
def test_context_of_one_returns_first_value_exactly(dtype, G):
    Hkv = 2 if G < 32 else 1
    case = make_decode_case([25, G], dtype, [1, 1, 1], G * Hkv, Hkv, 128)
    out = run_decode(case).cpu()
    v0 = case.paged.logical_v  # one token per sequence
    for s in range(3):
        for h in range(G * Hkv):
            assert torch.equal(bits(out[s, h]), bits(v0[s, h // G]))


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 1), ("f32", 1), ("bf16", 32)])
def test_empty_context_gives_zeros(dtype, G):
    Hkv = 2 if G < 32 else 1
    case = make_decode_case([26, G], dtype, [0, 20, 0], G * Hkv, Hkv, 64, max_blocks_per_seq=4)
    out = run_decode(case, partition_size=16)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    check_close(out, oracle_decode_case(case), dtype, "ctx 0")


@pytest.mark.parametrize("dtype,G,D", [("bf16", 4, 128), ("f16", 1, 64), ("bf16", 32, 128), ("f32", 1, 64),
                                       ("bf16", 2, 128)])
def test_dominant_key_probes(dtype, G, D):
    """Each (sequence, head) gets one key whose score beats the rest by ~64 (log e):
    the output must be that token's V (to the storage precision).  Targets sit on
    block edges, partition edges (partition 64), the first and the last token,
    which catches a single dropped or shifted token that tolerance parity cannot."""
    Hkv = 2 if G < 32 else 1
    ctx = [17, 64, 65, 130, 300]
    case = make_decode_case([27, G, D], dtype, ctx, G * Hkv, Hkv, D)
    p = case.paged
    q = torch.zeros(case.num_seqs, G * Hkv, D, dtype=torch.float64)
    k_log = torch.zeros_like(p.logical_k, dtype=torch.float64)
    per = max(1, D // max(G, 1))
    targets = {}
    for s, n in enumerate(ctx):
        cands = sorted({0, 15, 16, 63, 64, n - 1, n // 2} & set(range(n)))
        for h in range(G * Hkv):
            j = h % G
            lo = (j * per) % D
            q[s, h, lo:lo + min(per, 8)] = 1.0
            t = cands[(s * 7 + h) % len(cands)]
            targets[(s, h)] = t
    for (s, h), t in targets.items():
        k_log[p.cu_tokens[s] + t, h // G] += q[s, h] * (64.0 / (case.scale * float((q[s, h] ** 2).sum())))
    query = q.to(case.query.dtype)
    kl = k_log.to(p.logical_k.dtype)
    pool = case.pool.clone()
    write_tokens(pool, p.token_slots, kl, p.logical_v)
    ref = oracle.decode(query, pool.key_cache, pool.value_cache, case.block_tables, case.context_lens, Hkv, 16,
                        case.scale, dtype)
    vv = p.logical_v.to(torch.float64).numpy()
    for (s, h), t in targets.items():
        assert np.allclose(ref[s, h], vv[p.cu_tokens[s] + t, h // G], atol=1e-9), "probe construction"
    for part in (0, 64):
        out = run_decode(case, partition_size=part, kc=dev(pool.key_cache), vc=dev(pool.value_cache), query=query)
        check_close(out, ref, dtype, f"probe part={part}")
        o = out.cpu().to(torch.float64).numpy()
        step = 1e-6 if dtype == "f32" else (2.0 ** -8 if dtype == "bf16" else 2.0 ** -11)
        for (s, h), t in targets.items():
            target = vv[p.cu_tokens[s] + t, h // G]
            assert np.all(np.abs(o[s, h] - target) <= step * np.maximum(1.0, np.abs(target))), (s, h, t)


def test_nan_in_unused_slots_never_leaks():
    """Slots past each context and every unused block hold NaN: outputs stay finite."""
    case = make_decode_case([28], "bf16", [3, 18, 45, 77], 32, 8, 128)
    assert torch.isnan(case.pool.key_cache).any()
    out = run_decode(case)
    assert torch.isfinite(out).all()


def test_max_context_fills_every_table_entry():
    """context = max_blocks_per_seq * block_size (every table entry used)."""
    case = make_decode_case([29], "bf16", [64 * 16, 64 * 16 - 1], 8, 2, 128, max_blocks_per_seq=64)
    check_close(run_decode(case), oracle_decode_case(case), "bf16", "max ctx")


def test_streams_are_honoured():
    """A call on a side stream is ordered on that stream."""
    case = make_decode_case([30], "bf16", [700, 80], 8, 2, 128)
    s = torch.cuda.Stream()
    q = dev(case.query)
    kc, vc = dev(case.pool.key_cache), dev(case.pool.value_cache)
    bt, cl = dev(case.block_tables), dev(case.context_lens)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, case.scale)
    s.synchronize()
    check_close(out, oracle_decode_case(case), "bf16", "side stream")


@pytest.mark.parametrize("depth", ["2", "default"])
@pytest.mark.parametrize("dtype,G,Hkv,D,ctx", [
    ("bf16", 4, 1, 128, [50000]),               # one stream cut into pieces by every wave
    ("bf16", 4, 8, 128, [0, 3, 0, 900, 0]),     # empty contexts between live ones
    ("f16", 1, 2, 64, [1] * 40 + [5000]),       # many one-block streams, one long
    ("bf16", 32, 1, 128, [20000, 17, 4096]),
    ("bf16", 40, 2, 64, [3000, 33]),            # heads per kv head above one 32-head chunk
    ("f32", 2, 2, 64, [7000, 0, 16]),
    # more sequences than one round of in-wave loads: the start units come from the
    # prologue's scan (three rounds of 1024 sequences), empty contexts among them
    ("bf16", 4, 2, 128, [0 if i % 11 == 3 else 1 + (i * 37) % 200 for i in range(3000)]),
    ("f16", 1, 2, 64, [0] * 300 + [17]),
])
def test_balanced_split_edges(depth, dtype, G, Hkv, D, ctx):
    """The load-balanced schedule: streams split across many waves, empty streams,
    waves with no work, and both prefetch depths."""
    case = make_decode_case([34, G, len(ctx)], dtype, ctx, G * Hkv, Hkv, D)
    out = run_decode(case, partition_size=0, ring=2 if depth == "2" else 0)
    check_close(out, oracle_decode_case(case), dtype, f"split depth {depth}")
    for s, n in enumerate(ctx):
        if n == 0:
            assert torch.all(out[s] == 0)


@pytest.mark.parametrize("dtype,G,Hkv,ctx", [
    ("bf16", 4, 8, [32768, 5000]),     # few long streams: per-head merge, 2 groups
    ("f16", 1, 8, [20000]),            # ~128 pieces per stream: per-head merge, 8 groups
    ("bf16", 4, 8, [300] * 300),       # more streams than waves: per-stream merge, a workgroup per wave
    ("bf16", 4, 8, [300] * 60),        # fewer streams than waves: per-stream merge, a workgroup per stream
    ("bf16", 32, 1, [300] * 300),      # many MQA streams: per-stream merge of 32 heads, a workgroup per stream
    ("bf16", 32, 1, [40] * 1100),      # more MQA streams than waves: a workgroup per wave
    ("bf16", 32, 1, [20000, 30000, 9000, 25000]),  # 4 long MQA streams, 128 (stream, head) pairs: 8 groups
    ("bf16", 32, 1, [60000]),          # one long MQA stream: a quarter of a head per workgroup
])
def test_long_streams_and_all_split_merges(dtype, G, Hkv, ctx):
    """Every merge of the balanced split (per stream for many short streams, per head
    with two or eight groups for few long ones, per quarter head for one or two long
    sequences) against the oracle."""
    case = make_decode_case([47, G, len(ctx)], dtype, ctx, G * Hkv, Hkv, 128)
    check_close(run_decode(case), oracle_decode_case(case), dtype, f"long streams {ctx[:2]}")
