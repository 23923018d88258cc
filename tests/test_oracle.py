"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the fact it checks.  None of them re-types the oracle's
formula: the references are a NumPy dense attention on logical (unpaged) K/V,
closed forms, the pages' worked byte counts, library decoders, and invariants
(placement, chunking, caching) that hold for the exact result.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import workloads
from workloads.gen import (INT32_MAX, build_paged, make_chunked_case, make_cow_case, make_decode_case, new_pool,
                           reblock, write_tokens)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dec(case):
    return oracle.decode(case.query, case.pool.key_cache, case.pool.value_cache, case.block_tables,
                         case.context_lens, case.num_kv_heads, case.block_size, case.scale, case.dtype)


# --- worked example printed on the pages -------------------------------------------

def test_opt13b_kv_bytes_worked_example():
    """Page 1, section on why decoding is slow: OPT-13B needs 800 KB of KV per
    token (2 x 5120 x 40 layers x 2 B) and 1.6 GB for a 2048-token request."""
    g = json.load(open(os.path.join(GOLDEN, "opt13b_kv_bytes.json")))
    heads, head_dim = 40, 128
    assert heads * head_dim == g["hidden_size"]
    per_tok = oracle.kv_bytes_per_token(g["num_layers"], heads, head_dim, g["bytes_per_element"])
    assert per_tok == g["printed_per_token_bytes_binary"] == 800 * 1024
    per_req = per_tok * g["request_tokens"]
    assert per_req == g["printed_per_request_bytes"]
    assert round(per_req / 2**30, 1) == 1.6  # printed "1.6GB"
    # the generator's byte accounting agrees with the oracle's
    assert workloads.kv_bytes_per_token(40, 40, 128, 2) == per_tok


def test_block_bytes_formula():
    """Page 2, section 1.3: one layer's block = 2 x block_size x kv heads x head size x bytes."""
    assert oracle.kv_bytes_per_block(16, 40, 128, 2) == 327680
    # a block holds block_size tokens of one layer
    assert oracle.kv_bytes_per_block(16, 40, 128, 2) == 16 * oracle.kv_bytes_per_token(1, 40, 128, 2)
    pool = new_pool("f16", 10, 40, 128, 16)
    assert 2 * pool.block_bytes == oracle.kv_bytes_per_block(16, 40, 128, 2)


def test_two_token_closed_form():
    """Scores 0 and ln 2 give weights 1/3, 2/3 (golden fixture)."""
    g = json.load(open(os.path.join(GOLDEN, "two_token_closed_form.json")))
    D = g["head_dim"]
    pool = new_pool("f32", 4, 1, D, 16)
    k = torch.tensor(g["K"], dtype=torch.float32).reshape(2, 1, D)
    v = torch.tensor(g["V"], dtype=torch.float32).reshape(2, 1, D)
    write_tokens(pool, np.array([2 * 16 + 0, 2 * 16 + 1]), k, v)
    bt = np.array([[2]], dtype=np.int32)
    q = torch.tensor(g["q"], dtype=torch.float32).reshape(1, 1, D)
    out = oracle.decode(q, pool.key_cache, pool.value_cache, bt, np.array([2], np.int32), 1, 16, math.log(2.0),
                        "f32")
    np.testing.assert_allclose(out[0, 0], g["expected_out"], rtol=0, atol=g["tolerance"])


# --- decoders ----------------------------------------------------------------------

def test_f16_decoder_all_patterns():
    """The oracle's binary16 decoder equals NumPy's for all 65536 bit patterns."""
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.decode_elements(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_decoder_all_patterns():
    """The oracle's bfloat16 decoder equals torch's widening for all patterns."""
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.decode_elements(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f16_decoder_landmarks():
    vals = {0x3C00: 1.0, 0x0001: 2.0**-24, 0x0400: 2.0**-14, 0x7BFF: 65504.0, 0xC000: -2.0, 0x3555: 0.333251953125}
    bits = np.array(list(vals), dtype=np.uint16)
    assert list(oracle.decode_elements(bits, "f16")) == list(vals.values())


# --- brute force on tiny inputs --------------------------------------------------------

def _brute(case):
    p = case.paged
    return brute.decode(case.query, p.logical_k, p.logical_v, p.cu_tokens, case.scale)


def test_tiny_config_matches_brute_force():
    """Workload 1 (4 seqs, ctx 1/7/16/33, MHA, d64, fp32, 32-block pool)."""
    case = workloads.config_decode(1)
    assert case.num_blocks == 32 and case.max_blocks_per_seq == 3
    np.testing.assert_allclose(_dec(case), _brute(case), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("D", [64, 128])
def test_random_small_matches_brute_force(dtype, G, D):
    rng = np.random.default_rng([7, G, D, len(dtype)])
    S = int(rng.integers(1, 7))
    ctx = rng.integers(1, 71, size=S)
    Hkv = int(rng.integers(1, 4))
    case = make_decode_case([11, G, D], dtype, ctx, Hkv * G, Hkv, D)
    np.testing.assert_allclose(_dec(case), _brute(case), rtol=1e-12, atol=1e-12)


# --- invariants -----------------------------------------------------------------------

def _replace(case, rng):
    """Move every used block to a new random physical place."""
    old = case.pool
    NB = old.num_blocks
    perm = rng.permutation(NB)  # old block b -> new block perm[b]
    k = torch.empty_like(old.key_cache)
    v = torch.empty_like(old.value_cache)
    k[torch.from_numpy(perm)] = old.key_cache
    v[torch.from_numpy(perm)] = old.value_cache
    bt = case.block_tables.copy()
    used = bt != INT32_MAX
    bt[used] = perm[bt[used]]
    return k, v, bt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_placement_invariance_bitwise(dtype):
    """Page 1, blockwise-attention figure: physical placement does not change the result."""
    case = make_decode_case([3, 1], dtype, [5, 16, 17, 64, 100], 8, 2, 64)
    a = _dec(case)
    for seed in range(3):
        k, v, bt = _replace(case, np.random.default_rng(seed))
        b = oracle.decode(case.query, k, v, bt, case.context_lens, 2, 16, case.scale, dtype)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [8, 32])
def test_block_size_invariance(dtype, bs):
    """Page 1, paging section: a block is only the storage unit of the KV cache.  The
    same tokens stored in blocks of 8, 16 or 32 give the same attention bit for bit
    (the tokens are gathered back in logical order before any arithmetic), and that
    attention is the dense one on the logical K/V."""
    case = make_decode_case([3, 2], dtype, [1, 7, 8, 9, 16, 17, 31, 33, 100], 8, 2, 64)
    a = _dec(case)
    p = reblock(case.paged, bs, np.random.default_rng(bs))
    assert p.pool.key_cache.shape[2] == bs and p.pool.value_cache.shape[3] == bs
    b = oracle.decode(case.query, p.pool.key_cache, p.pool.value_cache, p.block_tables, p.context_lens, 2, bs,
                      case.scale, dtype)
    assert np.array_equal(a, b)
    ref = brute.decode(case.query, p.logical_k, p.logical_v, p.cu_tokens, case.scale)
    np.testing.assert_allclose(b, ref.reshape(b.shape), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bs", [8, 32])
def test_chunked_block_size_invariance(bs):
    """The chunked rows are the same for every block size of the pool."""
    case = make_chunked_case([5, bs], "bf16", [0, 9, 40], [7, 16, 33], 4, 2, 64)
    pool = case.paged.pool.clone()
    oracle.reshape_and_cache(case.new_key, case.new_value, pool.key_cache, pool.value_cache, case.slot_mapping,
                             "bf16")
    a = oracle.chunked(case.query, case.cu_q_lens, pool.key_cache, pool.value_cache, case.paged.block_tables,
                       case.paged.context_lens, 2, 16, case.scale, "bf16")
    p = reblock(case.paged, bs, np.random.default_rng(bs))
    # the chunk's own tokens go in through the cache write, at their slots in the new layout
    pend = np.nonzero(p.pending)[0]
    oracle.reshape_and_cache(p.logical_k[torch.from_numpy(pend)], p.logical_v[torch.from_numpy(pend)],
                             p.pool.key_cache, p.pool.value_cache, p.token_slots[pend], "bf16")
    b = oracle.chunked(case.query, case.cu_q_lens, p.pool.key_cache, p.pool.value_cache, p.block_tables,
                       p.context_lens, 2, bs, case.scale, "bf16")
    assert np.array_equal(a, b)


def test_ctx_one_is_first_value_exactly():
    """A single score has softmax weight 1, so o = V_0 exactly."""
    case = make_decode_case([4], "bf16", [1, 1, 1], 8, 2, 128)
    out = _dec(case)
    v0 = case.paged.logical_v.to(torch.float64).numpy()  # one token per sequence
    for s in range(3):
        for h in range(8):
            assert np.array_equal(out[s, h], v0[s, h // 4])


def test_ctx_zero_gives_zero():
    case = make_decode_case([5], "f16", [0, 3], 2, 1, 64)
    out = _dec(case)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out[1]))


def test_zero_query_gives_mean_of_values():
    """q = 0 makes every score 0: uniform weights, o = mean of V."""
    case = make_decode_case([6], "f16", [3, 40, 77], 4, 2, 128)
    case.query.zero_()
    out = _dec(case)
    p = case.paged
    vv = p.logical_v.to(torch.float64).numpy()
    for s in range(3):
        mean = vv[p.cu_tokens[s]:p.cu_tokens[s + 1]].mean(axis=0)
        for h in range(4):
            np.testing.assert_allclose(out[s, h], mean[h // 2], rtol=0, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dominant_key_selects_its_value(dtype):
    """A key whose score beats the rest by > 40 gets weight 1 - O(e^-40): o = V_t*.
    Targets sit at block edges, the first and the last token; each head of a group
    has its own target, which catches single-token addressing errors."""
    G, Hkv, D, BS = 4, 2, 64, 16
    ctx = [17, 33, 48, 70]
    case = make_decode_case([8], dtype, ctx, G * Hkv, Hkv, D, BS)
    p = case.paged
    q = case.query.to(torch.float64)
    targets = {}
    k_log = p.logical_k.clone()
    for s, n in enumerate(ctx):
        for g in range(Hkv):
            cands = [0, 15, 16, n - 1, min(31, n - 1)]
            for j in range(G):
                h = g * G + j
                t = cands[(s + j) % len(cands)]
                targets[(s, h)] = t
    # one target token per (s, h) needs a key aligned with q_h only: make the
    # query heads of a group orthogonal, then K_t = c * q_h
    qn = torch.zeros_like(q)
    for s in range(len(ctx)):
        for h in range(G * Hkv):
            qn[s, h, h % G * 8:(h % G) * 8 + 8] = 1.0
    case.query.copy_(qn.to(case.query.dtype))
    k_log.zero_()
    for (s, h), t in targets.items():
        g = h // G
        row = p.cu_tokens[s] + t
        k_log[row, g] += (qn[s, h] * 64.0).to(k_log.dtype)
    pool = case.pool
    write_tokens(pool, p.token_slots, k_log, p.logical_v)
    out = _dec(case)
    vv = p.logical_v.to(torch.float64).numpy()
    for (s, h), t in targets.items():
        # score of the target: scale * 64 * |q_h|^2 = 0.125 * 64 * 8 = 64; all others 0
        ref = vv[p.cu_tokens[s] + t, h // G]
        np.testing.assert_allclose(out[s, h], ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_gqa_equals_mha_with_repeated_kv_heads():
    """Page 3, section 4.1: a query group shares one K/V head; GQA(G) equals MHA
    whose kv heads are the shared head repeated G times (contiguous groups)."""
    G, Hkv, D = 4, 2, 64
    case = make_decode_case([9], "bf16", [9, 31, 50], G * Hkv, Hkv, D)
    a = _dec(case)
    k = case.pool.key_cache.repeat_interleave(G, dim=1).contiguous()
    v = case.pool.value_cache.repeat_interleave(G, dim=1).contiguous()
    b = oracle.decode(case.query, k, v, case.block_tables, case.context_lens, G * Hkv, 16, case.scale, "bf16")
    assert np.array_equal(a, b)


def test_chunked_rows_equal_dense_causal_rows():
    """Chunked prefill rows equal the rows of dense causal attention over the
    whole sequence (page 3, sections 3.1 and 4.6)."""
    rng = np.random.default_rng(12)
    n, L, Hq, Hkv, D = 45, 13, 4, 2, 64
    p = build_paged(rng, "bf16", Hkv, D, 16, [n], [n])
    q = torch.from_numpy(rng.standard_normal((L, Hq, D), dtype=np.float32)).to(torch.bfloat16)
    cu = np.array([0, L], np.int32)
    out = oracle.chunked(q, cu, p.pool.key_cache, p.pool.value_cache, p.block_tables, p.context_lens, Hkv, 16,
                         0.125, "bf16")
    ref = brute.chunk_rows(q, p.logical_k, p.logical_v, 0.125)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # the same rows split into chunks 3 + 4 + 6 give bitwise the same result
    parts, start = [], n - L
    for size in (3, 4, 6):
        cu_i = np.array([0, size], np.int32)
        qi = q[start - (n - L): start - (n - L) + size]
        parts.append(oracle.chunked(qi, cu_i, p.pool.key_cache, p.pool.value_cache, p.block_tables,
                                    np.array([start + size], np.int32), Hkv, 16, 0.125, "bf16"))
        start += size
    assert np.array_equal(np.concatenate(parts), out)


def test_chunk_of_one_equals_decode():
    case = make_decode_case([13], "f16", [20, 47], 4, 4, 64)
    cu = np.array([0, 1, 2], np.int32)
    out = oracle.chunked(case.query, cu, case.pool.key_cache, case.pool.value_cache, case.block_tables,
                         case.context_lens, 4, 16, case.scale, "f16")
    assert np.array_equal(out, _dec(case))


def test_incremental_cache_equals_recompute():
    """Page 3, sections 3.1 and 3.4: decoding with a cache (append the new K/V,
    then attend) gives, token by token, what recomputing from scratch gives."""
    rng = np.random.default_rng(14)
    n, Hq, Hkv, D, BS = 40, 4, 2, 64, 16
    qs = torch.from_numpy(rng.standard_normal((n, Hq, D), dtype=np.float32)).to(torch.float16)
    ks = torch.from_numpy(rng.standard_normal((n, Hkv, D), dtype=np.float32)).to(torch.float16)
    vs = torch.from_numpy(rng.standard_normal((n, Hkv, D), dtype=np.float32)).to(torch.float16)
    pool = new_pool("f16", 8, Hkv, D, BS)
    bt = np.array([[6, 1, 4]], dtype=np.int32)
    dense = brute.causal(qs, ks, vs, 0.125)
    for t in range(n):
        slot = np.array([bt[0, t // BS] * BS + t % BS], np.int64)
        oracle.reshape_and_cache(ks[t:t + 1], vs[t:t + 1], pool.key_cache, pool.value_cache, slot, "f16")
        o = oracle.decode(qs[t:t + 1], pool.key_cache, pool.value_cache, bt, np.array([t + 1], np.int32), Hkv,
                          BS, 0.125, "f16")
        np.testing.assert_allclose(o[0], dense[t], rtol=1e-12, atol=1e-12)


# --- writes -----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_reshape_and_cache_round_trip(dtype):
    """Tokens written through slot_mapping read back bit for bit; every other
    byte of the pool is unchanged; negative slots write nothing."""
    rng = np.random.default_rng(15)
    NB, H, D, BS, n = 12, 3, 64, 16, 40
    pool = new_pool(dtype, NB, H, D, BS)
    before_k = pool.key_cache.clone()
    before_v = pool.value_cache.clone()
    slots = rng.choice(NB * BS, size=n, replace=False).astype(np.int64)
    slots[3] = -1
    k = torch.from_numpy(rng.standard_normal((n, H, D), dtype=np.float32)).to(workloads.DTYPES[dtype][0])
    v = torch.from_numpy(rng.standard_normal((n, H, D), dtype=np.float32)).to(workloads.DTYPES[dtype][0])
    oracle.reshape_and_cache(k, v, pool.key_cache, pool.value_cache, slots, dtype)
    ib = lambda x: x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32)  # noqa: E731
    written = np.zeros((NB, BS), dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), BS)
        written[b, o] = True
        assert torch.equal(ib(pool.key_cache[b, :, o, :]), ib(k[i]))
        assert torch.equal(ib(pool.value_cache[b, :, :, o]), ib(v[i]))
    untouched = torch.from_numpy(~written)
    assert torch.equal(ib(pool.key_cache.permute(0, 2, 1, 3)[untouched]),
                       ib(before_k.permute(0, 2, 1, 3)[untouched]))
    assert torch.equal(ib(pool.value_cache.permute(0, 3, 1, 2)[untouched]),
                       ib(before_v.permute(0, 3, 1, 2)[untouched]))


def test_reshape_and_cache_rejects_out_of_pool_slot():
    pool = new_pool("bf16", 2, 1, 64, 16)
    k = torch.zeros(1, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(oracle.OracleError):
        oracle.reshape_and_cache(k, k, pool.key_cache, pool.value_cache, np.array([32]), "bf16")


def test_copy_blocks_copies_whole_blocks_in_every_layer():
    rng = np.random.default_rng(16)
    L, NB = 3, 10
    ks = [torch.from_numpy(rng.standard_normal((NB, 2, 16, 64), dtype=np.float32)).to(torch.bfloat16)
          for _ in range(L)]
    vs = [torch.from_numpy(rng.standard_normal((NB, 2, 64, 16), dtype=np.float32)).to(torch.bfloat16)
          for _ in range(L)]
    before_k = [x.clone() for x in ks]
    before_v = [x.clone() for x in vs]
    pairs = np.array([[1, 7], [4, 2], [1, 9]], dtype=np.int64)
    oracle.copy_blocks(ks, vs, pairs, "bf16")
    dst = set(pairs[:, 1])
    for layer in range(L):
        for s, d in pairs:
            assert torch.equal(ks[layer][d].view(torch.int16), before_k[layer][s].view(torch.int16))
            assert torch.equal(vs[layer][d].view(torch.int16), before_v[layer][s].view(torch.int16))
        for b in range(NB):
            if b not in dst:
                assert torch.equal(ks[layer][b].view(torch.int16), before_k[layer][b].view(torch.int16))
                assert torch.equal(vs[layer][b].view(torch.int16), before_v[layer][b].view(torch.int16))


def test_copy_on_write_parallel_sampling():
    """Page 1, copy-on-write paragraph: samples share the prompt's blocks with a
    refcount; a writer copies the shared partial block first (count drops by one)
    and the last sharer writes in place.  After the copies and the private writes
    each sample sees prompt ++ its own tokens, and shared blocks are unchanged."""
    c = make_cow_case([17], num_prompts=3, samples_per_prompt=4, prompt_blocks=4, max_private=40,
                      num_q_heads=8, num_kv_heads=2, head_dim=64,
                      private_lens=[0, 5, 17, 1, 3, 0, 0, 0, 2, 9, 4, 30])
    # copies: prompt 0 has 3 writers of 4 sharers -> 3 copies; prompt 1: 1 writer
    # -> 1 copy; prompt 2: 4 writers -> 3 copies and one in-place write
    assert len(c.block_mapping) == 7
    srcs = list(dict.fromkeys(c.block_mapping[:, 0].tolist()))  # the prompts' shared last blocks
    assert [int(c.refcount[b]) for b in srcs] == [1, 3, 1]
    pool = c.pool.clone()
    shared_before_k = pool.key_cache[torch.from_numpy(c.shared_blocks)].clone()
    oracle.copy_blocks([pool.key_cache], [pool.value_cache], c.block_mapping, "bf16")
    oracle.reshape_and_cache(c.new_key, c.new_value, pool.key_cache, pool.value_cache, c.slot_mapping, "bf16")
    out = oracle.decode(c.query, pool.key_cache, pool.value_cache, c.block_tables, c.context_lens, 2, 16,
                        c.scale, "bf16")
    for s in range(c.num_seqs):
        k, v = c.logical(s)
        ref = brute.attention_rows(c.query[s], k, v, c.scale)
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-12)
    # prompt blocks that are still shared and were not the in-place target keep their bytes
    inplace = {srcs[2]}
    assert int(c.block_tables[2 * 4 + 3, 3]) == srcs[2]
    for i, b in enumerate(c.shared_blocks):
        if int(b) not in inplace:
            assert torch.equal(pool.key_cache[b].view(torch.int16), shared_before_k[i].view(torch.int16))


def test_cow_workload_shape():
    c = workloads.config_cow()
    assert c.num_seqs == 128 and c.max_blocks_per_seq == 80
    assert (c.prompt_lens >= 1024 - 15).all() and (c.prompt_lens <= 1023).all()
    assert (c.private_lens >= 0).all() and (c.private_lens <= 256).all()
    # one copy per writing sample, except the 8th writer of a prompt writes in place
    writers = (c.private_lens > 0).reshape(16, 8).sum(axis=1)
    assert len(c.block_mapping) == int(np.minimum(writers, 7).sum())


def test_oracle_reports_bad_block_id():
    case = make_decode_case([18], "f32", [20], 1, 1, 64)
    bt = case.block_tables.copy()
    bt[0, 1] = case.num_blocks
    with pytest.raises(oracle.OracleError):
        oracle.decode(case.query, case.pool.key_cache, case.pool.value_cache, bt, case.context_lens, 1, 16, 1.0,
                      "f32")


def test_thread_count_does_not_change_results():
    """The oracle's parallel loops give each (sequence, kv head) row to one thread: one
    thread and all threads return the same bits (the benchmark times both)."""
    c = make_decode_case([40], "bf16", [1, 17, 100, 333, 64], 8, 2, 128)
    args = (c.query, c.pool.key_cache, c.pool.value_cache, c.block_tables, c.context_lens, 2, 16, c.scale, "bf16")
    many = oracle.max_threads()
    try:
        oracle.set_threads(1)
        one = oracle.decode(*args)
    finally:
        oracle.set_threads(many)
    assert np.array_equal(one, oracle.decode(*args))
