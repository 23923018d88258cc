"""GPU parity of paged_attention_chunked (causal chunked prefill over the paged pool)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_265_amd as pkv
from workloads.gen import make_chunked_case

from helpers import bits, check_close, dev, vmax_of

pytestmark = pytest.mark.gpu


def run_chunked(case, write_first=True):
    print(f"chunked {case.label} segs={case.num_segs} q_lens={np.diff(case.cu_q_lens).tolist()} "
          f"ctx={case.paged.context_lens.tolist()} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
          f"D={case.head_dim} {case.dtype}", flush=True)
    kc, vc = dev(case.paged.pool.key_cache), dev(case.paged.pool.value_cache)
    if write_first:
        pkv.reshape_and_cache(dev(case.new_key), dev(case.new_value), kc, vc, dev(case.slot_mapping))
    q = dev(case.query)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_chunked(out, q, dev(case.cu_q_lens), case.max_q_len, kc, vc, dev(case.paged.block_tables),
                                dev(case.paged.context_lens), case.scale)
    torch.cuda.synchronize()
    return out, kc, vc


def oracle_chunked(case):
    pool = case.paged.pool.clone()
    oracle.reshape_and_cache(case.new_key, case.new_value, pool.key_cache, pool.value_cache, case.slot_mapping,
                             case.dtype)
    return oracle.chunked(case.query, case.cu_q_lens, pool.key_cache, pool.value_cache, case.paged.block_tables,
                          case.paged.context_lens, case.num_kv_heads, case.block_size, case.scale, case.dtype), pool


CASES = [
    # dtype, G, Hkv, D, cached, q_lens
    ("bf16", 1, 2, 128, [0, 5, 40], [7, 16, 33]),
    ("f16", 4, 2, 64, [100, 0], [1, 50]),
    ("bf16", 4, 8, 128, [17, 300], [64, 30]),
    ("bf16", 32, 1, 128, [200, 31], [40, 17]),
    ("f16", 8, 1, 128, [0], [130]),
    ("bf16", 3, 2, 64, [10, 77, 0], [5, 9, 20]),
    ("bf16", 40, 1, 64, [33], [6]),
    ("bf16", 4, 2, 128, [1000, 37], [200, 95]),   # many 32-key steps, odd block counts
    ("f16", 32, 1, 64, [513], [77]),
]


@pytest.mark.parametrize("dtype,G,Hkv,D,cached,q_lens", CASES)
def test_chunked_matches_oracle(dtype, G, Hkv, D, cached, q_lens):
    case = make_chunked_case([31, G, D], dtype, cached, q_lens, G * Hkv, Hkv, D, label="random")
    ref, pool = oracle_chunked(case)
    out, kc, vc = run_chunked(case)
    check_close(out, ref, dtype, f"chunked {dtype} G={G}", weights_vmax=vmax_of(case.paged.logical_v))
    # the chunk's K/V went into the pool bit for bit
    assert torch.equal(bits(kc.cpu()), bits(pool.key_cache))
    assert torch.equal(bits(vc.cpu()), bits(pool.value_cache))


def test_chunk_of_one_row_equals_decode():
    """A one-token chunk is a decode step."""
    case = make_chunked_case([32], "bf16", [50, 300], [1, 1], 32, 8, 128, label="L=1")
    out, kc, vc = run_chunked(case)
    dec = torch.empty_like(out)
    pkv.paged_attention_decode(dec, dev(case.query), kc, vc, dev(case.paged.block_tables),
                               dev(case.paged.context_lens), case.scale)
    torch.cuda.synchronize()
    ref, _ = oracle_chunked(case)
    check_close(out, ref, "bf16", "L=1 chunked", weights_vmax=vmax_of(case.paged.logical_v))
    check_close(dec, ref, "bf16", "L=1 decode")


def test_chunked_deterministic_and_nan_safe():
    case = make_chunked_case([33], "bf16", [61, 5], [19, 40], 8, 2, 128, label="det")
    a, _, _ = run_chunked(case)
    b, _, _ = run_chunked(case)
    assert torch.isfinite(a).all()
    assert torch.equal(bits(a), bits(b))
