"""paged_attention_decode_static -- the decode entry point that allocates nothing --
against paged_attention_decode with a caller-given workspace, through the C ABI.

The two run the same kernels, so their outputs must agree bit for bit; both are
also held to the oracle's tolerance.  Two calls in a row per schedule, the second
on a smaller batch, so that the second call runs over scratch the first one left
behind."""

import numpy as np
import pytest
import torch

import paged_kv_cache_265_amd as pkv
from workloads.gen import make_decode_case

from helpers import bits, check_close, dev, oracle_decode_case

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def both_entry_points(case, partition_size):
    q = dev(case.query)
    kc, vc = dev(case.pool.key_cache), dev(case.pool.value_cache)
    bt, cl = dev(case.block_tables), dev(case.context_lens)
    ref_out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode(ref_out, q, kc, vc, bt, cl, case.scale, partition_size=partition_size)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode_static(out, q, kc, vc, bt, cl, case.scale, partition_size=partition_size)
    torch.cuda.synchronize()
    return out, ref_out


# (dtype, G, Hkv, contexts): a larger batch, then a smaller one
SEQUENCE = [
    ("bf16", 4, 8, [3000, 17, 0, 900, 40000, 1, 255, 4096]),
    ("bf16", 4, 8, [700, 33]),
    ("bf16", 32, 1, [20000, 5, 9000]),
    ("f16", 1, 4, [64]),
]


@pytest.mark.parametrize("partition_size", [0, 512])
def test_static_scratch_matches_workspace_entry_point(partition_size):
    for i, (dtype, G, Hkv, ctx) in enumerate(SEQUENCE):
        say(f"static scratch: partition_size={partition_size} {dtype} G={G} Hkv={Hkv} ctx={ctx}")
        case = make_decode_case([91, i, partition_size], dtype, ctx, G * Hkv, Hkv, 128)
        need = pkv.decode_workspace_size(case.num_seqs, G * Hkv, Hkv, 128, 16, case.max_blocks_per_seq,
                                         partition_size)
        assert need <= pkv.pkv.STATIC_SCRATCH_BYTES
        out, ref_out = both_entry_points(case, partition_size)
        assert torch.equal(bits(out), bits(ref_out)), "static scratch and workspace outputs differ"
        check_close(out, oracle_decode_case(case), dtype, f"static scratch {dtype} G={G}")
        for s, n in enumerate(ctx):
            if n == 0:
                assert torch.all(out[s] == 0)


def test_static_scratch_rejects_a_need_beyond_its_size():
    """Fixed 16-token partitions of 64 long MQA contexts need far more than the
    static scratch holds: the call fails before launching anything."""
    case = make_decode_case([92], "bf16", [16] * 64, 32, 1, 128, max_blocks_per_seq=4096)
    need = pkv.decode_workspace_size(64, 32, 1, 128, 16, 4096, 16)
    assert need > pkv.pkv.STATIC_SCRATCH_BYTES
    q = dev(case.query)
    out = torch.zeros_like(q)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_static(out, q, dev(case.pool.key_cache), dev(case.pool.value_cache),
                                          dev(case.block_tables), dev(case.context_lens), case.scale,
                                          partition_size=16)
    assert e.value.code == pkv.pkv.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
