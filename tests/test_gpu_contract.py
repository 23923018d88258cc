"""The contract pre-pass on the GPU (PKV_DEBUG_CHECKS=1 and the pkv_check_* calls).

1. The device pre-pass gives the host checks' verdict on every case of
   contract_cases.py and on the workloads' own tables (which keep the contract).
2. With checks on, valid calls return PKV_OK and the same bits as unchecked ones.
3. With checks on, calls whose inputs break the contract return PKV_ERR_CONTRACT and
   leave outputs and caches untouched.  The broken inputs used here would stay
   inside the buffers even unchecked (a block id equal to num_blocks names a spare
   block that the pool tensors really hold; repeated slots and a copy onto a source
   block write inside the pool), so nothing here can read or write out of bounds."""

import numpy as np
import pytest
import torch

import paged_kv_cache_265_amd as pkv
from workloads.gen import make_chunked_case, make_cow_case, make_decode_case

from contract_cases import BS, NB, copy_cases, segment_cases, slot_cases, table_cases
from helpers import bits, dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def test_device_pre_pass_gives_the_host_verdicts():
    for name, bt, ctx, want in table_cases():
        say(f"tables: {name}")
        assert pkv.check_tables(dev(bt), dev(ctx), BS, NB) == want == pkv.check_tables_host(bt, ctx, BS, NB)
    for name, bt, ctx, cu, tq, mq, want in segment_cases():
        say(f"segments: {name}")
        assert pkv.check_tables(dev(bt), dev(ctx), BS, NB, dev(cu), tq, mq) == want
    for name, slots, want in slot_cases():
        say(f"slots: {name}")
        assert pkv.check_slots(dev(slots), BS, NB) == want
    for name, m, want in copy_cases():
        say(f"copies: {name}")
        assert pkv.check_copies(dev(m), NB) == want


def test_device_pre_pass_on_large_inputs():
    """Many rows and grid-stride table walks; many tokens across slot tiles."""
    rng = np.random.default_rng(5)
    S, MB, nb = 3000, 40, 200000
    ctx = rng.integers(0, MB * 16 + 1, size=S).astype(np.int32)
    bt = rng.integers(0, nb, size=(S, MB)).astype(np.int32)
    say(f"tables {S} x {MB}")
    assert pkv.check_tables(dev(bt), dev(ctx), 16, nb) == pkv.CONTRACT_OK
    s_bad = int(np.nonzero(ctx > 16 * 30)[0][0])
    bt[s_bad, 29] = nb
    bt[S - 1, 0] = -1
    ctx[S - 1] = max(ctx[S - 1], 1)
    want = pkv.check_tables_host(bt, ctx, 16, nb)
    assert want == pkv.violation(s_bad, 29, pkv.pkv.BAD_BLOCK_ID)
    assert pkv.check_tables(dev(bt), dev(ctx), 16, nb) == want
    slots = rng.permutation(nb * 16)[:5000].astype(np.int64)
    say(f"slots {len(slots)}")
    assert pkv.check_slots(dev(slots), 16, nb) == pkv.CONTRACT_OK
    slots[4321] = slots[17]
    assert pkv.check_slots(dev(slots), 16, nb) == pkv.violation(4321, 0, pkv.pkv.DUPLICATE_SLOT)


@pytest.fixture
def checks_on(monkeypatch):
    monkeypatch.setenv("PKV_DEBUG_CHECKS", "1")


def test_checked_calls_give_the_unchecked_bits(monkeypatch):
    case = make_decode_case([81], "bf16", [5, 700, 3000, 0, 64], 32, 8, 128, append_last=True)
    kc, vc = dev(case.pool.key_cache), dev(case.pool.value_cache)
    q, bt, cl = dev(case.query), dev(case.block_tables), dev(case.context_lens)
    outs = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("PKV_DEBUG_CHECKS", mode)
        say(f"decode, checks={mode}")
        k2, v2 = kc.clone(), vc.clone()
        pkv.reshape_and_cache(dev(case.new_key), dev(case.new_value), k2, v2, dev(case.slot_mapping))
        for part in (0, 512):
            o = torch.full_like(q, float("nan"))
            pkv.paged_attention_decode(o, q, k2, v2, bt, cl, case.scale, partition_size=part)
            outs[(mode, part)] = bits(o).clone()
        o = torch.full_like(q, float("nan"))
        pkv.paged_attention_decode_static(o, q, k2, v2, bt, cl, case.scale)
        outs[(mode, "static")] = bits(o).clone()
        outs[(mode, "k")] = bits(k2).clone()
        torch.cuda.synchronize()
    for key in (0, 512, "static", "k"):
        assert torch.equal(outs[("0", key)], outs[("1", key)]), key

    ch = make_chunked_case([82], "bf16", [0, 700, 40], [1, 64, 30], 8, 2, 128)
    pend = np.nonzero(ch.paged.pending)[0]
    ti = torch.from_numpy(pend)
    for fn in (pkv.paged_attention_chunked, pkv.paged_attention_mixed):
        res = []
        for mode in ("0", "1"):
            monkeypatch.setenv("PKV_DEBUG_CHECKS", mode)
            say(f"{fn.__name__}, checks={mode}")
            kc, vc = dev(ch.paged.pool.key_cache), dev(ch.paged.pool.value_cache)
            pkv.reshape_and_cache(dev(ch.paged.logical_k[ti].contiguous()), dev(ch.paged.logical_v[ti].contiguous()),
                                  kc, vc, dev(ch.paged.token_slots[pend].copy()))
            o = torch.full_like(dev(ch.query), float("nan"))
            fn(o, dev(ch.query), dev(ch.cu_q_lens), ch.max_q_len, kc, vc, dev(ch.paged.block_tables),
               dev(ch.paged.context_lens), ch.scale)
            torch.cuda.synchronize()
            res.append(bits(o).clone())
        assert torch.equal(res[0], res[1])

    c = make_cow_case([83], num_prompts=2, samples_per_prompt=3, prompt_blocks=4, max_private=40)
    res = []
    for mode in ("0", "1"):
        monkeypatch.setenv("PKV_DEBUG_CHECKS", mode)
        say(f"copy_blocks, checks={mode}")
        kc, vc = dev(c.pool.key_cache), dev(c.pool.value_cache)
        pkv.copy_blocks([kc], [vc], dev(c.block_mapping))
        torch.cuda.synchronize()
        res.append((bits(kc).clone(), bits(vc).clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def spare_block_pool(case):
    """The case's pool on the device with one more block at the end, so that block id
    num_blocks (outside the pool the call is told about) still lies inside the tensors."""
    kc = torch.cat([case.pool.key_cache, case.pool.key_cache[:1]]).contiguous()
    vc = torch.cat([case.pool.value_cache, case.pool.value_cache[:1]]).contiguous()
    return dev(kc), dev(vc)


def expect_contract_error(fn, *args, **kw):
    with pytest.raises(pkv.PkvError) as e:
        fn(*args, **kw)
    assert e.value.code == pkv.pkv.ERR_CONTRACT
    return str(e.value)


def test_checked_calls_refuse_broken_inputs_and_touch_nothing(checks_on):
    """The binding sizes the pool from the tensors, so the spare-block cases call the
    C ABI directly with num_blocks one short of what the tensors hold."""
    lib = pkv.load_library()
    case = make_decode_case([84], "bf16", [40, 300, 17], 8, 2, 128)
    kc, vc = spare_block_pool(case)
    nb = case.num_blocks
    bt = case.block_tables.copy()
    bt[1, 5] = nb  # the spare block: inside the tensors, outside the pool
    # every device array the raw calls below take is held in a name until the calls
    # have finished, so that no freed block can be handed to another array meanwhile
    q, bt_d, cl_d = dev(case.query), dev(bt), dev(case.context_lens)
    for part in (0, 64):
        say(f"decode, block id = num_blocks, partition_size={part}")
        o = torch.full_like(q, 7.0)
        ws = torch.empty(max(1, pkv.decode_workspace_size(3, 8, 2, 128, 16, bt.shape[1], part)), dtype=torch.uint8,
                         device="cuda")
        rc = lib.paged_attention_decode(o.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt_d.data_ptr(),
                                        cl_d.data_ptr(), 3, 8, 2, 128, 16, nb, bt.shape[1],
                                        case.scale, pkv.BF16, part, ws.data_ptr(), ws.numel(),
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == pkv.pkv.ERR_CONTRACT
        msg = lib.pkv_last_error().decode()
        assert "block_tables[1][5]" in msg, msg
        torch.cuda.synchronize()
        assert torch.all(o == 7.0)
    say("decode_static, block id = num_blocks")
    o = torch.full_like(q, 7.0)
    rc = lib.paged_attention_decode_static(o.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                           bt_d.data_ptr(), cl_d.data_ptr(), 3, 8, 2, 128, 16,
                                           nb, bt.shape[1], case.scale, pkv.BF16, 0,
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == pkv.pkv.ERR_CONTRACT
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)

    ch = make_chunked_case([85], "bf16", [100, 30], [20, 9], 8, 1, 128)
    kc, vc = spare_block_pool(ch.paged)
    bt = ch.paged.block_tables.copy()
    bt[0, 2] = ch.paged.pool.num_blocks
    q, cu_d, bt_d, cl_d = dev(ch.query), dev(ch.cu_q_lens), dev(bt), dev(ch.paged.context_lens)
    for fn in (pkv.paged_attention_chunked, pkv.paged_attention_mixed):
        say(f"{fn.__name__}, block id = num_blocks")
        o = torch.full_like(q, 7.0)
        args = [o.data_ptr(), q.data_ptr(), cu_d.data_ptr(), 2, ch.total_q, ch.max_q_len, kc.data_ptr(),
                vc.data_ptr(), bt_d.data_ptr(), cl_d.data_ptr(), 8, 1, 128, 16,
                ch.paged.pool.num_blocks, bt.shape[1], ch.scale, pkv.BF16]
        stream = torch.cuda.current_stream().cuda_stream
        if fn is pkv.paged_attention_chunked:
            rc = lib.paged_attention_chunked(*args, stream)
        else:
            ws = torch.empty(pkv.mixed_workspace_size(2, 8, 1, 128, 16), dtype=torch.uint8, device="cuda")
            rc = lib.paged_attention_mixed(*args, ws.data_ptr(), ws.numel(), stream)
        assert rc == pkv.pkv.ERR_CONTRACT
        assert "block_tables[0][2]" in lib.pkv_last_error().decode()
        torch.cuda.synchronize()
        assert torch.all(o == 7.0)

    say("reshape_and_cache, repeated slot")
    kc, vc = dev(case.pool.key_cache), dev(case.pool.value_cache)
    k0, v0 = bits(kc).clone(), bits(vc).clone()
    new_k = dev(torch.randn(3, 2, 128).to(torch.bfloat16))
    slots = np.array([5, 9, 5], np.int64)
    msg = expect_contract_error(pkv.reshape_and_cache, new_k, new_k.clone(), kc, vc, dev(slots))
    assert "slot_mapping[2]" in msg
    torch.cuda.synchronize()
    assert torch.equal(bits(kc), k0) and torch.equal(bits(vc), v0)

    say("copy_blocks, destination is a source")
    msg = expect_contract_error(pkv.copy_blocks, [kc], [vc], dev(np.array([[1, 2], [2, 3]], np.int64)))
    assert "block_mapping[0]" in msg
    torch.cuda.synchronize()
    assert torch.equal(bits(kc), k0) and torch.equal(bits(vc), v0)
