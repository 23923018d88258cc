"""The matrix-core hazard scan of paged_kv_cache_265_amd/resource_report.py, on small
hand-written gfx950 assembly listings (no compiler run): a vector read of a product's
result needs 8 wait states after the product, on every path to it."""

from paged_kv_cache_265_amd import resource_report as rr

HEAD = "_Zfoo:\n"


def scan(body: str):
    lines = (HEAD + body).split("\n")
    return rr._short_reads(lines, 0, len(lines))


def test_read_right_after_the_product_is_flagged():
    found = scan("\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
                 "\tv_max_f32_e32 v20, v1, v2\n")
    assert len(found) == 1 and found[0][1] == "v_max_f32_e32" and found[0][2] == 0


def test_eight_wait_states_clear_it():
    assert scan("\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
                "\ts_nop 7\n"
                "\tv_max_f32_e32 v20, v1, v2\n") == []
    # seven are not enough
    assert len(scan("\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
                    "\ts_nop 6\n"
                    "\tv_max_f32_e32 v20, v1, v2\n")) == 1


def test_independent_instructions_count_as_wait_states():
    body = "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
    body += "".join(f"\tv_add_f32_e32 v{30 + i}, v{40 + i}, v{50 + i}\n" for i in range(8))
    body += "\tv_max_f32_e32 v20, v1, v2\n"
    assert scan(body) == []


def test_taken_branch_path_is_followed():
    """The fall-through path is padded, the branch target is not: the case the fence
    of the decode loops closes."""
    body = ("\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
            "\ts_cbranch_vccnz .LBB0_2\n"
            "\ts_nop 7\n"
            "\tv_max_f32_e32 v20, v1, v2\n"
            ".LBB0_2:\n"
            "\tv_cndmask_b32_e32 v21, v0, v9, vcc\n")
    found = scan(body)
    assert len(found) == 1 and found[0][1] == "v_cndmask_b32_e32" and found[0][2] == 1


def test_accumulator_registers_are_tracked():
    found = scan("\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]\n"
                 "\tv_accvgpr_read_b32 v20, a3\n")
    assert len(found) == 1


def test_a_later_product_into_the_same_registers_is_not_a_read():
    assert scan("\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
                "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[12:15], v[16:19], v[0:3]\n") == []
