// contract.h -- the device-side contract of the attention and cache calls, as checks
// of one item at a time that compile for the host and for gfx950 alike.
//
// What the kernels take for granted, and never check on their own (checking costs
// loads on the hot path):
//  * a block table entry names a physical block of the pool: every entry a
//    sequence uses (index < ceil(ctx / BS)) lies in [0, NB) ("每生成一个字都要把全部权重
//    读一遍", paging section: the block table maps each logical block to a physical
//    block number);
//  * a context fits its table: 0 <= ctx <= MB * BS;
//  * chunked segments ("现代 LLM 推理引擎剖析", sections 1.4 and 2.1): cu_q_lens starts
//    at 0, never decreases, ends at total_q; no segment has more than max_q_len rows
//    or more rows than its context holds tokens;
//  * reshape_and_cache ("现代 LLM 推理引擎剖析", section 1.6): a slot is < NB * BS and no
//    two tokens share one (negative slots are skipped);
//  * copy_blocks (copy-on-write paragraph of the first page): sources and
//    destinations are blocks of the pool, no destination repeats, and no block is
//    both a destination and a source.
//
// A check that fails yields a verdict word
//     (index << 32) | (sub-index << 8) | code
// (index: sequence, segment, token or pair; sub-index: logical block or which
// condition, clamped to 24 bits).  The verdict of a whole call is the smallest word
// over every violation, ~0 (PKV_CONTRACT_OK) when there is none: the first
// violation in index order, the same whoever computes it.
#pragma once

#include <stdint.h>

#include "pkv.h"

#ifdef __HIPCC__
#define PKV_HD __host__ __device__ __forceinline__
#else
#define PKV_HD inline
#endif

namespace pkv {
namespace contract {

PKV_HD uint64_t violation(int64_t index, int64_t sub, int code) {
    const uint64_t s = sub < 0 ? 0 : (sub > 0xffffff ? 0xffffff : (uint64_t)sub);
    return ((uint64_t)(uint32_t)index << 32) | (s << 8) | (uint64_t)(code & 0xff);
}

// Table entry (s, b) of a call with num_rows rows: the context of row s (checked on
// b == 0) and, when b is one of the row's blocks, the block id there.
PKV_HD uint64_t table_entry(const int32_t* block_tables, const int32_t* context_lens, int s, int b, int MB, int BS,
                            int NB) {
    const int ctx = context_lens[s];
    if (ctx < 0 || (int64_t)ctx > (int64_t)MB * BS) return b == 0 ? violation(s, 0, PKV_BAD_CONTEXT_LEN) : PKV_CONTRACT_OK;
    const int nb = (int)(((int64_t)ctx + BS - 1) / BS);
    if (b >= nb) return PKV_CONTRACT_OK;
    const int32_t id = block_tables[(size_t)s * MB + b];
    return (id < 0 || id >= NB) ? violation(s, b, PKV_BAD_BLOCK_ID) : PKV_CONTRACT_OK;
}

// Segment i of a chunked or mixed call (cu_q_lens has num_segs + 1 entries); segment
// num_segs stands for the end of the array.  Sub-indices: 0 first entry not 0,
// 1 rows negative or above max_q_len, 2 more rows than context tokens, 3 last entry
// not total_q.
PKV_HD uint64_t segment(const int32_t* cu_q_lens, const int32_t* context_lens, int i, int num_segs, int total_q,
                        int max_q_len) {
    if (i == num_segs) return cu_q_lens[num_segs] != total_q ? violation(i, 3, PKV_BAD_QUERY_LENS) : PKV_CONTRACT_OK;
    if (i == 0 && cu_q_lens[0] != 0) return violation(0, 0, PKV_BAD_QUERY_LENS);
    const int64_t L = (int64_t)cu_q_lens[i + 1] - cu_q_lens[i];
    if (L < 0 || L > max_q_len) return violation(i, 1, PKV_BAD_QUERY_LENS);
    if (L > context_lens[i]) return violation(i, 2, PKV_BAD_QUERY_LENS);
    return PKV_CONTRACT_OK;
}

// Token i of reshape_and_cache against the pool, and token i against an earlier token
// j (< i) holding the same slot.
PKV_HD uint64_t slot_in_pool(const int64_t* slots, int i, int BS, int NB) {
    return slots[i] >= (int64_t)NB * BS ? violation(i, 0, PKV_BAD_SLOT) : PKV_CONTRACT_OK;
}
PKV_HD uint64_t slot_pair(int64_t slot_i, int64_t slot_j, int i) {
    return (slot_i >= 0 && slot_i == slot_j) ? violation(i, 0, PKV_DUPLICATE_SLOT) : PKV_CONTRACT_OK;
}

// Pair p of copy_blocks ((src, dst) = mapping[2p], mapping[2p + 1]) against the pool
// (sub-index 0: src, 1: dst), and against pair q: its destination repeats q's
// (q < p), or is q's source (any q).
PKV_HD uint64_t copy_in_pool(const int64_t* mapping, int p, int NB) {
    if (mapping[2 * p] < 0 || mapping[2 * p] >= NB) return violation(p, 0, PKV_BAD_COPY_BLOCK);
    if (mapping[2 * p + 1] < 0 || mapping[2 * p + 1] >= NB) return violation(p, 1, PKV_BAD_COPY_BLOCK);
    return PKV_CONTRACT_OK;
}
PKV_HD uint64_t copy_pair(int64_t src_q, int64_t dst_q, int64_t dst_p, int p, int q) {
    if (dst_p == src_q) return violation(p, 0, PKV_COPY_DST_IS_SRC);
    if (q < p && dst_p == dst_q) return violation(p, 0, PKV_DUPLICATE_COPY_DST);
    return PKV_CONTRACT_OK;
}

PKV_HD uint64_t min_verdict(uint64_t a, uint64_t b) { return a < b ? a : b; }

}  // namespace contract
}  // namespace pkv
