/*
 * pkv.h -- C ABI of the paged-attention library for AMD Instinct MI355X (gfx950).
 *
 * Four calls make up the hot path of decoding over a paged KV cache:
 *   paged_attention_decode   one query token per sequence over its paged K/V
 *   paged_attention_chunked  causal attention of short query chunks (chunked prefill)
 *   reshape_and_cache        write new K/V tokens into their slots
 *   copy_blocks              whole-block copies for copy-on-write
 * and paged_attention_mixed runs a flattened batch of decode tokens and prefill
 * chunks (the chunked call's arguments) in one attention launch.
 *
 * Sources.  The operation is the one described on three web pages:
 *  [P1] "每生成一个字都要把全部权重读一遍：从 vLLM 看 LLM 推理提速" -- section on paging
 *       the KV cache: fixed-size blocks placed anywhere in a physical pool, a
 *       per-sequence block table, the blockwise attention equation
 *       s_j = q.K_j / sqrt(d_k), o = sum_j softmax(s)_j V_j (equal to attention over
 *       the blocks concatenated in logical order), and copy-on-write of a shared
 *       block with a reference count.
 *  [P2] "现代 LLM 推理引擎剖析" -- section 1.3 (block size 16 by default; block bytes
 *       2 x block_size x kv heads x head size x dtype bytes), section 1.6 (slot_mapping
 *       built when preparing inputs; custom paged-attention kernel over a
 *       flattened batch), section 2.1 (chunked prefill).
 *  [P3] "LLM 推理优化的系统视角：从 KV Cache 到调度" -- section 3.1 (dense causal
 *       attention; a decode step reads the cached K/V and appends the new one),
 *       section 4.1 (MHA / MQA / GQA: a group of query heads shares one K/V head).
 *
 * ---------------------------------------------------------------------------------
 * Memory layout (all device memory, row-major, no padding).  Notation:
 *   S  = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads, G = Hq / Hkv,
 *   D  = head_dim, BS = block_size, NB = num_blocks, MB = max_blocks_per_seq.
 *   query        [S][Hq][D]           (decode)  or [total_q][Hq][D] (chunked)
 *   out          same shape and type as query
 *   key_cache    [NB][Hkv][BS][D]     one (block, kv head) tile is token-major
 *   value_cache  [NB][Hkv][D][BS]     one (block, kv head) tile is head_dim-major
 *   block_tables int32 [rows][MB]     physical block of each logical block; entries
 *                                     at index >= ceil(ctx / BS) are never read
 *   context_lens int32 [rows]         tokens of each sequence, including the ones
 *                                     being decoded (write first, then attend)
 *   slot_mapping int64 [num_tokens]   slot = block * BS + offset; negative = skip
 * Query head h uses kv head h / G (contiguous groups; G = 1 is MHA, Hkv = 1 is MQA).
 * The value tile is stored transposed so that the token dimension of the P.V
 * product is contiguous.
 *
 * Element types: PKV_F32, PKV_F16 (IEEE binary16), PKV_BF16 (bfloat16).  Query,
 * caches and output share one type.  Arithmetic is fp32; outputs are rounded to
 * the element type with round-to-nearest-even.
 *
 * Supported: head_dim in {64, 128}, block_size in {8, 16, 32} ([P2] section 1.3
 * uses 16; the size is the caller's trade of table length against the unused
 * slots of each sequence's last block), Hq % Hkv == 0, Hkv >= 1.  The attention
 * kernels work in 16-token tiles at every block size (a tile is one 16-token
 * block, half of a 32-token block, or two 8-token blocks), so the same logical
 * K/V gives the same bits at every block size.
 *
 * Conventions for every call:
 *  - Ownership: the caller owns every buffer, the workspace included.  The library
 *    allocates, frees and synchronises nothing and keeps no state besides a
 *    thread-local error message.
 *  - Asynchrony: calls enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *    stream) and return.  Results are ready when the stream reaches that point.
 *  - Errors: arguments are validated on the host before anything is launched; an
 *    invalid argument returns a negative code and launches nothing.  A launch
 *    failure returns PKV_ERR_HIP.  pkv_last_error() gives a message.
 *  - Device-side contract (checked only with PKV_DEBUG_CHECKS=1, see below): block
 *    ids in tables and block_mapping are in [0, NB); 0 <= context_lens[i] <= MB * BS;
 *    cu_q_lens starts at 0, never decreases, ends at total_q, and no segment has
 *    more than max_q_len rows or more rows than context tokens; slots are unique and
 *    < NB * BS; the copy_blocks destination set has no duplicates and is disjoint
 *    from its source set; outputs do not alias inputs.  Unchecked, breaking it reads
 *    or writes out of bounds.
 *  - Pointers to query/out/caches/key/value must be 16-byte aligned.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 };

enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_INVALID = -1,     /* null pointer, bad size, Hq % Hkv != 0, bad scale, misaligned pointer */
    PKV_ERR_UNSUPPORTED = -2, /* head_dim, block_size or dtype outside the supported set */
    PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than pkv_decode_workspace_size() */
    PKV_ERR_HIP = -4,         /* the HIP runtime refused a launch */
    PKV_ERR_CONTRACT = -6     /* PKV_DEBUG_CHECKS=1: the device-side contract is broken */
};

/* Library version as major * 10000 + minor * 100 + patch. */
int pkv_version(void);

/* Partition length (tokens) that paged_attention_decode uses for the given
 * arguments: partition_size itself when > 0; 0 when partition_size is 0, meaning
 * the balanced split (see paged_attention_decode).  Returns a negative status
 * when block_size <= 0 or partition_size is negative or not a multiple of both
 * block_size and 16. */
int pkv_decode_partition_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int max_blocks_per_seq, int partition_size);

/* Bytes of workspace paged_attention_decode needs.
 *   partition_size == 0 (balanced split): depends on num_seqs, the heads per kv
 *     head, head_dim and the compute units of the current device -- an int64 per
 *     sequence, then for each wave the split may launch on that device (4 per
 *     compute unit when its inner loop is built for one wave per SIMD, which is
 *     the case at head_dim 128 with two or more query heads per kv head; up to 16
 *     otherwise; at most 8192) a 32-byte merge note and room for two fp32 records of
 *     (head_dim + 2) values per query head of a kv head: 4.3 MB at 4 query heads
 *     per kv head and 34 MB at 32, head_dim 128, on MI355X's 256 compute units.
 *     Size it with the device that will run the call current.
 *   partition_size > 0: one such record per (sequence, query head, partition);
 *     zero when every sequence fits one partition (max_blocks_per_seq *
 *     block_size <= partition_size).
 * 0 means no workspace is needed (num_seqs == 0 included).  Invalid arguments (those
 * paged_attention_decode would reject as PKV_ERR_INVALID) return PKV_SIZE_INVALID,
 * with pkv_last_error() saying why. */
#define PKV_SIZE_INVALID ((size_t)-1)
size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int partition_size);

/*
 * paged_attention_decode -- [P1] blockwise attention equation; [P3] section 3.1.
 *
 * For each sequence s and query head h (kv head g = h / G), with n = context_lens[s]:
 *   K_t = key_cache[block_tables[s][t / BS]][g][t % BS][:], V_t likewise from
 *   value_cache[...][g][:][t % BS], for t = 0 .. n-1;
 *   out[s][h][:] = sum_t exp(x_t - max x) V_t / sum_t exp(x_t - max x),
 *   x_t = scale * (query[s][h][:] . K_t).
 * The softmax is one softmax over all n tokens.  n = 0 gives a zero output.
 *
 * The work is cut into pieces, each keeping (reference max, sum, unnormalised
 * output) in the workspace; a second kernel merges the pieces of every cut
 * sequence ([P3] section 4.2: tiling changes the order of the sums, not the
 * result):
 *   partition_size == 0: balanced split -- the (sequence, kv head, 16-token
 *     tile) units of the whole batch are dealt out in equal contiguous ranges to
 *     as many one-wave workgroups as the GPU holds at once.
 *   partition_size > 0: fixed partitions of that many tokens per sequence.
 *   workspace / workspace_bytes: device buffer of at least
 *   pkv_decode_workspace_size(...) bytes, 16-byte aligned (may be NULL when that
 *   size is 0).  Its contents on entry do not matter and are undefined on
 *   return.  Calls that share a workspace must not overlap in time.
 *   partition_size: 0 or a positive multiple of both block_size and 16 (a
 *     partition is whole blocks and whole tiles); otherwise PKV_ERR_INVALID.
 * Results do not depend on partition_size beyond fp32 rounding order, and a
 * given call is deterministic (bit for bit on repeat).
 */
int paged_attention_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, float scale, int dtype, int partition_size, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_static -- paged_attention_decode without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call the allocator, harnesses that forbid it.
 *
 * Same arguments (minus workspace / workspace_bytes), same kernels, same result bit
 * for bit as paged_attention_decode.  The scratch it needs comes from a device
 * array of PKV_STATIC_SCRATCH_BYTES inside the library: each GPU the library runs
 * on holds its own copy from the first call on it until the process ends.  The call
 * allocates and frees nothing.
 *   - A call whose scratch need (pkv_decode_workspace_size of the same arguments)
 *     exceeds PKV_STATIC_SCRATCH_BYTES returns PKV_ERR_WORKSPACE and launches
 *     nothing; use paged_attention_decode with a workspace for it.
 *   - Every call on one GPU shares that GPU's array, and nothing in it has to start
 *     at any particular value.  Calls that overlap in time on one GPU (other
 *     streams, other host threads) race on it: order them.
 */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int paged_attention_decode_static(void* out, const void* query, const void* key_cache, const void* value_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, float scale, int dtype, int partition_size, void* stream);

/*
 * paged_attention_chunked -- [P2] sections 1.4 and 2.1 (a long prompt is cut into
 * chunks that run in a flattened batch); [P3] section 3.1 (causal attention).
 *
 * Segment i owns query rows cu_q_lens[i] .. cu_q_lens[i+1]-1 (L_i rows) and has
 * n_i = context_lens[i] tokens in the cache, its own chunk included (write the
 * chunk with reshape_and_cache first).  Row r of segment i sits at position
 * n_i - L_i + r and attends to tokens 0 .. n_i - L_i + r through block_tables[i].
 *   cu_q_lens: device int32 [num_segs + 1], cu_q_lens[0] = 0, non-decreasing,
 *              cu_q_lens[num_segs] = total_q.
 *   max_q_len: host bound on every L_i (sizes the grid; rows beyond L_i are idle).
 * Requires context_lens[i] >= L_i (device contract).
 */
int paged_attention_chunked(void* out, const void* query, const int32_t* cu_q_lens, int num_segs, int total_q,
                            int max_q_len, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int num_q_heads,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                            float scale, int dtype, void* stream);

/*
 * paged_attention_mixed -- [P2] sections 1.4 and 2.1: one pass over a flattened
 * batch that mixes prefill chunks and decode tokens.
 *
 * Computes exactly what paged_attention_chunked computes for the same arguments
 * (every segment, causal rows), in one attention launch plus a small merge
 * launch: segments with one query row are decode sequences, whose contexts are
 * cut across many waves (the balanced split of paged_attention_decode) and merged;
 * the other segments run as chunked-prefill tiles beside them, so the HBM-bound
 * decode and the matrix-core-bound prefill overlap.  16-bit types only.
 *   workspace / workspace_bytes: device buffer of at least
 *   pkv_mixed_workspace_size(...) bytes, 16-byte aligned; contents on entry do
 *   not matter.  Calls that share a workspace must not overlap in time.
 * Requires context_lens[i] >= L_i (device contract).  Deterministic bit for bit on
 * repeat; decode rows agree with paged_attention_decode to fp32 rounding order.
 */
int paged_attention_mixed(void* out, const void* query, const int32_t* cu_q_lens, int num_segs, int total_q,
                          int max_q_len, const void* key_cache, const void* value_cache, const int32_t* block_tables,
                          const int32_t* context_lens, int num_q_heads, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, int max_blocks_per_seq, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace paged_attention_mixed needs: the balanced-split layout of
 * paged_attention_decode for num_segs sequences and one four-wave workgroup of decode
 * waves per compute unit of the current device.  PKV_SIZE_INVALID on invalid
 * arguments. */
size_t pkv_mixed_workspace_size(int num_segs, int num_q_heads, int num_kv_heads, int head_dim, int block_size);

/*
 * reshape_and_cache -- [P2] section 1.6 (slot_mapping); [P3] section 3.1 (append the
 * new K/V to the cache).
 *
 * For token i with slot = slot_mapping[i] >= 0, b = slot / BS, o = slot % BS:
 *   key_cache[b][h][o][:] = key[i][h][:] and value_cache[b][h][:][o] = value[i][h][:]
 * for every kv head h.  A bit copy: no conversion, no rounding.
 *   key, value: device [num_tokens][Hkv][D].  num_tokens may be 0.
 */
int reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int dtype, void* stream);

/*
 * copy_blocks -- [P1] copy-on-write paragraph (a block shared by several sequences is
 * copied whole before one of them writes into it).
 *
 * For every layer l < num_layers and pair p < num_pairs with (src, dst) =
 * (block_mapping[2p], block_mapping[2p+1]): block dst of key_caches[l] and of
 * value_caches[l] becomes a bit copy of block src.
 *   key_caches, value_caches: HOST arrays of num_layers device pointers, each a
 *                             pool laid out as above.
 *   block_mapping: device int64 [num_pairs][2].  num_pairs and num_layers may be 0.
 */
int copy_blocks(void* const* key_caches, void* const* value_caches, int num_layers, const int64_t* block_mapping,
                int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype,
                void* stream);

/*
 * pkv_read_probe -- measurement utility, not part of the attention path.
 *
 * Streams `bytes` bytes of device memory at `buf` with the non-temporal 16-byte
 * loads the decode kernels use (one workgroup of four waves per compute unit,
 * each wave reading whole 4 KiB tiles, two in flight: the fastest shape of a
 * sweep on MI355X), so that a caller can time the practical HBM read ceiling
 * next to a decode call.
 *   buf:   device pointer, 16-byte aligned; bytes: a positive multiple of 4096.
 *   sink:  device buffer of at least 4 bytes; it is written only if the XOR of
 *          all words read equals 0x9e3779b9 (never for a zero-filled buffer), which
 *          keeps the loads from being optimised away.
 */
int pkv_read_probe(const void* buf, size_t bytes, void* sink, void* stream);

/*
 * Checking the device-side contract.
 *
 * With the environment variable PKV_DEBUG_CHECKS set to 1 (read at every call),
 * paged_attention_decode(_static), paged_attention_chunked, paged_attention_mixed,
 * reshape_and_cache and copy_blocks first enqueue a pre-pass over their tables,
 * context lengths, query lengths, slots or copy pairs (nothing else is read), and
 * every kernel of the call returns at once if it found a violation, so nothing is
 * read or written out of bounds.  The call then waits for its stream and returns
 * PKV_ERR_CONTRACT, pkv_last_error() naming the first violation.  Checked calls
 * synchronise, are serialised across the process, and must not be captured in a
 * graph; unchecked calls (the default) are unaffected.
 *
 * A verdict word packs a violation as (index << 32) | (sub-index << 8) | code,
 * with index the sequence / segment / token / pair and sub-index the logical block
 * (PKV_BAD_BLOCK_ID), the side of a pair (PKV_BAD_COPY_BLOCK: 0 source, 1
 * destination) or the broken condition (PKV_BAD_QUERY_LENS: 0 cu_q_lens[0] != 0,
 * 1 rows < 0 or > max_q_len, 2 rows > context, 3 last entry != total_q); the
 * verdict of a whole check is the smallest such word, PKV_CONTRACT_OK if none.
 */
#define PKV_CONTRACT_OK (~(uint64_t)0)
enum pkv_contract_code {
    PKV_BAD_CONTEXT_LEN = 1,    /* context_lens[s] < 0 or > MB * BS */
    PKV_BAD_BLOCK_ID = 2,       /* block_tables[s][b] outside [0, NB), b < ceil(ctx / BS) */
    PKV_BAD_QUERY_LENS = 3,     /* cu_q_lens breaks its rules */
    PKV_BAD_SLOT = 4,           /* slot_mapping[i] >= NB * BS */
    PKV_DUPLICATE_SLOT = 5,     /* slot_mapping[i] equals an earlier non-negative slot */
    PKV_BAD_COPY_BLOCK = 6,     /* a source or destination outside [0, NB) */
    PKV_DUPLICATE_COPY_DST = 7, /* a destination repeats an earlier pair's */
    PKV_COPY_DST_IS_SRC = 8     /* a destination is also a source */
};

/* The same checks as calls of their own.  The pkv_check_* calls take device arrays,
 * run the pre-pass on `stream`, wait for it and store the verdict in *verdict (host
 * memory); they return PKV_OK (whatever the verdict), PKV_ERR_INVALID for bad sizes
 * or null pointers, PKV_ERR_HIP on a runtime failure.  The *_host variants take host
 * arrays, run the very same item checks on the CPU and return the verdict.
 *   tables: rows x max_blocks_per_seq block_tables and rows context_lens; with
 *     cu_q_lens (rows + 1 entries) non-NULL the chunked/mixed query-length rules too. */
int pkv_check_tables(const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q_lens, int num_rows,
                     int max_blocks_per_seq, int block_size, int num_blocks, int total_q, int max_q_len,
                     uint64_t* verdict, void* stream);
int pkv_check_slots(const int64_t* slot_mapping, int num_tokens, int block_size, int num_blocks, uint64_t* verdict,
                    void* stream);
int pkv_check_copies(const int64_t* block_mapping, int num_pairs, int num_blocks, uint64_t* verdict, void* stream);
uint64_t pkv_check_tables_host(const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q_lens,
                               int num_rows, int max_blocks_per_seq, int block_size, int num_blocks, int total_q,
                               int max_q_len);
uint64_t pkv_check_slots_host(const int64_t* slot_mapping, int num_tokens, int block_size, int num_blocks);
uint64_t pkv_check_copies_host(const int64_t* block_mapping, int num_pairs, int num_blocks);

/*
 * pkv_decode_variant -- test and measurement hook, not part of the attention path's
 * interface: paged_attention_decode with its inner loop and prefetch depth chosen
 * by the caller instead of by the library, so that every loop can be compared with
 * the others on the same inputs.  Same arguments, result and conventions as
 * paged_attention_decode, plus
 *   inner_loop: 0 the library's choice, 1 the vector-ALU loop, 2 the matrix-core loop
 *               (16-bit types only; PKV_ERR_UNSUPPORTED for fp32);
 *   ring:       0 the loop's own prefetch depth, 2 a two-tile ring (one block in
 *               flight; used by the balanced split only).
 * Its workspace is pkv_decode_variant_workspace_size(...) bytes (the same arguments
 * as pkv_decode_workspace_size plus dtype, inner_loop and ring; PKV_SIZE_INVALID on
 * invalid ones).
 */
int pkv_decode_variant(void* out, const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                       float scale, int dtype, int partition_size, void* workspace, size_t workspace_bytes,
                       int inner_loop, int ring, void* stream);
size_t pkv_decode_variant_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int max_blocks_per_seq, int partition_size, int dtype,
                                         int inner_loop, int ring);

/* Fixed text for a status code. */
const char* pkv_error_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
