/*
 * pkv_block_manager.h -- host-side manager of the paged KV pool (C ABI).
 *
 * It produces the inputs of the kernels in pkv.h: per-sequence block tables and
 * context lengths, the slot_mapping of new tokens (reshape_and_cache) and the
 * block copies of copy-on-write (copy_blocks).  Host memory only; not thread-safe
 * (one manager per thread, or external locking).
 *
 * Sources: "现代 LLM 推理引擎剖析", section 1.3 (the KV cache manager keeps a queue
 * of free blocks; a block table maps each request to its blocks, allocated on
 * demand in blocks of 16 tokens) and section 2.2 (prefix caching: each full
 * 16-token chunk gets a hash that combines the previous block's hash with the
 * chunk's tokens; a request reuses the longest run of cached leading blocks and
 * raises their reference counts); "每生成一个字都要把全部权重读一遍：从 vLLM 看 LLM
 * 推理提速", paging section (block table of physical block and fill per entry;
 * forks of parallel sampling and beam search share blocks through a reference
 * count; a write into a shared block copies it first and lowers the count).
 *
 * Policies the pages leave open, fixed here:
 *  - the free queue is FIFO; at creation it holds blocks 0 .. num_blocks-1 in order;
 *  - a freed sequence releases its blocks from the last logical block to the first;
 *  - block hashes are FNV-1a 64 over (previous hash, 8 bytes little-endian; then
 *    the chunk's token ids, int32 little-endian); the first block chains from the
 *    FNV offset basis; a hit also requires equal token ids;
 *  - a cached block is a full prompt block registered by pkv_bm_commit_prompt; it
 *    stays findable while free and loses its hash when handed out again; when two
 *    blocks carry the same hash the first one registered keeps it;
 *  - copy-on-write lowers the shared block's count by one per copy.
 *
 * Errors: functions returning int give PKV_OK (0) or a negative status of pkv.h
 * (PKV_ERR_INVALID for unknown/duplicate sequences or bad sizes; PKV_ERR_NO_BLOCKS
 * when the pool runs out, in which case the manager is left as it was before the
 * call).  pkv_last_error() gives a message.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ERR_NO_BLOCKS (-5)

typedef struct pkv_block_manager pkv_block_manager;

/* A pool of num_blocks blocks of block_size tokens, all free.  NULL on bad sizes. */
pkv_block_manager* pkv_bm_create(int num_blocks, int block_size);
void pkv_bm_destroy(pkv_block_manager* bm);

int pkv_bm_num_free(const pkv_block_manager* bm);

/* New sequence `seq` (any int id not in use).  With prompt != NULL (n tokens), the
 * longest run of its leading full blocks found in the prefix cache is shared
 * (count + 1 each) and *cached_tokens (if not NULL) receives their token count;
 * the caller then appends the remaining prompt tokens. */
int pkv_bm_add_sequence(pkv_block_manager* bm, int seq, const int32_t* prompt, int n, int* cached_tokens);

/* `child` starts as a copy of `parent`'s table and length; all blocks are shared. */
int pkv_bm_fork(pkv_block_manager* bm, int parent, int child);

/* Room for n more tokens of `seq`: slots_out[n] receives each token's slot
 * (block * block_size + offset); copies_out (room for max_copies (src, dst)
 * pairs, int64 each) receives the copy-on-write copies to run before writing
 * (at most one per call); *num_copies their count. */
int pkv_bm_append(pkv_block_manager* bm, int seq, int n, int64_t* slots_out, int64_t* copies_out, int max_copies,
                  int* num_copies);

/* Register the hashes of `seq`'s full prompt blocks (call after their K/V were
 * written).  *added (if not NULL) receives how many blocks got a hash. */
int pkv_bm_commit_prompt(pkv_block_manager* bm, int seq, const int32_t* prompt, int n, int* added);

/* Release `seq` (finished or preempted): counts drop, unreferenced blocks rejoin
 * the free queue. */
int pkv_bm_free_sequence(pkv_block_manager* bm, int seq);

/* Context length (tokens) of `seq`, or a negative status. */
int64_t pkv_bm_context_len(const pkv_block_manager* bm, int seq);

/* Block table of `seq` into out[max_blocks] (int32, padded with pad_value);
 * *num_blocks receives its length.  PKV_ERR_INVALID when it does not fit. */
int pkv_bm_block_table(const pkv_block_manager* bm, int seq, int32_t* out, int max_blocks, int32_t pad_value,
                       int* num_blocks);

/* Reference count of a block, or a negative status. */
int pkv_bm_refcount(const pkv_block_manager* bm, int block);

/* The free queue from head to tail into out[max_n]; returns how many were written
 * (at most max_n), or a negative status. */
int pkv_bm_free_queue(const pkv_block_manager* bm, int32_t* out, int max_n);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
