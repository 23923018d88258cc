// api.cpp -- the C ABI declared in include/pkv.h: host-side validation of every
// argument, then kernel launches on the caller's stream.  No allocation, no
// synchronisation, no state besides a thread-local error message.
#include "pkv.h"
#include "pkv_block_manager.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "internal.h"

static_assert(PKV_STATIC_SCRATCH_BYTES == pkv::kStaticScratchBytes, "header and library agree on the static scratch");

namespace {
thread_local char g_msg[512] = "";
}  // namespace

namespace pkv {
int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return code;
}
}  // namespace pkv

namespace {

using pkv::set_error;

int hip_fail(hipError_t e, const char* what) {
    return set_error(PKV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

// End of a call made with the contract pre-pass: wait for the verdict and turn a
// violation into PKV_ERR_CONTRACT.
int finish_checked(const char* fn, pkv::DebugChecks& dbg) {
    if (!dbg.on()) return PKV_OK;
    uint64_t v = PKV_CONTRACT_OK;
    const hipError_t e = dbg.finish(&v);
    if (e != hipSuccess) return set_error(PKV_ERR_HIP, "%s: contract check failed: %s", fn, hipGetErrorString(e));
    if (v == PKV_CONTRACT_OK) return PKV_OK;
    char what[256];
    pkv::describe_violation(v, what, sizeof what);
    return set_error(PKV_ERR_CONTRACT, "%s: %s", fn, what);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dtype_ok(int dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }

// Checks shared by every call on the pool geometry.  Returns PKV_OK or a status.
int check_pool(const char* fn, int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype) {
    if (num_kv_heads <= 0) return set_error(PKV_ERR_INVALID, "%s: num_kv_heads must be positive (got %d)", fn, num_kv_heads);
    if (num_blocks <= 0) return set_error(PKV_ERR_INVALID, "%s: num_blocks must be positive (got %d)", fn, num_blocks);
    if (!dtype_ok(dtype)) return set_error(PKV_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (head_dim != 64 && head_dim != 128)
        return set_error(PKV_ERR_UNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", fn, head_dim);
    if (!pkv::supported_block_size(block_size))
        return set_error(PKV_ERR_UNSUPPORTED, "%s: block_size %d not supported (8, 16 or 32)", fn, block_size);
    return PKV_OK;
}

// A fixed partition is a whole number of blocks and of 16-token tiles.
bool partition_ok(int partition_size, int block_size) {
    const int unit = block_size > pkv::kTileTokens ? block_size : pkv::kTileTokens;
    return partition_size == 0 || (partition_size > 0 && partition_size % unit == 0);
}

int check_heads(const char* fn, int num_q_heads, int num_kv_heads) {
    if (num_q_heads <= 0) return set_error(PKV_ERR_INVALID, "%s: num_q_heads must be positive (got %d)", fn, num_q_heads);
    if (num_q_heads % num_kv_heads != 0)
        return set_error(PKV_ERR_INVALID, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", fn, num_q_heads,
                    num_kv_heads);
    return PKV_OK;
}

int max_parts(int max_blocks_per_seq, int block_size, int part) {
    const long long tokens = (long long)max_blocks_per_seq * block_size;
    return (int)((tokens + part - 1) / part);
}

// Balanced split workspace: the per-sequence start units (S + 1 int64, padded to 256
// bytes), one merge note per wave the split may launch, then two records per wave.
size_t split_starts_bytes(int num_seqs) { return (((size_t)num_seqs + 1) * 8 + 255) / 256 * 256; }
size_t split_prefix_bytes(int num_seqs, long long waves) {
    return split_starts_bytes(num_seqs) + ((size_t)waves * sizeof(pkv::MergeNote) + 255) / 256 * 256;
}

// Waves the balanced split launches at most on the current device: every compute
// unit holds at most kSimdsPerCu x (waves per SIMD of the inner loop); kind < 0
// takes the largest over the three element types.
long long split_wave_bound(int kind, int G, int D, int path, int ring) {
    int per_simd = 0;
    for (int k = PKV_F32; k <= PKV_BF16; ++k)
        if (kind < 0 || kind == k) per_simd = std::max(per_simd, pkv::split_waves_per_simd(k, G, D, path, ring));
    const long long w = (long long)pkv::device_compute_units() * pkv::kSimdsPerCu * per_simd;
    return std::min<long long>(w, pkv::kMaxSplitWaves);
}

// waves of the single mixed launch's decode part: one four-wave workgroup per compute unit
long long mixed_decode_waves() {
    return std::min<long long>((long long)pkv::device_compute_units() * pkv::kSimdsPerCu, pkv::kMaxSplitWaves);
}

// Largest (query-head chunks x record capacity) over the inner loops a decode
// with G heads per kv head may use, and the largest record capacity.
void record_shape(int G, long long* heads_per_kv, int* cap_max) {
    const int ht_mfma = G <= 16 ? 16 : 32;
    const int ht_valu = G == 1 ? 1 : (G == 2 ? 2 : 4);
    long long best = 0;
    int cap = 0;
    for (int ht : {ht_mfma, ht_valu}) {
        const int c = G < ht ? G : ht;
        const long long chunks = (G + ht - 1) / ht;
        if (chunks * c > best) best = chunks * c;
        if (c > cap) cap = c;
    }
    *heads_per_kv = best;
    *cap_max = cap;
}


// Workspace bytes of a decode (see pkv_decode_workspace_size); kind < 0: enough for
// every element type.  *waves: the wave bound the balanced split's layout uses.
// PKV_SIZE_INVALID (with a message) for arguments no decode call would accept.
size_t decode_need(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                   int max_blocks_per_seq, int partition_size, int kind, int path, int ring, long long* waves) {
    *waves = 0;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
        head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || !partition_ok(partition_size, block_size) ||
        path < 0 || path > 2 || (ring != 0 && ring != 2)) {
        set_error(PKV_ERR_INVALID,
                  "workspace size: invalid arguments (num_seqs >= 0, positive head counts with num_q_heads a multiple "
                  "of num_kv_heads, positive sizes, partition_size 0 or a multiple of block_size and 16)");
        return PKV_SIZE_INVALID;
    }
    if (num_seqs == 0) return 0;
    const int G = num_q_heads / num_kv_heads;
    long long heads_per_kv = 0;
    int cap = 0;
    record_shape(G, &heads_per_kv, &cap);
    const size_t per_head = ((size_t)head_dim + 2) * sizeof(float);
    if (partition_size == 0) {
        *waves = split_wave_bound(kind, G, head_dim, path, ring);
        return split_prefix_bytes(num_seqs, *waves) + (size_t)*waves * 2 * cap * per_head;
    }
    const int mp = max_parts(max_blocks_per_seq, block_size, partition_size);
    if (mp <= 1) return 0;
    return (size_t)num_seqs * num_kv_heads * heads_per_kv * mp * per_head;
}

}  // namespace

extern "C" {

int pkv_version(void) { return 100; }

const char* pkv_error_string(int status) {
    switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch failure";
    case PKV_ERR_NO_BLOCKS: return "no free block in the pool";
    case PKV_ERR_CONTRACT: return "device-side contract broken (PKV_DEBUG_CHECKS)";
    default: return "unknown status";
    }
}

const char* pkv_last_error(void) { return g_msg; }

int pkv_decode_partition_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int max_blocks_per_seq, int partition_size) {
    (void)num_seqs;
    (void)num_q_heads;
    (void)num_kv_heads;
    (void)head_dim;
    (void)max_blocks_per_seq;
    if (block_size <= 0) return PKV_ERR_INVALID;
    if (!partition_ok(partition_size, block_size)) return PKV_ERR_INVALID;
    return partition_size;  // 0: balanced split sized at launch
}

size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int partition_size) {
    long long waves = 0;
    return decode_need(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, partition_size,
                       -1, 0, 0, &waves);
}

}  // extern "C"

namespace {

// paged_attention_decode with its workspace either given by the caller or, with
// use_static, the library's per-device static scratch (paged_attention_decode_static).
int decode_call(const char* fn, void* out, const void* query, const void* key_cache, const void* value_cache,
                const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                int dtype, int partition_size, void* workspace, size_t workspace_bytes, bool use_static, int path,
                int ring, void* stream) {
    int rc;
    if ((rc = check_pool(fn, num_kv_heads, head_dim, block_size, num_blocks, dtype)) != PKV_OK) return rc;
    if ((rc = check_heads(fn, num_q_heads, num_kv_heads)) != PKV_OK) return rc;
    if (num_seqs < 0) return set_error(PKV_ERR_INVALID, "%s: num_seqs must be >= 0 (got %d)", fn, num_seqs);
    if (max_blocks_per_seq <= 0)
        return set_error(PKV_ERR_INVALID, "%s: max_blocks_per_seq must be positive (got %d)", fn, max_blocks_per_seq);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return set_error(PKV_ERR_INVALID, "%s: scale must be finite and positive", fn);
    if (!partition_ok(partition_size, block_size))
        return set_error(PKV_ERR_INVALID, "%s: partition_size %d must be 0 or a positive multiple of block_size and 16",
                         fn, partition_size);
    if (path < 0 || path > 2 || (ring != 0 && ring != 2))
        return set_error(PKV_ERR_INVALID, "%s: inner_loop must be 0, 1 or 2 and ring 0 or 2", fn);
    if (path == 2 && dtype == PKV_F32)
        return set_error(PKV_ERR_UNSUPPORTED, "%s: the matrix-core path takes 16-bit types only", fn);
    if (num_seqs == 0) return PKV_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
        return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return set_error(PKV_ERR_INVALID, "%s: misaligned pointer (16 bytes for tensors, 4 for int32 arrays)", fn);
    const int mp = partition_size > 0 ? max_parts(max_blocks_per_seq, block_size, partition_size) : 0;
    const int G = num_q_heads / num_kv_heads;
    const long long grid = (long long)(mp > 0 ? mp : 1) * num_q_heads * num_seqs;  // bound on workgroups
    if (grid > 0x7fffffffLL) return set_error(PKV_ERR_INVALID, "%s: problem too large for one launch", fn);
    long long waves = 0;
    const size_t need = decode_need(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                    partition_size, dtype, path, ring, &waves);
    if (use_static) {
        if (need > pkv::kStaticScratchBytes)
            return set_error(PKV_ERR_WORKSPACE,
                             "%s: this call needs %zu bytes of scratch, beyond the %zu bytes of the static scratch; "
                             "use paged_attention_decode with a workspace",
                             fn, need, pkv::kStaticScratchBytes);
        workspace = nullptr;
        if (need > 0) {
            hipError_t e = pkv::static_scratch_address(&workspace);
            if (e != hipSuccess)
                return set_error(PKV_ERR_HIP, "%s: static scratch lookup failed: %s", fn, hipGetErrorString(e));
        }
    } else {
        if (need > 0 && (!workspace || workspace_bytes < need))
            return set_error(PKV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                             workspace ? workspace_bytes : (size_t)0);
        if (need > 0 && !aligned(workspace, 16))
            return set_error(PKV_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
    }

    pkv::DebugChecks dbg((hipStream_t)stream, pkv::debug_checks_requested());
    (void)dbg.tables(block_tables, context_lens, nullptr, num_seqs, max_blocks_per_seq, block_size, num_blocks, 0, 0);
    if (dbg.error() != hipSuccess) return hip_fail(dbg.error(), fn);

    pkv::DecodeParams p;
    p.guard = dbg.guard();
    p.out = out;
    p.q = query;
    p.kc = key_cache;
    p.vc = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.cu_q = nullptr;
    if (partition_size == 0) {
        p.starts = (long long*)workspace;
        p.notes = (pkv::MergeNote*)((char*)workspace + split_starts_bytes(num_seqs));
        p.ws = (float*)((char*)workspace + split_prefix_bytes(num_seqs, waves));
    } else {
        p.starts = nullptr;
        p.notes = nullptr;
        p.ws = (float*)workspace;
    }
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.G = G;
    p.D = head_dim;
    p.NB = num_blocks;
    p.MB = max_blocks_per_seq;
    p.BS = block_size;
    p.chunks = 1;
    p.part_tokens = partition_size;
    p.max_parts = mp;
    p.scale_log2 = scale * pkv::kLog2eHost;
    hipError_t e = pkv::launch_decode_path(p, dtype, path, ring, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return finish_checked(fn, dbg);
}

}  // namespace

extern "C" {

int paged_attention_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, float scale, int dtype, int partition_size, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return decode_call("paged_attention_decode", out, query, key_cache, value_cache, block_tables, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       scale, dtype, partition_size, workspace, workspace_bytes, false, 0, 0, stream);
}

int pkv_decode_variant(void* out, const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                       float scale, int dtype, int partition_size, void* workspace, size_t workspace_bytes,
                       int inner_loop, int ring, void* stream) {
    return decode_call("pkv_decode_variant", out, query, key_cache, value_cache, block_tables, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       scale, dtype, partition_size, workspace, workspace_bytes, false, inner_loop, ring, stream);
}

size_t pkv_decode_variant_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int max_blocks_per_seq, int partition_size, int dtype,
                                         int inner_loop, int ring) {
    long long waves = 0;
    return decode_need(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, partition_size,
                       dtype, inner_loop, ring, &waves);
}

int paged_attention_decode_static(void* out, const void* query, const void* key_cache, const void* value_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, float scale, int dtype, int partition_size, void* stream) {
    return decode_call("paged_attention_decode_static", out, query, key_cache, value_cache, block_tables,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, dtype, partition_size, nullptr, 0, true, 0, 0, stream);
}

int paged_attention_chunked(void* out, const void* query, const int32_t* cu_q_lens, int num_segs, int total_q,
                            int max_q_len, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int num_q_heads,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                            float scale, int dtype, void* stream) {
    static const char* fn = "paged_attention_chunked";
    int rc;
    if ((rc = check_pool(fn, num_kv_heads, head_dim, block_size, num_blocks, dtype)) != PKV_OK) return rc;
    if ((rc = check_heads(fn, num_q_heads, num_kv_heads)) != PKV_OK) return rc;
    if (dtype == PKV_F32) return set_error(PKV_ERR_UNSUPPORTED, "%s: fp32 is not supported (16-bit types only)", fn);
    if (num_segs < 0 || total_q < 0 || max_q_len < 0)
        return set_error(PKV_ERR_INVALID, "%s: num_segs, total_q and max_q_len must be >= 0", fn);
    if (max_blocks_per_seq <= 0)
        return set_error(PKV_ERR_INVALID, "%s: max_blocks_per_seq must be positive (got %d)", fn, max_blocks_per_seq);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return set_error(PKV_ERR_INVALID, "%s: scale must be finite and positive", fn);
    if (max_q_len > total_q) return set_error(PKV_ERR_INVALID, "%s: max_q_len exceeds total_q", fn);
    if (num_segs == 0 || total_q == 0 || max_q_len == 0) return PKV_OK;
    if (!out || !query || !cu_q_lens || !key_cache || !value_cache || !block_tables || !context_lens)
        return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(cu_q_lens, 4))
        return set_error(PKV_ERR_INVALID, "%s: misaligned pointer", fn);
    const int G = num_q_heads / num_kv_heads;
    const long long tiles = ((long long)max_q_len * G + 127) / 128;
    if (tiles * num_kv_heads * num_segs > 0x7fffffffLL)
        return set_error(PKV_ERR_INVALID, "%s: problem too large for one launch", fn);
    pkv::DebugChecks dbg((hipStream_t)stream, pkv::debug_checks_requested());
    (void)dbg.tables(block_tables, context_lens, cu_q_lens, num_segs, max_blocks_per_seq, block_size, num_blocks, total_q,
               max_q_len);
    if (dbg.error() != hipSuccess) return hip_fail(dbg.error(), fn);
    pkv::ChunkedParams p;
    p.guard = dbg.guard();
    p.out = out;
    p.q = query;
    p.cu_q_lens = cu_q_lens;
    p.kc = key_cache;
    p.vc = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.num_segs = num_segs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.G = G;
    p.D = head_dim;
    p.NB = num_blocks;
    p.MB = max_blocks_per_seq;
    p.BS = block_size;
    p.head_chunk = G;
    p.max_q_len = max_q_len;
    p.scale_log2 = scale * pkv::kLog2eHost;
    hipError_t e = pkv::launch_chunked(p, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return finish_checked(fn, dbg);
}

size_t pkv_mixed_workspace_size(int num_segs, int num_q_heads, int num_kv_heads, int head_dim, int block_size) {
    if (num_segs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
        head_dim <= 0 || block_size <= 0) {
        set_error(PKV_ERR_INVALID, "pkv_mixed_workspace_size: invalid arguments");
        return PKV_SIZE_INVALID;
    }
    if (num_segs == 0) return 0;
    long long heads_per_kv = 0;
    int cap = 0;
    record_shape(num_q_heads / num_kv_heads, &heads_per_kv, &cap);
    const long long waves = mixed_decode_waves();
    return split_prefix_bytes(num_segs, waves) + (size_t)waves * 2 * cap * ((size_t)head_dim + 2) * sizeof(float);
}

int paged_attention_mixed(void* out, const void* query, const int32_t* cu_q_lens, int num_segs, int total_q,
                          int max_q_len, const void* key_cache, const void* value_cache, const int32_t* block_tables,
                          const int32_t* context_lens, int num_q_heads, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, int max_blocks_per_seq, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    static const char* fn = "paged_attention_mixed";
    int rc;
    if ((rc = check_pool(fn, num_kv_heads, head_dim, block_size, num_blocks, dtype)) != PKV_OK) return rc;
    if ((rc = check_heads(fn, num_q_heads, num_kv_heads)) != PKV_OK) return rc;
    if (dtype == PKV_F32) return set_error(PKV_ERR_UNSUPPORTED, "%s: fp32 is not supported (16-bit types only)", fn);
    if (num_segs < 0 || total_q < 0 || max_q_len < 0)
        return set_error(PKV_ERR_INVALID, "%s: num_segs, total_q and max_q_len must be >= 0", fn);
    if (max_blocks_per_seq <= 0)
        return set_error(PKV_ERR_INVALID, "%s: max_blocks_per_seq must be positive (got %d)", fn, max_blocks_per_seq);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return set_error(PKV_ERR_INVALID, "%s: scale must be finite and positive", fn);
    if (max_q_len > total_q) return set_error(PKV_ERR_INVALID, "%s: max_q_len exceeds total_q", fn);
    if (num_segs == 0 || total_q == 0 || max_q_len == 0) return PKV_OK;
    if (!out || !query || !cu_q_lens || !key_cache || !value_cache || !block_tables || !context_lens)
        return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(cu_q_lens, 4))
        return set_error(PKV_ERR_INVALID, "%s: misaligned pointer", fn);
    const int G = num_q_heads / num_kv_heads;
    const long long tiles = ((long long)max_q_len * G + 127) / 128;
    if (tiles * num_kv_heads * num_segs + 8192 > 0x7fffffffLL ||
        (long long)num_segs * num_q_heads > 0x7fffffffLL)
        return set_error(PKV_ERR_INVALID, "%s: problem too large for one launch", fn);
    const size_t need = pkv_mixed_workspace_size(num_segs, num_q_heads, num_kv_heads, head_dim, block_size);
    if (!workspace || workspace_bytes < need)
        return set_error(PKV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                         workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return set_error(PKV_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);

    pkv::DebugChecks dbg((hipStream_t)stream, pkv::debug_checks_requested());
    (void)dbg.tables(block_tables, context_lens, cu_q_lens, num_segs, max_blocks_per_seq, block_size, num_blocks, total_q,
               max_q_len);
    if (dbg.error() != hipSuccess) return hip_fail(dbg.error(), fn);
    pkv::ChunkedParams c;
    c.guard = dbg.guard();
    c.out = out;
    c.q = query;
    c.cu_q_lens = cu_q_lens;
    c.kc = key_cache;
    c.vc = value_cache;
    c.block_tables = block_tables;
    c.context_lens = context_lens;
    c.num_segs = num_segs;
    c.Hq = num_q_heads;
    c.Hkv = num_kv_heads;
    c.G = G;
    c.D = head_dim;
    c.NB = num_blocks;
    c.MB = max_blocks_per_seq;
    c.BS = block_size;
    c.head_chunk = G;
    c.max_q_len = max_q_len;
    c.scale_log2 = scale * pkv::kLog2eHost;

    pkv::DecodeParams d;
    d.guard = dbg.guard();
    d.out = out;
    d.q = query;
    d.kc = key_cache;
    d.vc = value_cache;
    d.block_tables = block_tables;
    d.context_lens = context_lens;
    d.cu_q = cu_q_lens;
    d.starts = (long long*)workspace;
    d.notes = (pkv::MergeNote*)((char*)workspace + split_starts_bytes(num_segs));
    d.ws = (float*)((char*)workspace + split_prefix_bytes(num_segs, mixed_decode_waves()));
    d.S = num_segs;
    d.Hq = num_q_heads;
    d.Hkv = num_kv_heads;
    d.G = G;
    d.D = head_dim;
    d.NB = num_blocks;
    d.MB = max_blocks_per_seq;
    d.BS = block_size;
    d.chunks = 1;
    d.part_tokens = 0;
    d.max_parts = 0;
    d.scale_log2 = c.scale_log2;
    hipError_t e = pkv::launch_mixed(d, c, dtype, (long long)total_q - num_segs, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return finish_checked(fn, dbg);
}

int reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int dtype, void* stream) {
    static const char* fn = "reshape_and_cache";
    int rc;
    if ((rc = check_pool(fn, num_kv_heads, head_dim, block_size, num_blocks, dtype)) != PKV_OK) return rc;
    if (num_tokens < 0) return set_error(PKV_ERR_INVALID, "%s: num_tokens must be >= 0 (got %d)", fn, num_tokens);
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
        return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
        !aligned(slot_mapping, 8))
        return set_error(PKV_ERR_INVALID, "%s: misaligned pointer", fn);
    pkv::DebugChecks dbg((hipStream_t)stream, pkv::debug_checks_requested());
    (void)dbg.slots(slot_mapping, num_tokens, block_size, num_blocks);
    if (dbg.error() != hipSuccess) return hip_fail(dbg.error(), fn);
    pkv::CacheParams p;
    p.guard = dbg.guard();
    p.key = key;
    p.value = value;
    p.kc = key_cache;
    p.vc = value_cache;
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.Hkv = num_kv_heads;
    p.D = head_dim;
    p.BS = block_size;
    hipError_t e = pkv::launch_reshape_and_cache(p, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return finish_checked(fn, dbg);
}

int copy_blocks(void* const* key_caches, void* const* value_caches, int num_layers, const int64_t* block_mapping,
                int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype,
                void* stream) {
    static const char* fn = "copy_blocks";
    int rc;
    if ((rc = check_pool(fn, num_kv_heads, head_dim, block_size, num_blocks, dtype)) != PKV_OK) return rc;
    if (num_layers < 0 || num_pairs < 0)
        return set_error(PKV_ERR_INVALID, "%s: num_layers and num_pairs must be >= 0", fn);
    if (num_layers == 0 || num_pairs == 0) return PKV_OK;
    if (!key_caches || !value_caches || !block_mapping) return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned(block_mapping, 8)) return set_error(PKV_ERR_INVALID, "%s: misaligned block_mapping", fn);
    for (int l = 0; l < num_layers; ++l) {
        if (!key_caches[l] || !value_caches[l])
            return set_error(PKV_ERR_INVALID, "%s: null cache pointer for layer %d", fn, l);
        if (!aligned(key_caches[l], 16) || !aligned(value_caches[l], 16))
            return set_error(PKV_ERR_INVALID, "%s: misaligned cache pointer for layer %d", fn, l);
    }
    const int esz = dtype == PKV_F32 ? 4 : 2;
    pkv::DebugChecks dbg((hipStream_t)stream, pkv::debug_checks_requested());
    (void)dbg.copies(block_mapping, num_pairs, num_blocks);
    if (dbg.error() != hipSuccess) return hip_fail(dbg.error(), fn);
    pkv::CopyParams p;
    p.guard = dbg.guard();
    p.mapping = block_mapping;
    p.num_pairs = num_pairs;
    p.block_bytes = (size_t)num_kv_heads * block_size * head_dim * esz;
    for (int l0 = 0; l0 < num_layers; l0 += pkv::kMaxLayersPerLaunch) {
        const int nl = num_layers - l0 < pkv::kMaxLayersPerLaunch ? num_layers - l0 : pkv::kMaxLayersPerLaunch;
        for (int i = 0; i < nl; ++i) {
            p.k[i] = key_caches[l0 + i];
            p.v[i] = value_caches[l0 + i];
        }
        hipError_t e = pkv::launch_copy_blocks(p, nl, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    return finish_checked(fn, dbg);
}

int pkv_read_probe(const void* buf, size_t bytes, void* sink, void* stream) {
    static const char* fn = "pkv_read_probe";
    if (!buf || !sink) return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    if (bytes == 0 || bytes % 4096 != 0) return set_error(PKV_ERR_INVALID, "%s: bytes must be a positive multiple of 4096", fn);
    if (!aligned(buf, 16) || !aligned(sink, 4)) return set_error(PKV_ERR_INVALID, "%s: misaligned pointer", fn);
    hipError_t e = pkv::launch_read_probe(buf, bytes, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return PKV_OK;
}

}  // extern "C"
