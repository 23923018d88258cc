// block_manager.cpp -- host-side manager of the paged KV pool (include/pkv_block_manager.h).
//
// The KV cache manager keeps a queue of free blocks and a block table per
// sequence, allocating blocks on demand ("现代 LLM 推理引擎剖析", section 1.3).
// Forked sequences share blocks through reference counts, and a write into a
// shared last block first copies it ("每生成一个字都要把全部权重读一遍", copy-on-write
// paragraph).  Full prompt blocks can be found again by a hash chained from the
// previous block's hash and the block's token ids ("现代 LLM 推理引擎剖析", section 2.2).
//
// Data structures: the free queue is an intrusive doubly linked list over block
// ids (O(1) removal when a prefix-cache hit revives a free block); cached blocks
// keep their token ids for the hit check; sequences live in a hash map.
#include "pkv.h"
#include "pkv_block_manager.h"

#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "internal.h"

using pkv::set_error;

struct pkv_block_manager {
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t len = 0;
    };
    int nb = 0, bs = 0;
    std::vector<int32_t> ref, prev, next;
    std::vector<uint8_t> in_free, hashed;
    std::vector<uint64_t> hash;
    std::vector<int32_t> tokens;  // [nb][bs] token ids of hashed blocks
    int32_t head = -1, tail = -1;
    int nfree = 0;
    std::unordered_map<uint64_t, int32_t> block_of;
    std::unordered_map<int, Seq> seqs;

    // ---- free queue ----------------------------------------------------------------
    void push_tail(int32_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0)
            next[tail] = b;
        else
            head = b;
        tail = b;
        in_free[b] = 1;
        ++nfree;
    }
    void unlink(int32_t b) {
        if (prev[b] >= 0)
            next[prev[b]] = next[b];
        else
            head = next[b];
        if (next[b] >= 0)
            prev[next[b]] = prev[b];
        else
            tail = prev[b];
        in_free[b] = 0;
        --nfree;
    }
    // head of the queue, now referenced once; a block handed out again loses its hash
    int32_t allocate() {
        const int32_t b = head;
        unlink(b);
        if (hashed[b]) {
            auto it = block_of.find(hash[b]);
            if (it != block_of.end() && it->second == b) block_of.erase(it);
            hashed[b] = 0;
        }
        ref[b] = 1;
        return b;
    }
    void release(int32_t b) {
        if (--ref[b] == 0) push_tail(b);
    }
};

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

// FNV-1a over bytes, continuing from h
uint64_t fnv1a(const uint8_t* p, size_t n, uint64_t h) {
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= kFnvPrime;
    }
    return h;
}

// hash of a full block: previous hash (8 bytes LE) then the token ids (int32 LE)
uint64_t block_hash(uint64_t prev, const int32_t* toks, int bs) {
    uint8_t buf[8];
    for (int i = 0; i < 8; ++i) buf[i] = (uint8_t)(prev >> (8 * i));
    uint64_t h = fnv1a(buf, 8, kFnvOffset);
    for (int t = 0; t < bs; ++t) {
        const uint32_t u = (uint32_t)toks[t];
        const uint8_t b4[4] = {(uint8_t)u, (uint8_t)(u >> 8), (uint8_t)(u >> 16), (uint8_t)(u >> 24)};
        h = fnv1a(b4, 4, h);
    }
    return h;
}

pkv_block_manager::Seq* find_seq(pkv_block_manager* bm, int seq, const char* fn) {
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) {
        set_error(PKV_ERR_INVALID, "%s: no sequence %d", fn, seq);
        return nullptr;
    }
    return &it->second;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int num_blocks, int block_size) {
    if (num_blocks <= 0 || block_size <= 0) {
        set_error(PKV_ERR_INVALID, "pkv_bm_create: num_blocks and block_size must be positive");
        return nullptr;
    }
    auto* bm = new (std::nothrow) pkv_block_manager;
    if (!bm) return nullptr;
    bm->nb = num_blocks;
    bm->bs = block_size;
    bm->ref.assign(num_blocks, 0);
    bm->prev.assign(num_blocks, -1);
    bm->next.assign(num_blocks, -1);
    bm->in_free.assign(num_blocks, 0);
    bm->hashed.assign(num_blocks, 0);
    bm->hash.assign(num_blocks, 0);
    bm->tokens.assign((size_t)num_blocks * block_size, 0);
    for (int b = 0; b < num_blocks; ++b) bm->push_tail(b);
    return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_num_free(const pkv_block_manager* bm) { return bm ? bm->nfree : PKV_ERR_INVALID; }

int pkv_bm_add_sequence(pkv_block_manager* bm, int seq, const int32_t* prompt, int n, int* cached_tokens) {
    static const char* fn = "pkv_bm_add_sequence";
    if (!bm || n < 0 || (n > 0 && !prompt)) return set_error(PKV_ERR_INVALID, "%s: bad arguments", fn);
    if (bm->seqs.count(seq)) return set_error(PKV_ERR_INVALID, "%s: sequence %d exists", fn, seq);
    pkv_block_manager::Seq s;
    if (prompt) {
        const int bs = bm->bs;
        uint64_t h = kFnvOffset;
        for (int i = 0; (i + 1) * bs <= n; ++i) {
            h = block_hash(h, prompt + (size_t)i * bs, bs);
            auto it = bm->block_of.find(h);
            if (it == bm->block_of.end()) break;
            const int32_t b = it->second;
            if (std::memcmp(&bm->tokens[(size_t)b * bs], prompt + (size_t)i * bs, sizeof(int32_t) * bs) != 0) break;
            if (bm->ref[b] == 0) bm->unlink(b);
            ++bm->ref[b];
            s.blocks.push_back(b);
        }
        s.len = (int64_t)s.blocks.size() * bs;
    }
    if (cached_tokens) *cached_tokens = (int)s.len;
    bm->seqs.emplace(seq, std::move(s));
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int parent, int child) {
    static const char* fn = "pkv_bm_fork";
    if (!bm) return set_error(PKV_ERR_INVALID, "%s: null manager", fn);
    auto* p = find_seq(bm, parent, fn);
    if (!p) return PKV_ERR_INVALID;
    if (bm->seqs.count(child)) return set_error(PKV_ERR_INVALID, "%s: sequence %d exists", fn, child);
    pkv_block_manager::Seq c = *p;
    for (int32_t b : c.blocks) ++bm->ref[b];
    bm->seqs.emplace(child, std::move(c));
    return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int seq, int n, int64_t* slots_out, int64_t* copies_out, int max_copies,
                  int* num_copies) {
    static const char* fn = "pkv_bm_append";
    if (!bm || n < 0 || (n > 0 && !slots_out) || max_copies < 0 || (max_copies > 0 && !copies_out))
        return set_error(PKV_ERR_INVALID, "%s: bad arguments", fn);
    auto* s = find_seq(bm, seq, fn);
    if (!s) return PKV_ERR_INVALID;
    const int bs = bm->bs;
    const int64_t off0 = s->len % bs;
    const bool cow = n > 0 && off0 != 0 && bm->ref[s->blocks.back()] > 1;
    const int64_t have = (s->len + bs - 1) / bs, need_total = (s->len + n + bs - 1) / bs;
    const int64_t fresh = need_total - have + (cow ? 1 : 0);
    if (fresh > bm->nfree)
        return set_error(PKV_ERR_NO_BLOCKS, "%s: %lld blocks needed, %d free", fn, (long long)fresh, bm->nfree);
    if (cow && max_copies < 1) return set_error(PKV_ERR_INVALID, "%s: a copy is needed but max_copies is 0", fn);
    int nc = 0;
    if (cow) {  // copy the shared last block before writing into it
        const int32_t old = s->blocks.back();
        const int32_t fresh_b = bm->allocate();
        copies_out[0] = old;
        copies_out[1] = fresh_b;
        nc = 1;
        --bm->ref[old];
        s->blocks.back() = fresh_b;
    }
    for (int i = 0; i < n; ++i) {
        const int64_t off = s->len % bs;
        if (off == 0) s->blocks.push_back(bm->allocate());
        slots_out[i] = (int64_t)s->blocks.back() * bs + off;
        ++s->len;
    }
    if (num_copies) *num_copies = nc;
    return PKV_OK;
}

int pkv_bm_commit_prompt(pkv_block_manager* bm, int seq, const int32_t* prompt, int n, int* added) {
    static const char* fn = "pkv_bm_commit_prompt";
    if (!bm || n < 0 || (n > 0 && !prompt)) return set_error(PKV_ERR_INVALID, "%s: bad arguments", fn);
    auto* s = find_seq(bm, seq, fn);
    if (!s) return PKV_ERR_INVALID;
    const int bs = bm->bs;
    const int64_t full = (n < s->len ? n : s->len) / bs;
    uint64_t h = kFnvOffset;
    int count = 0;
    for (int64_t i = 0; i < full; ++i) {
        h = block_hash(h, prompt + (size_t)i * bs, bs);
        const int32_t b = s->blocks[i];
        if (bm->hashed[b] || bm->block_of.count(h)) continue;
        bm->hashed[b] = 1;
        bm->hash[b] = h;
        std::memcpy(&bm->tokens[(size_t)b * bs], prompt + (size_t)i * bs, sizeof(int32_t) * bs);
        bm->block_of.emplace(h, b);
        ++count;
    }
    if (added) *added = count;
    return PKV_OK;
}

int pkv_bm_free_sequence(pkv_block_manager* bm, int seq) {
    static const char* fn = "pkv_bm_free_sequence";
    if (!bm) return set_error(PKV_ERR_INVALID, "%s: null manager", fn);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "%s: no sequence %d", fn, seq);
    const auto& blocks = it->second.blocks;
    for (size_t i = blocks.size(); i-- > 0;) bm->release(blocks[i]);
    bm->seqs.erase(it);
    return PKV_OK;
}

int64_t pkv_bm_context_len(const pkv_block_manager* bm, int seq) {
    if (!bm) return set_error(PKV_ERR_INVALID, "pkv_bm_context_len: null manager");
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "pkv_bm_context_len: no sequence %d", seq);
    return it->second.len;
}

int pkv_bm_block_table(const pkv_block_manager* bm, int seq, int32_t* out, int max_blocks, int32_t pad_value,
                       int* num_blocks) {
    static const char* fn = "pkv_bm_block_table";
    if (!bm || max_blocks < 0 || (max_blocks > 0 && !out)) return set_error(PKV_ERR_INVALID, "%s: bad arguments", fn);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "%s: no sequence %d", fn, seq);
    const auto& blocks = it->second.blocks;
    if ((int64_t)blocks.size() > max_blocks)
        return set_error(PKV_ERR_INVALID, "%s: %zu blocks do not fit in %d", fn, blocks.size(), max_blocks);
    for (int i = 0; i < max_blocks; ++i) out[i] = i < (int)blocks.size() ? blocks[i] : pad_value;
    if (num_blocks) *num_blocks = (int)blocks.size();
    return PKV_OK;
}

int pkv_bm_refcount(const pkv_block_manager* bm, int block) {
    if (!bm || block < 0 || block >= bm->nb) return set_error(PKV_ERR_INVALID, "pkv_bm_refcount: bad block");
    return bm->ref[block];
}

int pkv_bm_free_queue(const pkv_block_manager* bm, int32_t* out, int max_n) {
    if (!bm || max_n < 0 || (max_n > 0 && !out)) return set_error(PKV_ERR_INVALID, "pkv_bm_free_queue: bad arguments");
    int k = 0;
    for (int32_t b = bm->head; b >= 0 && k < max_n; b = bm->next[b]) out[k++] = b;
    return k;
}

}  // extern "C"
