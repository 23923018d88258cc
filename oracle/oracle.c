/*
 * oracle.c -- plain, slow, fp64 CPU reference for paged attention and its two
 * companion writes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may use this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no code, header, helper or table with the GPU library; the only
 * thing the two have in common is the pool layout that the library's header
 * defines as its interface:
 *
 *   key_cache   [num_blocks][num_kv_heads][block_size][head_dim]   (token-major tile)
 *   value_cache [num_blocks][num_kv_heads][head_dim][block_size]   (head_dim-major tile)
 *   block_tables int32 [num_seqs][max_blocks_per_seq], context_lens int32 [num_seqs]
 *   query / output [rows][num_q_heads][head_dim]
 *   slot = block * block_size + offset (int64; negative = no write)
 *
 * What it computes (sources: the three pages this project follows):
 *  - "每生成一个字都要把全部权重读一遍：从 vLLM 看 LLM 推理提速", section on paging the
 *    KV cache, blockwise attention equation and its figure: per block the scores
 *    s_j = q.K_j / sqrt(d_k), and the output is the softmax-weighted sum of the V
 *    blocks, which equals attention over the blocks concatenated in logical order;
 *    physical placement does not change the result.  So this oracle GATHERS every
 *    sequence's blocks through its block table into contiguous K and V and then
 *    runs plain dense softmax attention (one global softmax over all tokens).
 *  - "LLM 推理优化的系统视角：从 KV Cache 到调度", section 3.1, dense causal attention
 *    O_t = softmax(Q_t K_{1:t}^T / sqrt(d_h)) V_{1:t}: the chunked (prefill) rows
 *    attend to keys 0..pos with pos = ctx - q_len + i.
 *  - same page, section 3.2 and 4.1 (MHA / MQA / GQA): a group of query heads
 *    shares one K/V head; groups are contiguous, kv head = h / (Hq / Hkv).
 *  - page 1, copy-on-write paragraph: a shared block is copied whole to a fresh
 *    block before a sharer writes into it (copy_blocks).
 *  - "现代 LLM 推理引擎剖析", section 1.6: new K/V are written through slot_mapping
 *    (reshape_and_cache); section 1.3: block bytes = 2 x block_size x kv heads x
 *    head size x dtype bytes.
 *
 * All floating point is IEEE double.  Stored values are decoded exactly from
 * their bit patterns (fp32, IEEE binary16, bfloat16) by the decoders below.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_OK = 0, OR_EINVAL = -1, OR_ERANGE = -2, OR_ENOMEM = -3 };

/* ---- exact decoders -------------------------------------------------------- */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);    /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double dec_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load(const void* base, size_t i, int dt) {
    switch (dt) {
    case OR_F32: return (double)((const float*)base)[i];
    case OR_F16: return dec_f16(((const uint16_t*)base)[i]);
    default:     return dec_bf16(((const uint16_t*)base)[i]);
    }
}

static size_t esize(int dt) { return dt == OR_F32 ? 4 : 2; }

static int dtype_ok(int dt) { return dt == OR_F32 || dt == OR_F16 || dt == OR_BF16; }

/* K/V element addresses in the pool (see the layout in the header comment). */
static size_t k_index(int64_t blk, int h, int off, int d, int H, int BS, int D) {
    return (((size_t)blk * H + h) * BS + off) * D + d;
}
static size_t v_index(int64_t blk, int h, int off, int d, int H, int BS, int D) {
    return (((size_t)blk * H + h) * D + d) * BS + off;
}

/* Gather the first n logical tokens of one sequence's kv head g into
 * contiguous K[n][D], V[n][D].  Returns OR_ERANGE on a block id outside the pool. */
static int gather(double* K, double* V, const void* kc, const void* vc, const int32_t* table, int n, int g,
                  int Hkv, int D, int BS, int NB, int dt) {
    for (int t = 0; t < n; ++t) {
        int32_t blk = table[t / BS];
        int off = t % BS;
        if (blk < 0 || blk >= NB) return OR_ERANGE;
        for (int d = 0; d < D; ++d) {
            K[(size_t)t * D + d] = load(kc, k_index(blk, g, off, d, Hkv, BS, D), dt);
            V[(size_t)t * D + d] = load(vc, v_index(blk, g, off, d, Hkv, BS, D), dt);
        }
    }
    return OR_OK;
}

/* Dense softmax attention of one query row over keys 0..n-1 (n >= 0):
 *   x_t = scale * sum_d q[d] K[t][d];  w_t = exp(x_t - max x);  o = sum w_t V_t / sum w_t.
 * n == 0 gives o = 0 (empty sum).  x is scratch of n doubles. */
static void attend(double* o, const double* q, const double* K, const double* V, int n, int D, double scale,
                   double* x) {
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) return;
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += q[d] * K[(size_t)t * D + d];
        x[t] = scale * acc;
        if (x[t] > m) m = x[t];
    }
    double den = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(x[t] - m);
        den += w;
        for (int d = 0; d < D; ++d) o[d] += w * V[(size_t)t * D + d];
    }
    for (int d = 0; d < D; ++d) o[d] /= den;
}

static int geometry_ok(int Hq, int Hkv, int D, int BS, int NB, int MB, int dt) {
    return Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && D > 0 && BS > 0 && NB > 0 && MB > 0 && dtype_ok(dt);
}

/* ---- decode ------------------------------------------------------------------
 * out[s][h][:] for every sequence s and query head h (fp64).  Sequence s
 * attends to its context_lens[s] tokens (the newest token included). */
int oracle_decode(double* out, const void* query, const void* key_cache, const void* value_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                  int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                  double scale, int dtype) {
    const int S = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads, D = head_dim, BS = block_size;
    if (S < 0 || !geometry_ok(Hq, Hkv, D, BS, num_blocks, max_blocks_per_seq, dtype)) return OR_EINVAL;
    for (int s = 0; s < S; ++s)
        if (context_lens[s] < 0 || context_lens[s] > max_blocks_per_seq * BS) return OR_ERANGE;
    const int G = Hq / Hkv;
    int status = OR_OK;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < S; ++s) {
        for (int g = 0; g < Hkv; ++g) {
            int n = context_lens[s];
            size_t cap = (size_t)(n > 0 ? n : 1);
            double* K = (double*)malloc(cap * D * sizeof(double));
            double* V = (double*)malloc(cap * D * sizeof(double));
            double* x = (double*)malloc(cap * sizeof(double));
            double* q = (double*)malloc((size_t)D * sizeof(double));
            if (!K || !V || !x || !q) {
#pragma omp atomic write
                status = OR_ENOMEM;
            } else if (gather(K, V, key_cache, value_cache, block_tables + (size_t)s * max_blocks_per_seq, n, g,
                              Hkv, D, BS, num_blocks, dtype) != OR_OK) {
#pragma omp atomic write
                status = OR_ERANGE;
            } else {
                for (int j = 0; j < G; ++j) {
                    int h = g * G + j;
                    for (int d = 0; d < D; ++d) q[d] = load(query, ((size_t)s * Hq + h) * D + d, dtype);
                    attend(out + ((size_t)s * Hq + h) * D, q, K, V, n, D, scale, x);
                }
            }
            free(K); free(V); free(x); free(q);
        }
    }
    return status;
}

/* ---- chunked prefill -----------------------------------------------------------
 * Segment i owns query rows cu_q_lens[i] .. cu_q_lens[i+1]-1 and attends to
 * context_lens[i] tokens (its cached prefix plus its own chunk, already written).
 * Row r of the segment sits at position pos = ctx - q_len + r and sees keys
 * 0..pos (causal).  out is [total_q][Hq][D] fp64. */
int oracle_chunked(double* out, const void* query, const int32_t* cu_q_lens, int num_segs,
                   const void* key_cache, const void* value_cache, const int32_t* block_tables,
                   const int32_t* context_lens, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                   int num_blocks, int max_blocks_per_seq, double scale, int dtype) {
    const int Hq = num_q_heads, Hkv = num_kv_heads, D = head_dim, BS = block_size;
    if (num_segs < 0 || !geometry_ok(Hq, Hkv, D, BS, num_blocks, max_blocks_per_seq, dtype)) return OR_EINVAL;
    for (int i = 0; i < num_segs; ++i) {
        int L = cu_q_lens[i + 1] - cu_q_lens[i];
        if (L < 0 || context_lens[i] < L || context_lens[i] > max_blocks_per_seq * BS) return OR_ERANGE;
    }
    const int G = Hq / Hkv;
    int status = OR_OK;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int i = 0; i < num_segs; ++i) {
        for (int g = 0; g < Hkv; ++g) {
            int n = context_lens[i];
            int L = cu_q_lens[i + 1] - cu_q_lens[i];
            size_t cap = (size_t)(n > 0 ? n : 1);
            double* K = (double*)malloc(cap * D * sizeof(double));
            double* V = (double*)malloc(cap * D * sizeof(double));
            double* x = (double*)malloc(cap * sizeof(double));
            double* q = (double*)malloc((size_t)D * sizeof(double));
            if (!K || !V || !x || !q) {
#pragma omp atomic write
                status = OR_ENOMEM;
            } else if (gather(K, V, key_cache, value_cache, block_tables + (size_t)i * max_blocks_per_seq, n, g,
                              Hkv, D, BS, num_blocks, dtype) != OR_OK) {
#pragma omp atomic write
                status = OR_ERANGE;
            } else {
                for (int r = 0; r < L; ++r) {
                    size_t row = (size_t)cu_q_lens[i] + r;
                    int pos = n - L + r;
                    for (int j = 0; j < G; ++j) {
                        int h = g * G + j;
                        for (int d = 0; d < D; ++d) q[d] = load(query, (row * Hq + h) * D + d, dtype);
                        attend(out + (row * Hq + h) * D, q, K, V, pos + 1, D, scale, x);
                    }
                }
            }
            free(K); free(V); free(x); free(q);
        }
    }
    return status;
}

/* ---- reshape_and_cache -----------------------------------------------------------
 * Token i with slot_mapping[i] >= 0 is stored at block slot/BS, offset slot%BS:
 * its K row into the token-major K tile, its V row into the head_dim-major V
 * tile.  A byte copy; no conversion.  key/value are [num_tokens][Hkv][D]. */
int oracle_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                             const int64_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                             int block_size, int num_blocks, int dtype) {
    const int H = num_kv_heads, D = head_dim, BS = block_size;
    if (num_tokens < 0 || H <= 0 || D <= 0 || BS <= 0 || num_blocks <= 0 || !dtype_ok(dtype)) return OR_EINVAL;
    const size_t es = esize(dtype);
    for (int i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        if (slot >= (int64_t)num_blocks * BS) return OR_ERANGE;
        int64_t blk = slot / BS;
        int off = (int)(slot % BS);
        for (int h = 0; h < H; ++h)
            for (int d = 0; d < D; ++d) {
                size_t src = ((size_t)i * H + h) * D + d;
                memcpy((char*)key_cache + k_index(blk, h, off, d, H, BS, D) * es, (const char*)key + src * es, es);
                memcpy((char*)value_cache + v_index(blk, h, off, d, H, BS, D) * es, (const char*)value + src * es, es);
            }
    }
    return OR_OK;
}

/* ---- copy_blocks ------------------------------------------------------------------
 * For every layer and every (src, dst) pair of block_mapping ([num_pairs][2]),
 * the whole block dst of K and of V becomes a copy of block src. */
int oracle_copy_blocks(void** key_caches, void** value_caches, int num_layers, const int64_t* block_mapping,
                       int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype) {
    if (num_layers < 0 || num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0 || !dtype_ok(dtype))
        return OR_EINVAL;
    const size_t bytes = (size_t)num_kv_heads * block_size * head_dim * esize(dtype);
    for (int p = 0; p < num_pairs; ++p) {
        int64_t src = block_mapping[2 * p], dst = block_mapping[2 * p + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return OR_ERANGE;
    }
    for (int l = 0; l < num_layers; ++l)
        for (int p = 0; p < num_pairs; ++p) {
            int64_t src = block_mapping[2 * p], dst = block_mapping[2 * p + 1];
            memcpy((char*)key_caches[l] + dst * bytes, (const char*)key_caches[l] + src * bytes, bytes);
            memcpy((char*)value_caches[l] + dst * bytes, (const char*)value_caches[l] + src * bytes, bytes);
        }
    return OR_OK;
}

/* ---- sizes ------------------------------------------------------------------------
 * Per token over all layers: 2 (K and V) x layers x kv heads x head dim x bytes
 * ("LLM 推理优化的系统视角", section 3.2).  Per block and layer: 2 x block_size x kv
 * heads x head size x bytes ("现代 LLM 推理引擎剖析", section 1.3). */
long long oracle_kv_bytes_per_token(int num_layers, int num_kv_heads, int head_dim, int elem_bytes) {
    return 2LL * num_layers * num_kv_heads * head_dim * elem_bytes;
}

long long oracle_kv_bytes_per_block(int block_size, int num_kv_heads, int head_dim, int elem_bytes) {
    return 2LL * block_size * num_kv_heads * head_dim * elem_bytes;
}

/* Decode one stored element to double (lets tests pin the decoders). */
double oracle_decode_element(const void* base, long long index, int dtype) {
    return load(base, (size_t)index, dtype);
}

/* Threads used by the parallel loops above (timing only: every (sequence, head)
 * row is computed on its own, so results do not depend on it). */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_max_threads(void) { return omp_get_max_threads(); }
