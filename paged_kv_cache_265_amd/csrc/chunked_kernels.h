// chunked_kernels.h -- causal attention of chunked-prefill segments over the paged
// pool, gfx950 (launched by chunked.hip; also one half of the mixed launch).
//
// A long prompt is cut into chunks that run inside the flattened batch
// ("现代 LLM 推理引擎剖析", sections 1.4 and 2.1).  Query row r of a segment with L
// rows and n cached tokens (its own chunk included) sits at position n - L + r and
// attends to tokens 0 .. n - L + r (dense causal attention, "LLM 推理优化的系统视角",
// section 3.1), through the segment's block table.
//
// Rows are (query token, query head of the kv group) pairs, head fastest, so that
// the heads sharing one kv head share every K/V tile.  A workgroup of 4 waves takes
// 128 consecutive rows of one (segment, kv head); each wave owns 32 of them (two
// 16-row matrix-core columns), so every K/V operand read from LDS serves 32 rows.
// The keys go by in steps of 32 (two pool blocks of 16 tokens, one of 32, or four of
// 8): the workgroup stages a step's K and V into LDS once, double-buffered, and every
// wave folds it into its rows with an online softmax:
//   S^T = K Q^T        16x16x32 matrix cores, 16 keys x 16 rows per product
//   O^T += V^T P^T     16x16x32 matrix cores over all 32 keys of the step, P split
//                      into high and low 16-bit parts so that it keeps fp32 accuracy
// LDS layouts (rows padded so that the lanes of one read hit distinct banks):
//   K: [32 keys][D] as in the pool tile, rows padded by 32 bytes
//   V: [D][4 groups][8], rows padded by 16 bytes: group g holds keys 4g..4g+3 of the step's first 16 keys,
//      then keys 16+4g..16+4g+3 -- exactly the 8 keys whose probabilities lane group
//      g holds after the score product, so one 16-byte read is one matrix-core operand.
#pragma once

#include "device.h"
#include "internal.h"

namespace pkv {

namespace {

constexpr int NW = 4;                  // waves per workgroup
constexpr int NH = 2;                  // 16-row tiles per wave
constexpr int ROWS_PER_WAVE = 16 * NH;
constexpr int ROWS_PER_WG = NW * ROWS_PER_WAVE;
constexpr int KSTEP = 2 * kTileTokens; // keys per step: two 16-key halves

template <int D>
struct ChunkLds {
    // K rows padded by 32 bytes: the 32 lanes of a 16-byte K read (16 key rows x two
    // 16-byte columns) then fall on distinct banks; with 16 bytes of padding two of
    // them shared banks (MI355X counters on the long mixed batch: LDS bank-conflict
    // cycles 4.5e7 -> 2.7e7)
    static constexpr int KROW = D * 2 + 32;      // bytes per key row of K
    static constexpr int VROW = 4 * 16 + 16;     // bytes per head_dim row of V
    static constexpr int KBYTES = KSTEP * KROW;
    static constexpr int VBYTES = D * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int CHUNKS = KSTEP * D * 2 / 16 / (NW * 64);  // 16-byte K (and V) pieces per thread
};

// BS: tokens per KV block (8, 16 or 32); a step's 32 keys span KSTEP / BS blocks
// Workgroup `idx` of the chunked grid (tile, kv head, segment), with the stage
// buffers `lds`.  With skip_single, one-row segments are left alone (the mixed
// launch runs them as decode sequences).
template <int K, int D, int BS>
__device__ __forceinline__ void chunked_tile(const ChunkedParams& p, int idx, char* lds, bool skip_single) {
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    using Lds = ChunkLds<D>;
    constexpr uint32_t kTile = BS * D * 2;  // bytes of one (block, kv head) tile
    constexpr int NBS = KSTEP / BS;         // blocks per step
    constexpr int kPieces = (int)(kTile / 16);
    static_assert(kPieces % 64 == 0, "a wave's 64 pieces stay inside one block");

    const int G = p.G;
    const int tiles = (p.max_q_len * G + ROWS_PER_WG - 1) / ROWS_PER_WG;
    const int tile = idx % tiles;
    idx /= tiles;
    const int kvh = idx % p.Hkv;
    const int seg = idx / p.Hkv;

    const int qb0 = p.cu_q_lens[seg];
    const int L = p.cu_q_lens[seg + 1] - qb0;
    if (skip_single && L == 1) return;  // whole workgroup, before any barrier
    const int n = p.context_lens[seg];
    const int nrows = L * G;
    const int wg_row0 = tile * ROWS_PER_WG;
    if (wg_row0 >= nrows) return;  // whole workgroup idle, before any barrier
    const int nblk = (n + BS - 1) / BS;
    // keys the workgroup needs: 0 .. position of its last live row
    const int wg_last = min(wg_row0 + ROWS_PER_WG, nrows) - 1;
    const int nsteps = (n - L + wg_last / G) / KSTEP + 1;

    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = lane_id();
    const int col = lane & 15;
    const int gq = lane >> 4;
    const int row0 = wg_row0 + w * ROWS_PER_WAVE;
    const bool wave_live = row0 < nrows;
    // positions of the wave's first and last live rows (rows are sorted by position)
    const int wave_first_pos = n - L + row0 / G;
    const int wave_last_pos = n - L + (min(row0 + ROWS_PER_WAVE, nrows) - 1) / G;

    // this lane's rows: Q as the B operand of the score product; dead rows see
    // every key with a zero query (finite, never stored)
    int pos[NH];
    uint4 qv[NH][KS];
    const uint16_t* qp = (const uint16_t*)p.q;
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        const int r = row0 + ht * 16 + col;
        const bool live = r < nrows;
        const int tok = live ? r / G : 0;
        const int j = live ? r - tok * G : 0;
        pos[ht] = live ? n - L + tok : n - 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qv[ht][ks] = live ? *(const uint4*)(qp + ((size_t)(qb0 + tok) * p.Hq + kvh * G + j) * D + (gq + 4 * ks) * 8)
                              : make_uint4(0, 0, 0, 0);
    }
    float m[NH], l[NH];
    f32x4 acc[NH][DT];
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        m[ht] = kNegInf;
        l[ht] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- staging: this thread's 16-byte pieces of K and V for one step -------------
    const int32_t* table = p.block_tables + (size_t)seg * p.MB;
    struct Staged {
        uint4 k[Lds::CHUNKS], v[Lds::CHUNKS];
    };
    // loads of blocks past the context are empty (zero bytes, no memory access), so
    // every step issues the same loads and the wait before staging counts exactly
    auto fetch = [&](int step, Staged& r) {
        const int b0 = step * NBS;
        rsrc_t kr[NBS], vr[NBS];
#pragma unroll
        for (int b = 0; b < NBS; ++b) {
            const bool live = b0 + b < nblk;
            const int ph = live ? scalar_load(table, (size_t)uniform(b0 + b)) : 0;
            const size_t t = ((size_t)ph * p.Hkv + kvh) * kTile;
            kr[b] = tile_rsrc((const char*)p.kc + t, live ? kTile : 0);
            vr[b] = tile_rsrc((const char*)p.vc + t, live ? kTile : 0);
        }
#pragma unroll
        for (int i = 0; i < Lds::CHUNKS; ++i) {
            const int c = tid + i * NW * 64;  // piece c of the step lies in block c / kPieces
            const uint32_t off = (uint32_t)(c % kPieces) * 16;
            // a wave's 64 pieces never straddle two blocks: the block is wave-uniform,
            // and picking its resources is a chain of scalar selects
            const int blk = uniform(c / kPieces);
            rsrc_t k = kr[0], v = vr[0];
#pragma unroll
            for (int b = 1; b < NBS; ++b)
                if (blk == b) {
                    k = kr[b];
                    v = vr[b];
                }
            r.k[i] = stream_load16(k, off);
            r.v[i] = stream_load16(v, off);
        }
    };
    auto stage = [&](int step, const Staged& r, int buf) {
        char* kl = lds + buf * Lds::STAGE;
        char* vl = kl + Lds::KBYTES;
#pragma unroll
        for (int i = 0; i < Lds::CHUNKS; ++i) {
            const int c = tid + i * NW * 64;
            const int blk = c / kPieces;
            const int off = (c % kPieces) * 16;
            // K: key row (within the step), 16-byte column
            const int key = blk * BS + off / (D * 2);
            *(uint4*)(kl + key * Lds::KROW + off % (D * 2)) = r.k[i];
            // V: head_dim row d, keys kk .. kk+7 of the step (8 h .. 8 h + 7 of block
            // blk); slots past the context may hold anything and are zeroed
            const int d = off / (BS * 2);
            const int h = (off % (BS * 2)) / 16;
            const int kk = blk * BS + 8 * h;
            uint4 v = r.v[i];
            const int tok0 = step * KSTEP + kk;
            if (tok0 + 8 > n) {
                uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (tok0 + e >= n) u[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                v = make_uint4(u[0], u[1], u[2], u[3]);
            }
            // row d of the LDS V tile: 16-byte chunk j holds keys 4j .. 4j+3 of the
            // step's first 16-key half, then the same keys of its second half
            const int jj = (kk % kTileTokens) / 4;
            char* vrow = vl + d * Lds::VROW + (kk / kTileTokens) * 8;
            *(uint2*)(vrow + jj * 16) = make_uint2(v.x, v.y);
            *(uint2*)(vrow + (jj + 1) * 16) = make_uint2(v.z, v.w);
        }
    };

    // ---- one step: 32 keys into this wave's 32 rows ----------------------------------
    auto fold = [&](int step, int buf) {
        const char* kl = lds + buf * Lds::STAGE;
        const char* vl = kl + Lds::KBYTES;
        const int key0 = step * KSTEP;
        // four independent score chains (2 key halves x 2 row tiles) per k-step, so
        // consecutive matrix-core products never wait on each other
        uint4 kf[2][KS];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[kh][ks] = *(const uint4*)(kl + (kh * kTileTokens + col) * Lds::KROW + (gq + 4 * ks) * 16);
        f32x4 sc[2][NH];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int ht = 0; ht < NH; ++ht) sc[kh][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int ht = 0; ht < NH; ++ht) sc[kh][ht] = mma_16x16x32<K>(kf[kh][ks], qv[ht][ks], sc[kh][ht]);
        // V fragments, read while the first softmax runs
        uint4 vf[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[dt] = *(const uint4*)(vl + (dt * 16 + col) * Lds::VROW + gq * 16);
        // keys of this lane's eight scores: key0 + 4 gq + j and key0 + 16 + 4 gq + j
        const bool masked = key0 + KSTEP - 1 > wave_first_pos;
        const float c = p.scale_log2;
        // row tile by row tile: the P.V products of one tile run on the matrix
        // cores while the next tile's softmax runs on the vector ALU
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            float s[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[j] = sc[0][ht][j];
                s[4 + j] = sc[1][ht][j];
            }
            if (masked) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (key0 + 4 * gq + j > pos[ht]) s[j] = kNegInf;
                    if (key0 + kTileTokens + 4 * gq + j > pos[ht]) s[4 + j] = kNegInf;
                }
            }
            float bm = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
            bm = xor_max(bm, 16);
            bm = xor_max(bm, 32);
            bm *= c;  // the scale is positive: the max of the scaled scores
            // key 0 is visible to every row, so m is finite from the first step on
            if (__ballot(bm > m[ht] + kRescaleSlack)) {
                const float mn = fmaxf(m[ht], bm);
                const float alpha = fast_exp2(m[ht] - mn);
                l[ht] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[ht][dt] *= alpha;
                m[ht] = mn;
            }
            const float off = -m[ht];
            float pr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pr[j] = fast_exp2(__builtin_fmaf(s[j], c, off));
            l[ht] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
            const uint2 h0 = pack4<K>(pr[0], pr[1], pr[2], pr[3]);
            const uint2 h1 = pack4<K>(pr[4], pr[5], pr[6], pr[7]);
            const uint2 l0 = pack4<K>(pr[0] - lo16<K>(h0.x), pr[1] - hi16<K>(h0.x), pr[2] - lo16<K>(h0.y),
                                      pr[3] - hi16<K>(h0.y));
            const uint2 l1 = pack4<K>(pr[4] - lo16<K>(h1.x), pr[5] - hi16<K>(h1.x), pr[6] - lo16<K>(h1.y),
                                      pr[7] - hi16<K>(h1.y));
            const uint4 phi = make_uint4(h0.x, h0.y, h1.x, h1.y);
            const uint4 plo = make_uint4(l0.x, l0.y, l1.x, l1.y);
            // high parts, then the remainders: an accumulator is reused DT products later
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[ht][dt] = mma_16x16x32<K>(vf[dt], phi, acc[ht][dt]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[ht][dt] = mma_16x16x32<K>(vf[dt], plo, acc[ht][dt]);
        }
    };

    // step s lives in LDS buffer s % 2; its loads were issued two steps earlier
    // into register set s % 2
    Staged r0, r1;
    fetch(0, r0);
    fetch(1, r1);
    stage(0, r0, 0);
    __syncthreads();
    for (int step = 0; step < nsteps; step += 2) {
        fetch(step + 2, r0);
        // a wave whose rows all lie before this step's first key has nothing to fold
        if (wave_live && step * KSTEP <= wave_last_pos) fold(step, 0);
        stage(step + 1, r1, 1);
        __syncthreads();
        if (step + 1 >= nsteps) break;
        fetch(step + 3, r1);
        if (wave_live && (step + 1) * KSTEP <= wave_last_pos) fold(step + 1, 1);
        stage(step + 2, r0, 0);
        __syncthreads();
    }
    if (!wave_live) return;

#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        l[ht] = xor_sum(xor_sum(l[ht], 16), 32);
        const int r = row0 + ht * 16 + col;
        if (r >= nrows) continue;
        const int tok = r / G;
        const int j = r - tok * G;
        const float inv = 1.f / l[ht];
        char* orow = (char*)p.out + ((size_t)(qb0 + tok) * p.Hq + kvh * G + j) * D * 2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 a = acc[ht][dt];
            *(uint2*)(orow + (dt * 16 + 4 * gq) * 2) = pack4<K>(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
        }
    }
}

template <int K, int D, int BS>
__global__ __launch_bounds__(NW * 64, 2) void chunked_fa(ChunkedParams p) {
    __shared__ __attribute__((aligned(16))) char lds[2 * ChunkLds<D>::STAGE];
    if (contract_broken(p.guard)) return;
    chunked_tile<K, D, BS>(p, blockIdx.x, lds, false);
}

}  // namespace

}  // namespace pkv
