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
// The keys go by in steps of 32.  A step's K and V travel from the pool straight
// into LDS (gfx950 buffer loads to LDS, 16 bytes a lane: no registers, no vector
// instructions on the way), two steps ahead, in a ring of three LDS stages, and
// every wave folds the step into its rows with an online softmax:
//   S^T = K Q^T        16x16x32 matrix cores, 16 keys x 16 rows per product
//   O^T += V^T P^T     16x16x32 matrix cores over all 32 keys of the step, P rounded
//                      to the element type (bf16 or f16) as the product's operand, and
//                      the softmax sum taken over the rounded weights: every output row
//                      is then a convex combination of V rows whose weights are within
//                      one rounding of the exact ones (a context of one token gives its
//                      V row exactly)
// The two score products of a step take the keys in the order that makes each
// lane's eight probabilities the eight consecutive keys of one 16-byte V chunk:
// product h (0, 1) has key 8 (i / 4) + 4 h + i % 4 as its row i, so lane group g
// ends up with keys 8 g .. 8 g + 3 from product 0 and 8 g + 4 .. 8 g + 7 from
// product 1 (a sum over keys does not care about their order).
// LDS layouts of a stage:
//   K: [32 keys][D / 8 chunks of 16 bytes], chunk c of key row r stored at position
//      c ^ f(r): the 16 rows one score operand read touches then fall on distinct
//      banks (f: two bits of the row within its group of four, two of its group of
//      eight)
//   V: [2 halves of 16 keys][2 chunks of 8 keys][D] x 16 bytes: one 16-byte read is
//      one matrix-core operand (8 keys of one head_dim row), and the 16 lanes of one
//      read take 256 consecutive bytes.
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
constexpr int kStages = 3;             // LDS ring: the step being folded and two in flight

template <int D>
struct ChunkLds {
    static constexpr int KCH = D / 8;                 // 16-byte chunks per key row
    static constexpr int KBYTES = KSTEP * D * 2;      // K of one step
    static constexpr int VBYTES = KSTEP * D * 2;      // V of one step
    static constexpr int STAGE = KBYTES + VBYTES;
    // 1 KiB loads-to-LDS (64 lanes x 16 bytes) per step, and per wave
    static constexpr int KLOADS = KBYTES / 1024, VLOADS = VBYTES / 1024;
    static constexpr int KLOADS_W = KLOADS / NW, VLOADS_W = VLOADS / NW;
    static_assert(KLOADS % NW == 0 && VLOADS % NW == 0, "every wave moves the same share");
    // key row of lane `lane` in K load j of wave w, and the first key of the 8-key
    // chunk of V load j of wave w
    static constexpr __host__ __device__ int k_row(int w, int j, int lane) {
        return (w * KLOADS_W + j) * (64 / KCH) + lane / KCH;
    }
    static constexpr __host__ __device__ int v_key(int w, int j, int lane) {
        return 8 * (((w * VLOADS_W + j) * 64 + lane) / D);
    }
    static constexpr __host__ __device__ int block_of_wave(int w, int bs) { return k_row(w, 0, 0) / bs; }
    // every load of a wave, K and V, lies in the wave's one block
    static constexpr bool one_block_per_wave(int bs) {
        for (int w = 0; w < NW; ++w)
            for (int lane = 0; lane < 64; ++lane) {
                for (int j = 0; j < KLOADS_W; ++j)
                    if (k_row(w, j, lane) / bs != block_of_wave(w, bs)) return false;
                for (int j = 0; j < VLOADS_W; ++j)
                    if (v_key(w, j, lane) / bs != block_of_wave(w, bs) || (v_key(w, j, lane) + 7) / bs !=
                                                                             block_of_wave(w, bs))
                        return false;
            }
        return true;
    }
    static_assert(one_block_per_wave(8) && one_block_per_wave(16) && one_block_per_wave(32),
                  "each wave's loads of a step come from one pool block");
    // position of chunk c of key row r
    static __device__ __forceinline__ int kpos(int r, int c) {
        if constexpr (D == 128)
            return c ^ ((r & 3) | (((r >> 3) & 3) << 2));
        else
            return c ^ (((r >> 1) & 1) | (((r >> 3) & 3) << 1));
    }
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// gfx950 16-byte buffer load to LDS: lane t's 16 bytes at `voff` land at lds + 16 t
// (kAux: cache policy bits)
template <int kAux> __device__ __forceinline__ void load_to_lds(rsrc_t r, char* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, (int)voff, 0, 0, kAux);
}

// BS: tokens per KV block (8, 16 or 32); a step's 32 keys span KSTEP / BS blocks
// Workgroup `idx` of the chunked grid (tile, kv head, segment), with the three LDS
// stages st0, st1, st2 (ChunkLds<D>::STAGE bytes each; three distinct LDS
// variables, so that the compiler can tell a stage being filled from the one being
// read and does not make the reads wait for loads still in flight to the others).
// With skip_single, one-row segments are left alone (the mixed launch runs them as
// decode sequences).
template <int K, int D, int BS>
__device__ __forceinline__ void chunked_tile(const ChunkedParams& p, int idx, char* st0, char* st1, char* st2,
                                             bool skip_single) {
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    using Lds = ChunkLds<D>;
    constexpr uint32_t kTile = BS * D * 2;  // bytes of one (block, kv head) tile
    constexpr int NBS = KSTEP / BS;         // blocks per step

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

    // ---- loads of one step straight into an LDS stage ------------------------------
    // Loads of blocks past the context are empty (zero bytes written, no memory
    // access), so every step issues the same loads and the wait before a fold counts
    // exactly: KLOADS_W + VLOADS_W per wave and step.
    const int32_t* table = p.block_tables + (size_t)seg * p.MB;
    // this lane's part of each of the wave's loads: K load j covers key rows
    // rows_per_load j'..+rows_per_load-1 (j' = the workgroup-wide load index), V load j
    // covers 64 head_dim rows of one (half, chunk).  Every load of wave w lies in one
    // pool block of the step, block_of_wave(w) (checked at compile time below), so a
    // wave reads one table entry and builds one K and one V resource per step.
    const int myblk = uniform(ChunkLds<D>::block_of_wave(w, BS));
    uint32_t koff[Lds::KLOADS_W], voff[Lds::VLOADS_W];
#pragma unroll
    for (int j = 0; j < Lds::KLOADS_W; ++j) {
        const int r = Lds::k_row(w, j, lane);           // key row in the step
        const int c = Lds::kpos(r, lane % Lds::KCH);  // the chunk this slot holds
        koff[j] = (uint32_t)((r % BS) * D * 2 + c * 16);
    }
#pragma unroll
    for (int j = 0; j < Lds::VLOADS_W; ++j) {
        const int slot = (w * Lds::VLOADS_W + j) * 64 + lane;  // [half][chunk][d]
        const int d = slot % D;
        const int key = Lds::v_key(w, j, lane);  // first key of the chunk within the step
        voff[j] = (uint32_t)(d * BS * 2 + (key % BS) * 2);
    }
    auto issue = [&](int step, char* stage) {
        char* kl = stage;
        char* vl = kl + Lds::KBYTES;
        const int b = step * NBS + myblk;
        const bool live = b < nblk;
        const int ph = live ? scalar_load(table, (size_t)uniform(b)) : 0;
        const size_t t = ((size_t)ph * p.Hkv + kvh) * kTile;
        const rsrc_t kr = tile_rsrc((const char*)p.kc + t, live ? kTile : 0);
        const rsrc_t vr = tile_rsrc((const char*)p.vc + t, live ? kTile : 0);
#pragma unroll
        for (int j = 0; j < Lds::KLOADS_W; ++j)
            load_to_lds<kNonTemporal>(kr, kl + (w * Lds::KLOADS_W + j) * 1024, koff[j]);
        // V chunks are 16 of the 32 bytes of a head_dim row (block size 16 or 32): the
        // other half is read by the neighbouring load, so V keeps the default policy
#pragma unroll
        for (int j = 0; j < Lds::VLOADS_W; ++j)
            load_to_lds<BS == 8 ? kNonTemporal : 0>(vr, vl + (w * Lds::VLOADS_W + j) * 1024, voff[j]);
    };

    // ---- this lane's rows: Q as the B operand of the score product; dead rows see
    // every key with a zero query (finite, never stored) ------------------------------
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
    // the softmax sums come out of the matrix cores: a head_dim tile of ones beside V,
    // so that every element of lsum[ht] is the row's sum of its rounded weights
    float m[NH];
    f32x4 acc[NH][DT], lsum[NH];
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        m[ht] = kNegInf;
        lsum[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const uint32_t one2 = pack4<K>(1.f, 1.f, 1.f, 1.f).x;  // two 16-bit ones
    const uint4 ones = make_uint4(one2, one2, one2, one2);

    // ---- one step: 32 keys into this wave's 32 rows ----------------------------------
    auto fold = [&](int step, const char* stage) {
        const char* kl = stage;
        const char* vl = kl + Lds::KBYTES;
        const int key0 = step * KSTEP;
        // four independent score chains (2 key sets x 2 row tiles) per k-step, so
        // consecutive matrix-core products never wait on each other; key set h takes
        // key 8 (col / 4) + 4 h + col % 4 as its row col
        uint4 kf[2][KS];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 8 * (col >> 2) + 4 * h + (col & 3);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[h][ks] = *(const uint4*)(kl + r * (D * 2) + Lds::kpos(r, gq + 4 * ks) * 16);
        }
        f32x4 sc[2][NH];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ht = 0; ht < NH; ++ht) sc[h][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        // the score products at raised wave priority: the matrix cores take this wave's
        // chain first while the other wave of the SIMD runs its softmax (1-3 % a call).
        // Not in the mixed launch, where it slows the decode waves sharing the SIMDs.
        if (!skip_single) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ht = 0; ht < NH; ++ht) sc[h][ht] = mma_16x16x32<K>(kf[h][ks], qv[ht][ks], sc[h][ht]);
        if (!skip_single) __builtin_amdgcn_s_setprio(0);
        // V fragments: head_dim row 16 dt + col, keys 8 gq .. 8 gq + 7 (half gq / 2,
        // chunk gq % 2), read while the first softmax runs
        uint4 vf[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[dt] = *(const uint4*)(vl + (gq * D + dt * 16 + col) * 16);
        // slots past the context may hold anything (NaN): zero them, last step only
        if (key0 + KSTEP > n) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                uint32_t u[4] = {vf[dt].x, vf[dt].y, vf[dt].z, vf[dt].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (key0 + 8 * gq + e >= n) u[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                vf[dt] = make_uint4(u[0], u[1], u[2], u[3]);
            }
        }
        // keys of this lane's eight scores: key0 + 8 gq + j (set 0), key0 + 8 gq + 4 + j (set 1)
        const bool masked = key0 + KSTEP - 1 > wave_first_pos;
        const float c = p.scale_log2;
        // The maxima (and the rare rescales) of both row tiles first, so that the
        // exponentials, packing and P.V products of both tiles form one branch-free block
        // the compiler can schedule as a whole (+3 % against tile after tile).
        float s[NH][8];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[ht][j] = sc[0][ht][j];
                s[ht][4 + j] = sc[1][ht][j];
            }
            if (masked) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (key0 + 8 * gq + j > pos[ht]) s[ht][j] = kNegInf;
            }
        }
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            // this lane's maximum of its eight scaled scores (the scale is positive); only
            // when one exceeds the reference by the slack is the row maximum over the
            // four lanes of the row needed
            // (IEEE maximum: no NaN can be among the scores here -- slots past the context are
            // masked above -- so it needs none of the operand quieting fmaxf costs)
            const float lm = max_nonan(max_nonan(max_nonan(s[ht][0], s[ht][1]), max_nonan(s[ht][2], s[ht][3])),
                                       max_nonan(max_nonan(s[ht][4], s[ht][5]), max_nonan(s[ht][6], s[ht][7]))) *
                             c;
            // key 0 is visible to every row, so m is finite from the first step on
            if (__ballot(lm > m[ht] + kRescaleSlack)) {
                const float mn = fmaxf(m[ht], xor_max(xor_max(lm, 16), 32));
                const float alpha = fast_exp2(m[ht] - mn);
                lsum[ht] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[ht][dt] *= alpha;
                m[ht] = mn;
            }
        }
        uint4 pw[NH];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            const float off = -m[ht];
            float pr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pr[j] = fast_exp2(__builtin_fmaf(s[ht][j], c, off));
            const uint2 h0 = pack4<K>(pr[0], pr[1], pr[2], pr[3]);
            const uint2 h1 = pack4<K>(pr[4], pr[5], pr[6], pr[7]);
            pw[ht] = make_uint4(h0.x, h0.y, h1.x, h1.y);
        }
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[ht][dt] = mma_16x16x32<K>(vf[dt], pw[ht], acc[ht][dt]);
            lsum[ht] = mma_16x16x32<K>(ones, pw[ht], lsum[ht]);
        }
    };

    // Step s lives in LDS stage s % 3; its loads were issued two steps earlier.  Before
    // folding step s: wait until this wave's loads of step s have landed (those of
    // step s + 1 may stay in flight), then a workgroup barrier, after which every
    // wave's loads of step s are in LDS and every wave has finished folding step
    // s - 1 -- so stage (s + 2) % 3 is free for the loads of step s + 2.  Plain
    // barriers: the loads to LDS are waited for explicitly, and no other LDS store
    // happens in the loop.
    constexpr int kPerStep = Lds::KLOADS_W + Lds::VLOADS_W;
    // fold step s from stage `cur` after issuing the loads of step s + 2 into `next`
    auto step_once = [&](int s, const char* cur, char* next) {
        vm_wait_le<kPerStep>();
        __builtin_amdgcn_s_barrier();
        issue(s + 2, next);
        // a wave whose rows all lie before this step's first key has nothing to fold
        if (wave_live && s * KSTEP <= wave_last_pos) fold(s, cur);
    };
    issue(0, st0);
    issue(1, st1);
    for (int step = 0; step < nsteps; step += kStages) {
        step_once(step, st0, st2);
        if (step + 1 >= nsteps) break;
        step_once(step + 1, st1, st0);
        if (step + 2 >= nsteps) break;
        step_once(step + 2, st2, st1);
    }
    vm_wait_le<0>();  // no load to LDS outlives the workgroup
    if (!wave_live) return;

#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        const int r = row0 + ht * 16 + col;
        if (r >= nrows) continue;
        const int tok = r / G;
        const int j = r - tok * G;
        mfma_result_fence();
        const float inv = 1.f / lsum[ht][0];
        char* orow = (char*)p.out + ((size_t)(qb0 + tok) * p.Hq + kvh * G + j) * D * 2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 a = acc[ht][dt];
            *(uint2*)(orow + (dt * 16 + 4 * gq) * 2) = pack4<K>(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
        }
    }
}

// Work items of the chunked grid: n = tiles x P items (P = segments x kv heads, item =
// pair x tiles + tile); the row tiles of one (segment, kv head) pair share its K/V
// prefix.  The dispatcher hands workgroup i to XCD i mod 8, so items are renumbered
// for each XCD's L2 to serve whole pairs:
//  * xcd_item: each XCD takes a contiguous share of the items (the chunked launch);
//  * chunk_item: the order runs through the pairs p = r, r + 8, r + 16, ... for
//    r = 0 .. 7 in turn, a pair's tiles together, and each XCD takes a contiguous share
//    of that order.  The mixed launch numbers its one-row segments (which return at
//    once) before the prefill chunks; this spreads the chunks over the XCDs instead of
//    stacking them onto the last ones, as long as there are at least eight prefill
//    pairs (with fewer, the mixed launch keeps launch order).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_item(int i, int n) {
    const int q = n / kXcds, rem = n % kXcds;
    const int x = i % kXcds, k = i / kXcds;
    return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + k;
}
__device__ __forceinline__ int chunk_item(int i, int tiles, int P) {
    int o = xcd_item(i, tiles * P);
    // position o -> (residue class r, pair, tile)
    for (int r = 0; r < kXcds; ++r) {
        const int pairs = (P - r + kXcds - 1) / kXcds;  // pairs p < P with p mod 8 = r
        if (o < pairs * tiles) return (r + kXcds * (o / tiles)) * tiles + o % tiles;
        o -= pairs * tiles;
    }
    return 0;  // not reached: o < tiles * P
}
__device__ __forceinline__ int chunk_tiles(const ChunkedParams& p) { return (p.max_q_len * p.G + ROWS_PER_WG - 1) / ROWS_PER_WG; }

template <int K, int D, int BS>
__global__ __launch_bounds__(NW * 64, 2) void chunked_fa(ChunkedParams p) {
    __shared__ __attribute__((aligned(16))) char st0[ChunkLds<D>::STAGE];
    __shared__ __attribute__((aligned(16))) char st1[ChunkLds<D>::STAGE];
    __shared__ __attribute__((aligned(16))) char st2[ChunkLds<D>::STAGE];
    if (contract_broken(p.guard)) return;
    chunked_tile<K, D, BS>(p, xcd_item((int)blockIdx.x, (int)gridDim.x), st0, st1, st2, false);
}

}  // namespace

}  // namespace pkv
