// decode_inner.h -- the two per-block inner loops of paged decode (gfx950), shared
// by the fixed-partition and the load-balanced kernels.
//
// One wave owns one (sequence, kv head, query-head tile) stream at a time and
// folds 16-token blocks into an online softmax: running max m and running sum l
// per query head (scores in log2 units), accumulator rescaled by 2^(m_old - m_new).
// Tokens at or past the context end are masked; their V slots may hold anything
// (NaN), so those V values are zeroed before the P.V product.
#pragma once

#include "device.h"
#include "internal.h"

namespace pkv {

// Cache policy of the V loads: a tile of a 32-token block reads half of every
// head_dim row of the block's V tile, and the block's other tile -- folded next by
// the same wave -- reads the other half of the same cache lines, so those loads keep
// the default policy; everything else streams.
template <int BS> constexpr int kVPolicy = BS == 32 ? 0 : kNonTemporal;

// Where the 16 tokens of one tile of a (sequence, kv head) are.  Units are
// (physical block * Hkv + kv head), i.e. (block, kv head) tiles of the pools, each
// BS * D elements (K: [BS][D] token-major; V: [D][BS] head_dim-major).
//  * block size 16: the tile is unit u0;
//  * block size 32: the tile is 16-token half `part` of unit u0;
//  * block size 8: its tokens 0-7 are unit u0, tokens 8-15 unit u1.
// An empty source (live = false) loads zeros and reads nothing (block sizes 16, 32),
// or reads unit 0 of the pools (block size 8); an empty tile is never folded.
struct TileSrc {
    size_t u0, u1;
    int part;
    bool live;
};

// ---------------------------------------------------------------------------------------
// Matrix-core inner loop (16-bit types).  Scores S^T[16 tokens][16 heads] = K Q^T on
// 16x16x32 MFMA (lane l: token row l%16 of K, head column l%16 of Q, d-chunk
// (l/16 + 4*step) -- the same head_dim permutation on both operands).  The result
// leaves lane l with 4 tokens (4*(l/16)+j) of head l%16, exactly the B operand of
// O^T[d][head] += V^T[d][16 tokens] P^T[16 tokens][head] on 16x16x16 MFMA, whose
// A operand is 8 contiguous bytes of the head_dim-major V tile.  P is split into a
// 16-bit high part and a 16-bit remainder, so the product keeps ~16 bits of P.
// ---------------------------------------------------------------------------------------
template <int K, int D, int NH, int BS>
struct MfmaLoop {
    static constexpr int kBS = BS;
    static constexpr int kElemBytes = Elem<K>::bytes;
    static constexpr int KS = D / 32;
    static constexpr int DT = D / 16;
    static constexpr int HT = 16 * NH;
    // Waves per SIMD the register budget is sized for, and tiles in the prefetch
    // ring.  At head_dim 128 one wave per SIMD with a five-tile ring keeps as many
    // bytes in flight as two waves with three tiles each, and its waves progress
    // evenly: two waves on one SIMD share issue slots by age, so with equal work
    // the younger one finishes far behind the older.  Two head tiles (many query
    // heads per kv head) spend longer on each block, so they keep one more tile in
    // flight (six tiles x 12 loads stays under the 63 outstanding loads a wave
    // can count).
    static constexpr int kWaves = (NH == 1 && D == 64) ? 2 : 1;
    static constexpr bool kCoop = false;
    static constexpr int kRing = D == 128 ? (NH == 2 ? 6 : 5) : 3;

    struct Tile {
        uint4 k[KS];
        uint2 v[DT];
    };
    static constexpr int kTileLoads = KS + DT;  // load instructions per tile
    struct State {
        float m[NH], l[NH];
        f32x4 acc[NH][DT];
        uint4 q[NH][KS];
    };

    int col, gq;
    uint32_t koff, voff;  // byte offsets of this lane's first K / V piece inside its unit
    bool ksel, vsel;      // block size 8: this lane's K row / V tokens lie in unit u1

    __device__ __forceinline__ void init_lane(int lane) {
        col = lane & 15;
        gq = lane >> 4;
        if constexpr (BS == 8) {
            ksel = col >= 8;
            vsel = gq >= 2;
            koff = (uint32_t)((col & 7) * D + gq * 8) * 2;  // + ks * 64 bytes
            voff = (uint32_t)(col * 8 + 4 * (gq & 1)) * 2;   // + dt * 16 rows
        } else {
            ksel = vsel = false;
            koff = (uint32_t)(col * D + gq * 8) * 2;
            voff = (uint32_t)(col * BS + 4 * gq) * 2;
        }
    }

    // query rows head0 .. head0 + nh - 1 of token row `qrow` (q is [rows][Hq][D])
    __device__ __forceinline__ void start(State& st, const void* q, size_t qrow, int Hq, int head0, int nh) {
        const uint16_t* qp = (const uint16_t*)q;
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            const int h = ht * 16 + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                st.q[ht][ks] = h < nh ? *(const uint4*)(qp + (qrow * Hq + head0 + h) * D + (gq + 4 * ks) * 8)
                                      : make_uint4(0, 0, 0, 0);
            st.m[ht] = kNegInf;
            st.l[ht] = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) st.acc[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // K/V of the tile `src` names
    __device__ __forceinline__ void load(Tile& t, const void* kc, const void* vc, const TileSrc& src) const {
        constexpr size_t kUnit = (size_t)BS * D * 2;
        if constexpr (BS == 8) {
            const char* kp = (const char*)kc + (ksel ? src.u1 : src.u0) * kUnit + koff;
            const char* vp = (const char*)vc + (vsel ? src.u1 : src.u0) * kUnit + voff;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) t.k[ks] = stream_load16(kp + ks * 64);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) t.v[dt] = stream_load8(vp + dt * 16 * BS * 2);
        } else {
            const size_t kb = src.live ? src.u0 * kUnit + (size_t)src.part * kTileTokens * D * 2 : 0;
            const size_t vb = src.live ? src.u0 * kUnit + (size_t)src.part * kTileTokens * 2 : 0;
            const rsrc_t kr = tile_rsrc((const char*)kc + kb, src.live ? kTileTokens * D * 2 : 0);
            const rsrc_t vr =
                tile_rsrc((const char*)vc + vb, src.live ? (uint32_t)(kUnit - src.part * kTileTokens * 2) : 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) t.k[ks] = stream_load16(kr, koff + ks * 64);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) t.v[dt] = policy_load8<kVPolicy<BS>>(vr, voff + dt * 16 * BS * 2);
        }
    }

    // fold one block whose first `valid` tokens are inside the context
    __device__ __forceinline__ void block(State& st, Tile& t, int valid, float scale_log2) const {
        uint2 phi[NH], plo[NH];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc = mma_16x16x32<K>(t.k[ks], st.q[ht][ks], sc);
            mfma_result_fence();
            float sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[j] = sc[j];
            if (valid < kTileTokens) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * gq + j >= valid) sv[j] = kNegInf;
            }
            float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            bm = xor_max(bm, 16);
            bm = xor_max(bm, 32);
            bm *= scale_log2;  // the scale is positive: the max of the scaled scores
            if (__ballot(bm > st.m[ht] + kRescaleSlack)) {
                const float mn = fmaxf(st.m[ht], bm);
                const float alpha = fast_exp2(st.m[ht] - mn);
                st.l[ht] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) st.acc[ht][dt] *= alpha;
                st.m[ht] = mn;
            }
            const float off = -st.m[ht];
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(__builtin_fmaf(sv[j], scale_log2, off));
            st.l[ht] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            phi[ht] = pack4<K>(pr[0], pr[1], pr[2], pr[3]);
            plo[ht] = pack4<K>(pr[0] - lo16<K>(phi[ht].x), pr[1] - hi16<K>(phi[ht].x), pr[2] - lo16<K>(phi[ht].y),
                               pr[3] - hi16<K>(phi[ht].y));
        }
        if (valid < kTileTokens) {
            const int tk = 4 * gq;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                uint32_t x = t.v[dt].x, y = t.v[dt].y;
                if (tk + 0 >= valid) x &= 0xffff0000u;
                if (tk + 1 >= valid) x &= 0x0000ffffu;
                if (tk + 2 >= valid) y &= 0xffff0000u;
                if (tk + 3 >= valid) y &= 0x0000ffffu;
                t.v[dt] = make_uint2(x, y);
            }
        }
        // high parts first, then the remainders: consecutive MFMAs never share an accumulator
#pragma unroll
        for (int ht = 0; ht < NH; ++ht)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) st.acc[ht][dt] = mma_16x16x16<K>(t.v[dt], phi[ht], st.acc[ht][dt]);
#pragma unroll
        for (int ht = 0; ht < NH; ++ht)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) st.acc[ht][dt] = mma_16x16x16<K>(t.v[dt], plo[ht], st.acc[ht][dt]);
    }

    // sum l over the four lane groups (each holds a quarter of the tokens)
    __device__ __forceinline__ void finish(State& st) const {
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) st.l[ht] = xor_sum(xor_sum(st.l[ht], 16), 32);
    }

    // normalised output of heads head0 .. head0 + nh - 1 of token row `orow`
    __device__ __forceinline__ void store_out(const State& st, void* out, size_t orow, int Hq, int head0,
                                              int nh) const {
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            const int h = ht * 16 + col;
            if (h >= nh) continue;
            const float inv = st.l[ht] > 0.f ? 1.f / st.l[ht] : 0.f;
            uint16_t* o = (uint16_t*)out + (orow * Hq + head0 + h) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 a = st.acc[ht][dt];
                *(uint2*)(o + dt * 16 + 4 * gq) = pack4<K>(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
            }
        }
    }

    // partial record: acc[cap][D], m[cap], l[cap] (cap = head capacity of a record)
    __device__ __forceinline__ void store_partial(const State& st, float* rec, int cap, int nh) const {
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            const int h = ht * 16 + col;
            if (h >= nh) continue;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) *(f32x4*)(rec + h * D + dt * 16 + 4 * gq) = st.acc[ht][dt];
            if (gq == 0) {
                rec[cap * D + h] = st.m[ht];
                rec[cap * D + cap + h] = st.l[ht];
            }
        }
    }
};

// ---------------------------------------------------------------------------------------
// Matrix-core inner loop for 17..32 query heads per kv head (MQA-like streams).
// Scores as in MfmaLoop (two 16-head 16x16x32 products per k-step), but
//   O^T[d][head] += V^T[d][tokens] . P^T[tokens][head]
// runs on 32x32x16 products with all 32 heads as columns: the A operand is 8
// consecutive tokens of one head_dim row -- 16 contiguous bytes of the V tile -- so a
// tile takes half the V load instructions and a quarter of the P.V products.  The
// P operand (lane l: head l%32, tokens 8*(l/32)..+7) comes from the score layout
// (lane l: tokens 4*(l/16)..+3 of head l%16 of each 16-head tile) with one 16-lane
// row swap per packed word: rows 0/2 keep their head-tile-0 values and take row 1/3's,
// rows 1/3 take row 0/2's head-tile-1 values and keep their own.
// ---------------------------------------------------------------------------------------
template <int K, int D, int BS>
struct MfmaWideLoop {
    static constexpr int kBS = BS;
    static constexpr int kElemBytes = Elem<K>::bytes;
    static constexpr int KS = D / 32;
    static constexpr int DQ = D / 32;  // 32-row head_dim tiles of the output
    static constexpr int HT = 32;
    static constexpr int kWaves = 1;
    static constexpr int kKind = K;
    static constexpr int kD = D;
    // the balanced split runs this loop on cooperative workgroups (decode_split_coop)
    static constexpr bool kCoop = true;
    // half the V loads of MfmaLoop: at head_dim 128 six tiles fit the register file
    static constexpr int kRing = D == 128 ? 6 : 8;
    static constexpr int kTileLoads = KS + DQ;

    struct Tile {
        uint4 k[KS];
        uint4 v[DQ];
    };
    struct State {
        float m[2], l[2];
        f32x16 acc[DQ];
        uint4 q[2][KS];
    };

    int lane, col, gq;
    uint32_t koff, voff;
    bool ksel, vsel;  // block size 8: this lane's K row / V tokens lie in unit u1

    __device__ __forceinline__ void init_lane(int ln) {
        lane = ln;
        col = ln & 15;
        gq = ln >> 4;
        if constexpr (BS == 8) {
            ksel = col >= 8;
            vsel = (ln >> 5) != 0;
            koff = (uint32_t)((col & 7) * D + gq * 8) * 2;  // + ks * 64 bytes
            voff = (uint32_t)(ln & 31) * 8 * 2;              // + dq * 32 rows
        } else {
            ksel = vsel = false;
            koff = (uint32_t)(col * D + gq * 8) * 2;
            voff = (uint32_t)((ln & 31) * BS + 8 * (ln >> 5)) * 2;
        }
    }

    __device__ __forceinline__ void start(State& st, const void* q, size_t qrow, int Hq, int head0, int nh) {
        const uint16_t* qp = (const uint16_t*)q;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int h = ht * 16 + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                st.q[ht][ks] = h < nh ? *(const uint4*)(qp + (qrow * Hq + head0 + h) * D + (gq + 4 * ks) * 8)
                                      : make_uint4(0, 0, 0, 0);
            st.m[ht] = kNegInf;
            st.l[ht] = 0.f;
        }
#pragma unroll
        for (int dq = 0; dq < DQ; ++dq)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.acc[dq][r] = 0.f;
    }

    __device__ __forceinline__ void load(Tile& t, const void* kc, const void* vc, const TileSrc& src) const {
        constexpr size_t kUnit = (size_t)BS * D * 2;
        if constexpr (BS == 8) {
            const char* kp = (const char*)kc + (ksel ? src.u1 : src.u0) * kUnit + koff;
            const char* vp = (const char*)vc + (vsel ? src.u1 : src.u0) * kUnit + voff;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) t.k[ks] = stream_load16(kp + ks * 64);
#pragma unroll
            for (int dq = 0; dq < DQ; ++dq) t.v[dq] = stream_load16(vp + dq * 32 * BS * 2);
        } else {
            const size_t kb = src.live ? src.u0 * kUnit + (size_t)src.part * kTileTokens * D * 2 : 0;
            const size_t vb = src.live ? src.u0 * kUnit + (size_t)src.part * kTileTokens * 2 : 0;
            const rsrc_t kr = tile_rsrc((const char*)kc + kb, src.live ? kTileTokens * D * 2 : 0);
            const rsrc_t vr =
                tile_rsrc((const char*)vc + vb, src.live ? (uint32_t)(kUnit - src.part * kTileTokens * 2) : 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) t.k[ks] = stream_load16(kr, koff + ks * 64);
#pragma unroll
            for (int dq = 0; dq < DQ; ++dq) t.v[dq] = policy_load16<kVPolicy<BS>>(vr, voff + dq * 32 * BS * 2);
        }
    }

    // this lane's output column is head lane % 32: head tile (lane / 16) % 2 (two
    // scalars, not an array, so that the choice stays a select)
    __device__ __forceinline__ float pick(float x0, float x1) const { return (lane & 16) ? x1 : x0; }

    __device__ __forceinline__ void block(State& st, Tile& t, int valid, float scale_log2) const {
        float sv[2][4];
        f32x4 sc[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            sc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc[ht] = mma_16x16x32<K>(t.k[ks], st.q[ht][ks], sc[ht]);
        }
        mfma_result_fence();
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[ht][j] = sc[ht][j];
        if (valid < kTileTokens) {
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * gq + j >= valid) sv[ht][j] = kNegInf;
        }
        float bm[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            bm[ht] = fmaxf(fmaxf(sv[ht][0], sv[ht][1]), fmaxf(sv[ht][2], sv[ht][3]));
            bm[ht] = xor_max(bm[ht], 16);
            bm[ht] = xor_max(bm[ht], 32);
            bm[ht] *= scale_log2;
        }
        if (__ballot(bm[0] > st.m[0] + kRescaleSlack || bm[1] > st.m[1] + kRescaleSlack)) {
            float alpha[2];
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                const float mn = fmaxf(st.m[ht], bm[ht]);
                alpha[ht] = fast_exp2(st.m[ht] - mn);
                st.l[ht] *= alpha[ht];
                st.m[ht] = mn;
            }
            const float a = pick(alpha[0], alpha[1]);
#pragma unroll
            for (int dq = 0; dq < DQ; ++dq) st.acc[dq] *= a;
        }
        uint32_t hi[2][2], lo[2][2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const float off = -st.m[ht];
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(__builtin_fmaf(sv[ht][j], scale_log2, off));
            st.l[ht] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            const uint2 h = pack4<K>(pr[0], pr[1], pr[2], pr[3]);
            const uint2 r = pack4<K>(pr[0] - lo16<K>(h.x), pr[1] - hi16<K>(h.x), pr[2] - lo16<K>(h.y),
                                     pr[3] - hi16<K>(h.y));
            hi[ht][0] = h.x;
            hi[ht][1] = h.y;
            lo[ht][0] = r.x;
            lo[ht][1] = r.y;
        }
        // to the P operand layout: tokens 8*(lane/32)..+7 of head lane%32
        uint4 phi, plo;
        row_swap16(hi[0][0], hi[1][0], phi.x, phi.z);
        row_swap16(hi[0][1], hi[1][1], phi.y, phi.w);
        row_swap16(lo[0][0], lo[1][0], plo.x, plo.z);
        row_swap16(lo[0][1], lo[1][1], plo.y, plo.w);
        if (valid < kTileTokens) {
            const int tk = 8 * (lane >> 5);
#pragma unroll
            for (int dq = 0; dq < DQ; ++dq) {
                uint32_t w[4] = {t.v[dq].x, t.v[dq].y, t.v[dq].z, t.v[dq].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (tk + e >= valid) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                t.v[dq] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
#pragma unroll
        for (int dq = 0; dq < DQ; ++dq) st.acc[dq] = mma_32x32x16<K>(t.v[dq], phi, st.acc[dq]);
#pragma unroll
        for (int dq = 0; dq < DQ; ++dq) st.acc[dq] = mma_32x32x16<K>(t.v[dq], plo, st.acc[dq]);
    }

    __device__ __forceinline__ void finish(State& st) const {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) st.l[ht] = xor_sum(xor_sum(st.l[ht], 16), 32);
    }

    // element r of acc[dq] is head_dim row 32*dq + 8*(r/4) + 4*(lane/32) + r%4
    __device__ __forceinline__ void store_out(const State& st, void* out, size_t orow, int Hq, int head0,
                                              int nh) const {
        const int h = lane & 31;
        if (h >= nh) return;
        const float lsum = pick(st.l[0], st.l[1]);
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        uint16_t* o = (uint16_t*)out + (orow * Hq + head0 + h) * D;
#pragma unroll
        for (int dq = 0; dq < DQ; ++dq)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x16 a = st.acc[dq];
                *(uint2*)(o + 32 * dq + 8 * j + 4 * (lane >> 5)) =
                    pack4<K>(a[4 * j] * inv, a[4 * j + 1] * inv, a[4 * j + 2] * inv, a[4 * j + 3] * inv);
            }
    }

    __device__ __forceinline__ void store_partial(const State& st, float* rec, int cap, int nh) const {
        const int h = lane & 31;
        if (h >= nh) return;
#pragma unroll
        for (int dq = 0; dq < DQ; ++dq)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x16 a = st.acc[dq];
                *(f32x4*)(rec + h * D + 32 * dq + 8 * j + 4 * (lane >> 5)) =
                    f32x4{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
            }
        if (lane < 32) {
            rec[cap * D + h] = pick(st.m[0], st.m[1]);
            rec[cap * D + cap + h] = pick(st.l[0], st.l[1]);
        }
    }
};

// ---------------------------------------------------------------------------------------
// Vector-ALU inner loop (fp32, or few query heads per kv head).  Four lanes per
// token share its dot products (shuffle reductions).  For P.V every load
// instruction reads 1 KiB of the head_dim-major V tile contiguously: lane l's
// piece c is 16-byte chunk c*64+l, i.e. VE tokens of head_dim row (c*64+l)/CPR.
// Each lane keeps partial sums for its rows over its tokens; the CPR lanes that
// share a row are added together once, at the end.
// ---------------------------------------------------------------------------------------
template <int K> __device__ __forceinline__ void widen16(uint4 c, float* f) {
    if constexpr (K == KF32) {
        f[0] = __uint_as_float(c.x);
        f[1] = __uint_as_float(c.y);
        f[2] = __uint_as_float(c.z);
        f[3] = __uint_as_float(c.w);
    } else {
        const uint32_t u[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = lo16<K>(u[i]);
            f[2 * i + 1] = hi16<K>(u[i]);
        }
    }
}

template <int K, int D, int GT, int BS>
struct ValuLoop {
    static constexpr int kBS = BS;
    static constexpr int kElemBytes = Elem<K>::bytes;
    static constexpr int EB = Elem<K>::bytes;
    static constexpr int VE = 16 / EB;                 // elements per 16-byte chunk
    static constexpr int KC = D / VE / 4;              // K chunks per lane
    static constexpr int CPR = kTileTokens / VE;       // V chunks per head_dim row of a tile (2 or 4)
    static constexpr int VC = D * CPR / 64;            // V chunks per lane
    static constexpr int HT = GT;
    static constexpr int kWaves = ((D == 128 && (EB == 4 || GT >= 2)) || (EB == 4 && GT == 4)) ? 1 : 2;
    static constexpr bool kCoop = false;
    static constexpr int kRing = 3;

    struct Tile {
        uint4 k[KC];
        uint4 v[VC];
    };
    static constexpr int kTileLoads = KC + VC;  // load instructions per tile
    struct State {
        float m[GT], l[GT], acc[GT][VC];
        float q[GT][KC * VE];
    };

    int lane, tq, sub, tg;
    uint32_t kt, vt;  // byte offsets of this lane's first K / V chunk inside its unit
    bool ksel, vsel;  // block size 8: this lane's K row / V tokens lie in unit u1

    __device__ __forceinline__ void init_lane(int ln) {
        lane = ln;
        tq = ln >> 2;
        sub = ln & 3;
        tg = ln % CPR;  // which VE tokens of a V row this lane holds
        if constexpr (BS == 8) {
            ksel = tq >= 8;
            vsel = tg >= CPR / 2;
            kt = (uint32_t)((tq & 7) * D * EB);
            vt = (uint32_t)((ln / CPR) * 8 * EB + (tg % (CPR / 2)) * 16);
        } else {
            ksel = vsel = false;
            kt = (uint32_t)(tq * D * EB);
            vt = (uint32_t)((ln / CPR) * BS * EB + tg * 16);
        }
    }

    __device__ __forceinline__ void start(State& st, const void* q, size_t qrow, int Hq, int head0, int nh) {
        const char* qp = (const char*)q;
#pragma unroll
        for (int j = 0; j < GT; ++j) {
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                uint4 c = make_uint4(0, 0, 0, 0);
                if (j < nh) c = *(const uint4*)(qp + ((qrow * Hq + head0 + j) * D + (sub + 4 * k) * VE) * EB);
                widen16<K>(c, &st.q[j][k * VE]);
            }
            st.m[j] = kNegInf;
            st.l[j] = 0.f;
#pragma unroll
            for (int c = 0; c < VC; ++c) st.acc[j][c] = 0.f;
        }
    }

    // K/V of the tile `src` names; V chunk c of this lane is head_dim row
    // lane / CPR + c * 64 / CPR
    __device__ __forceinline__ void load(Tile& t, const void* kc, const void* vc, const TileSrc& src) const {
        constexpr size_t kUnit = (size_t)BS * D * EB;
        constexpr uint32_t kRowStep = 64 / CPR * BS * EB;  // bytes between V chunks c and c + 1
        if constexpr (BS == 8) {
            const char* kp = (const char*)kc + (ksel ? src.u1 : src.u0) * kUnit + kt;
            const char* vp = (const char*)vc + (vsel ? src.u1 : src.u0) * kUnit + vt;
#pragma unroll
            for (int k = 0; k < KC; ++k) t.k[k] = stream_load16(kp + (sub + 4 * k) * 16);
#pragma unroll
            for (int c = 0; c < VC; ++c) t.v[c] = stream_load16(vp + c * kRowStep);
        } else {
            const size_t kb = src.live ? src.u0 * kUnit + (size_t)src.part * kTileTokens * D * EB : 0;
            const size_t vb = src.live ? src.u0 * kUnit + (size_t)src.part * kTileTokens * EB : 0;
            const rsrc_t kr = tile_rsrc((const char*)kc + kb, src.live ? kTileTokens * D * EB : 0);
            const rsrc_t vr =
                tile_rsrc((const char*)vc + vb, src.live ? (uint32_t)(kUnit - src.part * kTileTokens * EB) : 0);
#pragma unroll
            for (int k = 0; k < KC; ++k) t.k[k] = stream_load16(kr, kt + (sub + 4 * k) * 16);
#pragma unroll
            for (int c = 0; c < VC; ++c) t.v[c] = policy_load16<kVPolicy<BS>>(vr, vt + c * kRowStep);
        }
    }

    __device__ __forceinline__ void block(State& st, Tile& t, int valid, float scale_log2) const {
        float kf[KC * VE];
#pragma unroll
        for (int k = 0; k < KC; ++k) widen16<K>(t.k[k], &kf[k * VE]);
        float pj[GT];
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < KC * VE; ++i) dot = fmaf(st.q[j][i], kf[i], dot);
            dot = xor_sum(dot, 1);
            dot = xor_sum(dot, 2);
            const float sv = tq < valid ? dot * scale_log2 : kNegInf;
            float bm = xor_max(sv, 4);
            bm = xor_max(bm, 8);
            bm = xor_max(bm, 16);
            bm = xor_max(bm, 32);
            if (__ballot(bm > st.m[j] + kRescaleSlack)) {  // bm is the same in every lane
                const float mn = fmaxf(st.m[j], bm);
                const float alpha = fast_exp2(st.m[j] - mn);
                st.l[j] *= alpha;
#pragma unroll
                for (int c = 0; c < VC; ++c) st.acc[j][c] *= alpha;
                st.m[j] = mn;
            }
            pj[j] = fast_exp2(sv - st.m[j]);
            st.l[j] += sub == 0 ? pj[j] : 0.f;
        }
        float vf[VC][VE];
#pragma unroll
        for (int c = 0; c < VC; ++c) widen16<K>(t.v[c], vf[c]);
        if (valid < kTileTokens) {
#pragma unroll
            for (int e = 0; e < VE; ++e)
                if (tg * VE + e >= valid)
#pragma unroll
                    for (int c = 0; c < VC; ++c) vf[c][e] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            float ps[kTileTokens];  // p of every token of the block (wave-uniform)
#pragma unroll
            for (int tk = 0; tk < kTileTokens; ++tk) ps[tk] = read_lane(pj[j], 4 * tk);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                float pe = ps[e];
#pragma unroll
                for (int g = 1; g < CPR; ++g) pe = tg == g ? ps[g * VE + e] : pe;
#pragma unroll
                for (int c = 0; c < VC; ++c) st.acc[j][c] = fmaf(pe, vf[c][e], st.acc[j][c]);
            }
        }
    }

    __device__ __forceinline__ void finish(State& st) const {
#pragma unroll
        for (int j = 0; j < GT; ++j) {
#pragma unroll
            for (int mask = 1; mask < 64; mask <<= 1) st.l[j] = xor_sum(st.l[j], mask);
#pragma unroll
            for (int c = 0; c < VC; ++c)
#pragma unroll
                for (int mask = 1; mask < CPR; mask <<= 1) st.acc[j][c] = xor_sum(st.acc[j][c], mask);
        }
    }

    __device__ __forceinline__ int row(int c) const { return (c * 64 + lane) / CPR; }

    __device__ __forceinline__ void store_out(const State& st, void* out, size_t orow, int Hq, int head0,
                                              int nh) const {
        if (tg != 0) return;
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            if (j >= nh) continue;
            const float inv = st.l[j] > 0.f ? 1.f / st.l[j] : 0.f;
#pragma unroll
            for (int c = 0; c < VC; ++c) store_elem<K>(out, (orow * Hq + head0 + j) * D + row(c), st.acc[j][c] * inv);
        }
    }

    __device__ __forceinline__ void store_partial(const State& st, float* rec, int cap, int nh) const {
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            if (j >= nh) continue;
            if (tg == 0) {
#pragma unroll
                for (int c = 0; c < VC; ++c) rec[j * D + row(c)] = st.acc[j][c];
            }
            if (lane == 0) {
                rec[cap * D + j] = st.m[j];
                rec[cap * D + cap + j] = st.l[j];
            }
        }
    }
};

}  // namespace pkv
