// chunked.hip -- causal attention of chunked-prefill segments over the paged pool,
// gfx950.
//
// A long prompt is cut into chunks that run inside the flattened batch
// ("现代 LLM 推理引擎剖析", sections 1.4 and 2.1).  Query row r of a segment with L
// rows and n cached tokens (its own chunk included) sits at position n - L + r and
// attends to tokens 0 .. n - L + r (dense causal attention, "LLM 推理优化的系统视角",
// section 3.1), through the segment's block table.
//
// Rows are (query token, query head of the kv group) pairs, head fastest, so
// that the heads sharing one kv head share every K/V tile.  A workgroup of 4 waves
// takes 128 consecutive rows; each wave owns 32 rows (two 16-row matrix-core
// columns), walks the key blocks 0 .. (its last position)/16, and keeps an online
// softmax per row.  Scores S^T = K Q^T use 16x16x32 matrix cores, P V uses
// 16x16x16 matrix cores with P split into high and low 16-bit parts.
#include "device.h"
#include "internal.h"

namespace pkv {

namespace {

constexpr int NW = 4;
constexpr int BS = kBlockSize;
constexpr int ROWS_PER_WAVE = 32;
constexpr int ROWS_PER_WG = NW * ROWS_PER_WAVE;

template <int K, int D>
__global__ __launch_bounds__(NW * 64) void chunked_mfma(ChunkedParams p) {
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    constexpr int NH = ROWS_PER_WAVE / 16;

    const int G = p.G;
    const int tiles = (p.max_q_len * G + ROWS_PER_WG - 1) / ROWS_PER_WG;
    int idx = blockIdx.x;
    const int tile = idx % tiles;
    idx /= tiles;
    const int kvh = idx % p.Hkv;
    const int seg = idx / p.Hkv;

    const int qb0 = p.cu_q_lens[seg];
    const int L = p.cu_q_lens[seg + 1] - qb0;
    const int n = p.context_lens[seg];
    const int nrows = L * G;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = tile * ROWS_PER_WG + w * ROWS_PER_WAVE;
    if (row0 >= nrows) return;  // whole wave idle (no barriers in this kernel)

    const int lane = lane_id();
    const int col = lane & 15;
    const int gq = lane >> 4;

    // rows of this lane's two columns
    int pos[NH];
    bool live[NH];
    uint4 qb[NH][KS];
    const uint16_t* qp = (const uint16_t*)p.q;
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        const int r = row0 + ht * 16 + col;
        live[ht] = r < nrows;
        const int tok = live[ht] ? r / G : 0;
        const int j = live[ht] ? r - tok * G : 0;
        pos[ht] = live[ht] ? n - L + tok : 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ht][ks] = live[ht] ? *(const uint4*)(qp + ((size_t)(qb0 + tok) * p.Hq + kvh * G + j) * D +
                                                    (gq + 4 * ks) * 8)
                                  : make_uint4(0, 0, 0, 0);
    }
    const int last_row = min(row0 + ROWS_PER_WAVE, nrows) - 1;
    const int last_pos = n - L + last_row / G;
    const int nkb = last_pos / BS + 1;

    float m[NH], l[NH];
    f32x4 acc[NH][DT];
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        m[ht] = kNegInf;
        l[ht] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const uint16_t* kc = (const uint16_t*)p.kc;
    const uint16_t* vc = (const uint16_t*)p.vc;
    const int32_t* table = p.block_tables + (size_t)seg * p.MB;
    const size_t tsz = (size_t)BS * D;
    int koff[KS], voff[DT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = col * D + (gq + 4 * ks) * 8;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) voff[dt] = (dt * 16 + col) * BS + 4 * gq;

    struct Tile {
        uint4 k[KS];
        uint2 v[DT];
    };
    auto load = [&](int kb, Tile& t) {
        const int phys = table[kb];
        const size_t base = ((size_t)phys * p.Hkv + kvh) * tsz;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) t.k[ks] = *(const uint4*)(kc + base + koff[ks]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) t.v[dt] = *(const uint2*)(vc + base + voff[dt]);
    };
    auto compute = [&](int kb, Tile& t) {
        const int key0 = kb * BS + 4 * gq;  // keys of this lane's four score rows
        uint2 phi[NH], plo[NH];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc = mma_16x16x32<K>(t.k[ks], qb[ht][ks], sc);
            float sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[j] = (key0 + j <= pos[ht]) ? sc[j] * p.scale_log2 : kNegInf;
            float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            bm = xor_max(bm, 16);
            bm = xor_max(bm, 32);
            // key 0 is visible to every row, so m is finite from the first block on
            const float mn = fmaxf(m[ht], bm);
            const float alpha = fast_exp2(m[ht] - mn);
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(sv[j] - mn);
            l[ht] = l[ht] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
            m[ht] = mn;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[ht][dt] *= alpha;
            phi[ht] = pack4<K>(pr[0], pr[1], pr[2], pr[3]);
            plo[ht] = pack4<K>(pr[0] - lo16<K>(phi[ht].x), pr[1] - hi16<K>(phi[ht].x), pr[2] - lo16<K>(phi[ht].y),
                               pr[3] - hi16<K>(phi[ht].y));
        }
        if (kb * BS + BS > n) {  // slots past the context may hold anything (NaN)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                uint32_t x = t.v[dt].x, y = t.v[dt].y;
                if (key0 + 0 >= n) x &= 0xffff0000u;
                if (key0 + 1 >= n) x &= 0x0000ffffu;
                if (key0 + 2 >= n) y &= 0xffff0000u;
                if (key0 + 3 >= n) y &= 0x0000ffffu;
                t.v[dt] = make_uint2(x, y);
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int ht = 0; ht < NH; ++ht) {
                acc[ht][dt] = mma_16x16x16<K>(t.v[dt], phi[ht], acc[ht][dt]);
                acc[ht][dt] = mma_16x16x16<K>(t.v[dt], plo[ht], acc[ht][dt]);
            }
        }
    };

    Tile ta, tb;
    load(0, ta);
    for (int kb = 0; kb < nkb; kb += 2) {
        if (kb + 1 < nkb) load(kb + 1, tb);
        compute(kb, ta);
        if (kb + 2 < nkb) load(kb + 2, ta);
        if (kb + 1 < nkb) compute(kb + 1, tb);
    }

#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        l[ht] = xor_sum(xor_sum(l[ht], 16), 32);
        if (!live[ht]) continue;
        const int r = row0 + ht * 16 + col;
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

template <int K, int D>
hipError_t run(const ChunkedParams& p, hipStream_t st) {
    const long long tiles = ((long long)p.max_q_len * p.G + ROWS_PER_WG - 1) / ROWS_PER_WG;
    const long long grid = tiles * p.Hkv * p.num_segs;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((chunked_mfma<K, D>), dim3((unsigned)grid), dim3(NW * 64), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunked(const ChunkedParams& p, int kind, hipStream_t st) {
    switch (kind * 1000 + p.D) {
    case KF16 * 1000 + 64: return run<KF16, 64>(p, st);
    case KF16 * 1000 + 128: return run<KF16, 128>(p, st);
    case KBF16 * 1000 + 64: return run<KBF16, 64>(p, st);
    case KBF16 * 1000 + 128: return run<KBF16, 128>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
