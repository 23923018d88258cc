// decode.hip -- paged-attention decode for gfx950.
//
// Blockwise attention over a paged KV pool ("每生成一个字都要把全部权重读一遍", section on
// paging the KV cache, blockwise attention equation): each query head's scores
// against every cached token, one softmax over all of them, and the weighted sum
// of V -- read block by block through the sequence's block table.  The softmax is
// computed online (running max m and running sum l per head, the accumulator
// rescaled by 2^(m_old - m_new) whenever the max grows), which reorders the sum
// without changing what is computed ("LLM 推理优化的系统视角", section 4.2: tiling
// changes execution order, not semantics).
//
// Work decomposition.  One workgroup of 4 waves handles one (sequence, kv head,
// head tile, partition); the partition is split block-cyclically over the
// waves, each wave keeping its own (m, l, acc) and prefetching its next 16-token
// block while it computes the current one.  The waves are merged in LDS.  A
// sequence longer than one partition leaves (m, l, unnormalised acc) per
// partition in the workspace and decode_reduce merges them.
//
// Two inner loops:
//  * decode_mfma (16-bit types, >= 4 query heads per kv head): scores S^T = K Q^T on
//    16x16x32 matrix cores (16 tokens x 16 heads per block), P V on 16x16x16 matrix
//    cores with P split into a high and a low 16-bit part so that P keeps ~16
//    significant bits.  Query heads beyond the group are zero columns.
//  * decode_valu (fp32, or fewer than 4 heads per kv head): four lanes per token
//    for the dot products (DPP/shuffle reductions), each lane owning head_dim/64
//    output columns for P V.
#include "device.h"
#include "internal.h"

namespace pkv {

namespace {

constexpr int NW = 4;            // waves per workgroup
constexpr int BS = kBlockSize;   // tokens per block

struct WorkItem {
    int s, kvh, hc0, nh, head0, part, nparts, t0, t1, b0, nb;
};

// Decode the flattened workgroup index: partition fastest, then head tile, then sequence.
__device__ __forceinline__ bool work_item(const DecodeParams& p, int HT, WorkItem& wi) {
    const int chunks = (p.G + HT - 1) / HT;
    int idx = blockIdx.x;
    wi.part = idx % p.max_parts;
    idx /= p.max_parts;
    const int hy = idx % (p.Hkv * chunks);
    wi.s = idx / (p.Hkv * chunks);
    wi.kvh = hy / chunks;
    wi.hc0 = (hy % chunks) * HT;
    wi.nh = min(HT, p.G - wi.hc0);
    wi.head0 = wi.kvh * p.G + wi.hc0;
    const int ctx = p.context_lens[wi.s];
    wi.nparts = ctx > 0 ? (ctx + p.part_tokens - 1) / p.part_tokens : 1;
    if (wi.part >= wi.nparts) return false;
    wi.t0 = wi.part * p.part_tokens;
    wi.t1 = min(ctx, wi.t0 + p.part_tokens);
    wi.b0 = wi.t0 / BS;
    wi.nb = wi.t1 > wi.t0 ? (wi.t1 - wi.t0 + BS - 1) / BS : 0;
    return true;
}

// LDS layout of the wave merge: m[NW][HT], l[NW][HT], acc[NW][MH][D + 4], where
// MH <= 16 heads are merged per round.
__host__ __device__ constexpr int merge_stride(int D) { return D + 4; }

size_t merge_lds_bytes(int HT, int MH, int D) {
    return sizeof(float) * (size_t)(2 * NW * HT + NW * MH * merge_stride(D));
}

// Merge the waves' (m, l, acc) for heads h0 .. h0+nm-1 of the tile (acc of head
// h0+i at sm_acc[(w * nm + i) * DP + d]) and write either the normalised output
// (single partition) or the partition's partial result.
template <int K>
__device__ void merge_waves(const DecodeParams& p, const WorkItem& wi, const float* sm_m, const float* sm_l,
                            const float* sm_acc, int HT, int h0, int nm) {
    const int D = p.D;
    const int DP = merge_stride(D);
    for (int e = threadIdx.x; e < nm * D; e += NW * 64) {
        const int i = e / D, d = e - i * D;
        const int h = h0 + i;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * HT + h]);
        float L = 0.f, O = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float wt = fast_exp2(sm_m[w * HT + h] - M);
                L += wt * sm_l[w * HT + h];
                O += wt * sm_acc[(w * nm + i) * DP + d];
            }
        }
        const size_t row = (size_t)wi.s * p.Hq + wi.head0 + h;
        if (wi.nparts == 1) {
            store_elem<K>(p.out, row * D + d, L > 0.f ? O / L : 0.f);
        } else {
            const size_t pr = row * p.max_parts + wi.part;
            p.ws_acc[pr * D + d] = O;
            if (d == 0) p.ws_ml[pr] = make_float2(M, L);
        }
    }
}

// ---------------------------------------------------------------------------------------
// matrix-core inner loop
// ---------------------------------------------------------------------------------------
template <int K, int D, int NH>
__global__ __launch_bounds__(NW * 64) void decode_mfma(DecodeParams p) {
    constexpr int KS = D / 32;   // k-steps of the score product
    constexpr int DT = D / 16;   // 16-column tiles of the output
    constexpr int HT = 16 * NH;  // query heads per workgroup
    extern __shared__ float lds[];

    WorkItem wi;
    if (!work_item(p, HT, wi)) return;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;  // token row of K / head column of the scores
    const int gq = lane >> 4;   // lane group: which 8 (or 4) k-elements
    const int nbw = wi.nb > w ? (wi.nb - w + NW - 1) / NW : 0;

    const uint16_t* qp = (const uint16_t*)p.q;
    uint4 qb[NH][KS];
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        const int h = ht * 16 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // d-chunk (gq + 4*ks): the same permutation of head_dim is used for K
            qb[ht][ks] = h < wi.nh ? *(const uint4*)(qp + ((size_t)wi.s * p.Hq + wi.head0 + h) * D + (gq + 4 * ks) * 8)
                                   : make_uint4(0, 0, 0, 0);
        }
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

    const uint16_t* kc = (const uint16_t*)p.kc;
    const uint16_t* vc = (const uint16_t*)p.vc;
    const int32_t* table = p.block_tables + (size_t)wi.s * p.MB;
    const size_t tile = (size_t)BS * D;
    int koff[KS], voff[DT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = col * D + (gq + 4 * ks) * 8;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) voff[dt] = (dt * 16 + col) * BS + 4 * gq;

    struct Tile {
        uint4 k[KS];
        uint2 v[DT];
    };
    auto load = [&](int it, Tile& t) {
        const int phys = table[wi.b0 + w + NW * it];
        const size_t base = ((size_t)phys * p.Hkv + wi.kvh) * tile;
        const uint16_t* kt = kc + base;
        const uint16_t* vt = vc + base;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) t.k[ks] = *(const uint4*)(kt + koff[ks]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) t.v[dt] = *(const uint2*)(vt + voff[dt]);
    };
    auto compute = [&](int it, Tile& t) {
        const int valid = wi.t1 - (wi.b0 + w + NW * it) * BS;  // tokens of this block inside the context
        uint2 phi[NH], plo[NH];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc = mma_16x16x32<K>(t.k[ks], qb[ht][ks], sc);
            float sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[j] = (4 * gq + j < valid) ? sc[j] * p.scale_log2 : kNegInf;
            float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            bm = xor_max(bm, 16);
            bm = xor_max(bm, 32);
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
        if (valid < BS) {  // last block of the context: slots past it may hold anything (NaN)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                uint32_t x = t.v[dt].x, y = t.v[dt].y;
                const int tk = 4 * gq;
                if (tk + 0 >= valid) x &= 0xffff0000u;
                if (tk + 1 >= valid) x &= 0x0000ffffu;
                if (tk + 2 >= valid) y &= 0xffff0000u;
                if (tk + 3 >= valid) y &= 0x0000ffffu;
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
    if (nbw > 0) load(0, ta);
    for (int it = 0; it < nbw; it += 2) {
        if (it + 1 < nbw) load(it + 1, tb);
        compute(it, ta);
        if (it + 2 < nbw) load(it + 2, ta);
        if (it + 1 < nbw) compute(it + 1, tb);
    }

    // per-head sums over the four lane groups
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) l[ht] = xor_sum(xor_sum(l[ht], 16), 32);

    float* sm_m = lds;
    float* sm_l = lds + NW * HT;
    float* sm_acc = lds + 2 * NW * HT;
    const int DP = merge_stride(D);
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        const int h = ht * 16 + col;
        if (gq == 0) {
            sm_m[w * HT + h] = m[ht];
            sm_l[w * HT + h] = l[ht];
        }
    }
    // one round of (up to) 16 heads at a time keeps the LDS footprint small
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
        const int nm = min(16, wi.nh - ht * 16);
        if (nm <= 0) break;
        if (ht > 0) __syncthreads();
        if (col < nm) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(f32x4*)(sm_acc + (w * nm + col) * DP + dt * 16 + 4 * gq) = acc[ht][dt];
        }
        __syncthreads();
        merge_waves<K>(p, wi, sm_m, sm_l, sm_acc, HT, ht * 16, nm);
    }
}

// ---------------------------------------------------------------------------------------
// vector-ALU inner loop
// ---------------------------------------------------------------------------------------
template <int K> __device__ __forceinline__ void widen16(uint4 c, float* f);
template <> __device__ __forceinline__ void widen16<KF32>(uint4 c, float* f) {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
}
template <int K> __device__ __forceinline__ void widen16(uint4 c, float* f) {
    const uint32_t u[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo16<K>(u[i]);
        f[2 * i + 1] = hi16<K>(u[i]);
    }
}

template <int K, int D, int GT>
__global__ __launch_bounds__(NW * 64) void decode_valu(DecodeParams p) {
    constexpr int EB = Elem<K>::bytes;
    constexpr int VE = 16 / EB;          // elements per 16-byte chunk
    constexpr int KC = D / VE / 4;       // K chunks per lane (four lanes per token)
    constexpr int DR = D / 64;           // output columns per lane
    constexpr int VC = DR * BS * EB / 16;  // V chunks per lane
    extern __shared__ float lds[];

    WorkItem wi;
    if (!work_item(p, GT, wi)) return;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tq = lane >> 2;   // token of the block this lane scores
    const int sub = lane & 3;   // which quarter of head_dim
    const int nbw = wi.nb > w ? (wi.nb - w + NW - 1) / NW : 0;

    const char* qp = (const char*)p.q;
    float qf[GT][KC * VE];
#pragma unroll
    for (int j = 0; j < GT; ++j) {
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            uint4 c = make_uint4(0, 0, 0, 0);
            if (j < wi.nh)
                c = *(const uint4*)(qp + (((size_t)wi.s * p.Hq + wi.head0 + j) * D + (sub + 4 * k) * VE) * EB);
            widen16<K>(c, &qf[j][k * VE]);
        }
    }

    float m[GT], l[GT], acc[GT][DR];
#pragma unroll
    for (int j = 0; j < GT; ++j) {
        m[j] = kNegInf;
        l[j] = 0.f;
#pragma unroll
        for (int r = 0; r < DR; ++r) acc[j][r] = 0.f;
    }

    const char* kc = (const char*)p.kc;
    const char* vc = (const char*)p.vc;
    const int32_t* table = p.block_tables + (size_t)wi.s * p.MB;
    const size_t tile_bytes = (size_t)BS * D * EB;

    struct Tile {
        uint4 k[KC];
        uint4 v[VC];
    };
    auto load = [&](int it, Tile& t) {
        const int phys = table[wi.b0 + w + NW * it];
        const size_t base = ((size_t)phys * p.Hkv + wi.kvh) * tile_bytes;
        const char* kt = kc + base + (size_t)tq * D * EB;
        const char* vt = vc + base + (size_t)lane * DR * BS * EB;
#pragma unroll
        for (int k = 0; k < KC; ++k) t.k[k] = *(const uint4*)(kt + (sub + 4 * k) * 16);
#pragma unroll
        for (int c = 0; c < VC; ++c) t.v[c] = *(const uint4*)(vt + c * 16);
    };
    auto compute = [&](int it, Tile& t) {
        const int valid = wi.t1 - (wi.b0 + w + NW * it) * BS;
        float kf[KC * VE];
#pragma unroll
        for (int k = 0; k < KC; ++k) widen16<K>(t.k[k], &kf[k * VE]);
        float pj[GT];
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < KC * VE; ++i) dot = fmaf(qf[j][i], kf[i], dot);
            dot = xor_sum(dot, 1);
            dot = xor_sum(dot, 2);
            const float sv = tq < valid ? dot * p.scale_log2 : kNegInf;
            float bm = xor_max(sv, 4);
            bm = xor_max(bm, 8);
            bm = xor_max(bm, 16);
            bm = xor_max(bm, 32);
            const float mn = fmaxf(m[j], bm);
            const float alpha = fast_exp2(m[j] - mn);
            pj[j] = fast_exp2(sv - mn);
            l[j] = l[j] * alpha + (sub == 0 ? pj[j] : 0.f);
            m[j] = mn;
#pragma unroll
            for (int r = 0; r < DR; ++r) acc[j][r] *= alpha;
        }
        float vf[DR * BS];  // vf[r * BS + token]
#pragma unroll
        for (int c = 0; c < VC; ++c) widen16<K>(t.v[c], &vf[c * VE]);
        if (valid < BS) {
#pragma unroll
            for (int r = 0; r < DR; ++r)
#pragma unroll
                for (int tk = 0; tk < BS; ++tk)
                    if (tk >= valid) vf[r * BS + tk] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < GT; ++j) {
#pragma unroll
            for (int tk = 0; tk < BS; ++tk) {
                const float pt = read_lane(pj[j], 4 * tk);
#pragma unroll
                for (int r = 0; r < DR; ++r) acc[j][r] = fmaf(pt, vf[r * BS + tk], acc[j][r]);
            }
        }
    };

    Tile ta, tb;
    if (nbw > 0) load(0, ta);
    for (int it = 0; it < nbw; it += 2) {
        if (it + 1 < nbw) load(it + 1, tb);
        compute(it, ta);
        if (it + 2 < nbw) load(it + 2, ta);
        if (it + 1 < nbw) compute(it + 1, tb);
    }

#pragma unroll
    for (int j = 0; j < GT; ++j) {
#pragma unroll
        for (int mask = 1; mask < 64; mask <<= 1) l[j] = xor_sum(l[j], mask);
    }

    float* sm_m = lds;
    float* sm_l = lds + NW * GT;
    float* sm_acc = lds + 2 * NW * GT;
    const int DP = merge_stride(D);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            sm_m[w * GT + j] = m[j];
            sm_l[w * GT + j] = l[j];
        }
    }
#pragma unroll
    for (int j = 0; j < GT; ++j) {
        if (j < wi.nh) {
#pragma unroll
            for (int r = 0; r < DR; ++r) sm_acc[(w * wi.nh + j) * DP + lane * DR + r] = acc[j][r];
        }
    }
    __syncthreads();
    merge_waves<K>(p, wi, sm_m, sm_l, sm_acc, GT, 0, wi.nh);
}

// ---------------------------------------------------------------------------------------
// merge of the partitions of one (sequence, query head)
// ---------------------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(128) void decode_reduce(DecodeParams p) {
    const int row = blockIdx.x;  // s * Hq + h
    const int s = row / p.Hq;
    const int ctx = p.context_lens[s];
    const int nparts = ctx > 0 ? (ctx + p.part_tokens - 1) / p.part_tokens : 1;
    if (nparts <= 1) return;
    const float2* ml = p.ws_ml + (size_t)row * p.max_parts;
    const float* acc = p.ws_acc + (size_t)row * p.max_parts * p.D;
    float M = kNegInf;
    for (int i = 0; i < nparts; ++i) M = fmaxf(M, ml[i].x);
    for (int d = threadIdx.x; d < p.D; d += blockDim.x) {
        float L = 0.f, O = 0.f;
        for (int i = 0; i < nparts; ++i) {
            const float2 v = ml[i];
            const float wt = fast_exp2(v.x - M);
            L += wt * v.y;
            O += wt * acc[(size_t)i * p.D + d];
        }
        store_elem<K>(p.out, (size_t)row * p.D + d, L > 0.f ? O / L : 0.f);
    }
}

template <int K, int D, int NH>
hipError_t run_mfma(const DecodeParams& p, hipStream_t st) {
    constexpr int HT = 16 * NH;
    const int chunks = (p.G + HT - 1) / HT;
    const size_t lds = merge_lds_bytes(HT, p.G < 16 ? p.G : 16, D);
    const long long grid = (long long)p.max_parts * p.Hkv * chunks * p.S;
    hipLaunchKernelGGL((decode_mfma<K, D, NH>), dim3((unsigned)grid), dim3(NW * 64), lds, st, p);
    return hipGetLastError();
}

template <int K, int D, int GT>
hipError_t run_valu(const DecodeParams& p, hipStream_t st) {
    const int chunks = (p.G + GT - 1) / GT;
    const size_t lds = merge_lds_bytes(GT, p.G < GT ? p.G : GT, D);
    const long long grid = (long long)p.max_parts * p.Hkv * chunks * p.S;
    hipLaunchKernelGGL((decode_valu<K, D, GT>), dim3((unsigned)grid), dim3(NW * 64), lds, st, p);
    return hipGetLastError();
}

template <int K, int D>
hipError_t dispatch(const DecodeParams& p, bool use_mfma, hipStream_t st) {
    hipError_t e;
    if (K != KF32 && use_mfma)
        e = p.G <= 16 ? run_mfma<K == KF32 ? KBF16 : K, D, 1>(p, st) : run_mfma<K == KF32 ? KBF16 : K, D, 2>(p, st);
    else
        e = p.G == 1 ? run_valu<K, D, 1>(p, st) : p.G == 2 ? run_valu<K, D, 2>(p, st) : run_valu<K, D, 4>(p, st);
    if (e != hipSuccess || p.max_parts <= 1) return e;
    hipLaunchKernelGGL((decode_reduce<K>), dim3((unsigned)(p.S * p.Hq)), dim3(128), 0, st, p);
    return hipGetLastError();
}

}  // namespace

// path: 0 = automatic (matrix cores for 16-bit types with >= 4 heads per kv head),
// 1 = vector ALU, 2 = matrix cores
hipError_t launch_decode_path(const DecodeParams& p, int kind, int path, hipStream_t st) {
    const bool mfma = kind != KF32 && (path == 2 || (path == 0 && p.G >= 4));
    switch (kind * 1000 + p.D) {
    case KF32 * 1000 + 64: return dispatch<KF32, 64>(p, false, st);
    case KF32 * 1000 + 128: return dispatch<KF32, 128>(p, false, st);
    case KF16 * 1000 + 64: return dispatch<KF16, 64>(p, mfma, st);
    case KF16 * 1000 + 128: return dispatch<KF16, 128>(p, mfma, st);
    case KBF16 * 1000 + 64: return dispatch<KBF16, 64>(p, mfma, st);
    case KBF16 * 1000 + 128: return dispatch<KBF16, 128>(p, mfma, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeParams& p, int kind, hipStream_t st) {
    return launch_decode_path(p, kind, 0, st);
}

}  // namespace pkv
