// decode_kernels.h -- paged-attention decode for gfx950, templated on the KV block
// size; decode.hip, decode_bs8.hip and decode_bs32.hip instantiate one block size each.
//
// Blockwise attention over a paged KV pool ("每生成一个字都要把全部权重读一遍", section on
// paging the KV cache, blockwise attention equation): each query head's scores
// against every cached token of its sequence, one softmax over all of them, and
// the weighted sum of V, read block by block through the block table.  Online
// softmax and split contexts reorder the sums without changing what is computed
// ("LLM 推理优化的系统视角", section 4.2: tiling changes execution order, not
// semantics).
//
// Work is counted in units: one unit is one 16-token tile of one stream, a stream
// being a (sequence, kv head, query-head chunk) triple (a tile is a 16-token block,
// half of a 32-token block, or two 8-token blocks).  Two schedules:
//  * balanced split (partition_size == 0): exactly as many one-wave workgroups as
//    fit on the GPU at once; wave w takes units [w U / N, (w+1) U / N) of the U
//    units in (sequence, stream, tile) order.  It walks them with several tiles in
//    flight, writes the normalised output of every stream it covers whole, and
//    leaves (m, l, acc) records for the at most two streams it covers in part (its
//    first and its last).  A merge kernel joins the pieces of split streams.
//  * fixed partitions (partition_size > 0): one wave per (stream, partition of
//    partition_size tokens); multi-partition streams leave one record per
//    partition for the merge kernel.
#pragma once

#include "decode_inner.h"
#include "device.h"
#include "internal.h"

#include <atomic>
#include <cstdlib>

namespace pkv {

namespace {

// 16-token tiles of a context of ctx tokens
__device__ __forceinline__ int ntiles(int ctx) { return ctx > 0 ? (ctx + kTileTokens - 1) / kTileTokens : 0; }

// Sequence s of a flattened batch is a decode sequence when its segment has one
// query row; dec_ctx is its context as the decode sees it (0 for other segments,
// which then hold no units), row_of its query/output row.
__device__ __forceinline__ bool is_decode(const DecodeParams& p, int s) {
    return !p.cu_q || p.cu_q[s + 1] - p.cu_q[s] == 1;
}
__device__ __forceinline__ int dec_ctx(const DecodeParams& p, int s) { return is_decode(p, s) ? p.context_lens[s] : 0; }
__device__ __forceinline__ size_t row_of(const DecodeParams& p, int s) { return p.cu_q ? (size_t)p.cu_q[s] : (size_t)s; }
// the same with a wave-uniform s, through scalar loads
__device__ __forceinline__ int dec_ctx_uniform(const DecodeParams& p, int s) {
    if (p.cu_q && scalar_load(p.cu_q, (size_t)s + 1) - scalar_load(p.cu_q, s) != 1) return 0;
    return scalar_load(p.context_lens, s);
}
__device__ __forceinline__ size_t row_of_uniform(const DecodeParams& p, int s) {
    return p.cu_q ? (size_t)scalar_load(p.cu_q, s) : (size_t)s;
}

// source of tile b of sequence s for kv head kvh (scalar loads of the block table;
// s and b are wave-uniform)
template <int BS>
__device__ __forceinline__ TileSrc tile_src(const DecodeParams& p, int s, int b, int kvh, int ctx, bool live) {
    TileSrc t{0, 0, 0, live};
    if (!live) return t;
    const size_t row = (size_t)uniform(s) * p.MB;
    if constexpr (BS == 16) {
        t.u0 = (size_t)scalar_load(p.block_tables, row + uniform(b)) * p.Hkv + kvh;
    } else if constexpr (BS == 32) {
        t.u0 = (size_t)scalar_load(p.block_tables, row + uniform(b >> 1)) * p.Hkv + kvh;
        t.part = b & 1;
    } else {
        static_assert(BS == 8, "block sizes 8, 16, 32");
        t.u0 = (size_t)scalar_load(p.block_tables, row + uniform(2 * b)) * p.Hkv + kvh;
        // a last tile with a single 8-token block reads that block twice (masked)
        t.u1 = 2 * b + 1 < (ctx + 7) / 8 ? (size_t)scalar_load(p.block_tables, row + uniform(2 * b + 1)) * p.Hkv + kvh
                                         : t.u0;
    }
    return t;
}

__device__ __forceinline__ long long wave_incl_scan(long long v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    return v;
}

// stream c of a sequence -> first query head and number of heads
struct Heads {
    int kvh, head0, nh;
};
template <int HT>
__device__ __forceinline__ Heads stream_heads(const DecodeParams& p, int c) {
    Heads h;
    h.kvh = c / p.chunks;
    const int k = c - h.kvh * p.chunks;
    h.head0 = h.kvh * p.G + k * HT;
    h.nh = min(HT, p.G - k * HT);
    return h;
}

// ---------------------------------------------------------------------------------------
// Where the balanced split's waves start.  Every wave needs the batch's unit count U
// and the sequence holding its first unit; the merge needs starts[s] = NS * (tiles of
// the decode sequences before s) for s = 0..S (starts[S] = U).
//  * Batches of at most kInWaveSeqs sequences: every split wave loads all context
//    lengths in one round (four per lane) and finds both from its registers; wave 0
//    writes starts[].
//  * Larger batches: a first launch of one workgroup (decode_split_prologue) scans the
//    tile counts, kPrologueThreads sequences at a time, into starts[]; each split wave
//    then reads U and finds its sequence with 64-way searches over starts[] (two
//    rounds of one load per lane for up to 4096 sequences), so the start-up of a wave
//    no longer grows with the batch.
// Empty decode sequences get a zero output: from the prologue, or from split wave
// s mod N in small batches (16-byte stores of a whole output row).
// ---------------------------------------------------------------------------------------
constexpr int kInWaveSeqs = 256;
constexpr int kPrologueThreads = 1024;

template <int EB>
__global__ __launch_bounds__(kPrologueThreads) void decode_split_prologue(DecodeParams p, int NS) {
    constexpr int kWaves = kPrologueThreads / 64;
    __shared__ long long wave_tot[kWaves];
    if (contract_broken(p.guard)) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    long long carry = 0;
    for (int base = 0; base < p.S; base += kPrologueThreads) {
        const int s = base + tid;
        const bool dec = s < p.S && is_decode(p, s);
        const int nb = dec ? ntiles(p.context_lens[s]) : 0;
        const long long incl = wave_incl_scan((long long)nb, lane);
        if (lane == 63) wave_tot[wv] = incl;
        __syncthreads();
        long long before = carry, round = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            const long long t = wave_tot[k];
            before += k < wv ? t : 0;
            round += t;
        }
        if (s < p.S) p.starts[s] = (long long)NS * (before + incl - nb);
        if (dec && nb == 0) {
            const size_t n16 = (size_t)p.Hq * p.D * EB / 16;
            uint4* row = (uint4*)((char*)p.out + row_of(p, s) * p.Hq * p.D * EB);
            for (size_t i = 0; i < n16; ++i) row[i] = make_uint4(0, 0, 0, 0);
        }
        carry += round;
        __syncthreads();  // wave_tot is rewritten by the next round
    }
    if (tid == 0) p.starts[p.S] = (long long)NS * carry;
}

// The sequence s whose units [starts[s], starts[s+1]) contain unit u (0 <= u < U):
// the last s with starts[s] <= u, found by 64-way searches (one load per lane each;
// two rounds for up to 4096 sequences).
__device__ __forceinline__ long long read_lane64(long long v, int src) {
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), src);
    return (long long)(lo | (hi << 32));
}

__device__ __forceinline__ int sequence_of_unit(const long long* starts, int S, long long u, int lane) {
    int a = 0, b = S;  // starts[a] <= u; the answer lies in [a, b)
    while (b - a > 1) {
        const int step = (b - a + 63) / 64;
        const int idx = a + lane * step;
        const unsigned long long le = __ballot(idx < b && starts[idx] <= u);
        a += (63 - __builtin_clzll(le)) * step;  // lane 0 always qualifies (idx = a)
        b = min(b, a + step);
        a = uniform(a);
        b = uniform(b);
    }
    return a;
}

// Which merge joins the pieces of the balanced split, from what the host knows (the
// streams of the batch against the split waves):
//  * at least one stream per four waves (many short streams, each cut into a couple of
//    pieces): one workgroup merges every head of a stream (decode_merge_stream) -- one
//    per split wave, reading the merge note the wave left, when there are at least as
//    many streams as waves; one per stream, finding its pieces through starts[], when
//    there are fewer (then most waves own no stream, and a workgroup per wave would
//    launch up to four times the workgroups, each as wide as a stream's heads);
//  * otherwise one workgroup per (stream, head) (decode_merge_head) with 2 groups of
//    128 lanes, or 8 when a stream averages more than 64 pieces -- and then, when there
//    are fewer than 64 (stream, head) pairs (one or two long sequences), one workgroup
//    per quarter of a (stream, head) with 32 groups of 32 lanes instead: four times the
//    workgroups, each group folding a handful of pieces in one round of loads.
struct MergeChoice {
    // 0: per stream, a workgroup per wave; 4: per stream, a workgroup per stream;
    // per head with 1: 2 groups, 2: 8 groups; 3: per quarter head, 32 groups
    int kind;
};
inline MergeChoice merge_choice(long long streams, int cap, int waves) {
    if (streams * 4 >= waves) return {streams >= waves ? 0 : 4};
    if (streams * 64 >= waves) return {1};
    return {streams * cap < 64 ? 3 : 2};
}

// Waves of the balanced split that take units: all N launched, unless the batch has
// fewer than kUnitsPerWave units per wave; then only enough for that many each (at
// least kMinWorkingWaves), so that a small batch or one long stream is not cut into a
// thousand pieces for the merge.  Every wave and both merges compute it from U alone,
// so it does not depend on the block size.
constexpr long long kUnitsPerWave = 32;
constexpr long long kMinWorkingWaves = 64;
__host__ __device__ __forceinline__ long long working_waves(long long U, long long N) {
    const long long want = (U + kUnitsPerWave - 1) / kUnitsPerWave;
    const long long n = want > kMinWorkingWaves ? want : kMinWorkingWaves;
    return n < N ? n : N;
}

// first wave whose unit range contains unit u (ranges [w U / N, (w+1) U / N))
__host__ __device__ __forceinline__ long long wave_of(long long u, long long U, long long N) {
    return ((u + 1) * N - 1) / U;
}

// wave_of where a merge finds its pieces: U < N there only with fewer units than
// kMinWorkingWaves (every unit then a piece of its own), so 32-bit arithmetic serves;
// otherwise the pieces are the consecutive waves from w0
__device__ __forceinline__ long long piece_wave(long long w0, long long i, long long a, long long U, long long N) {
    return U >= N ? w0 + i : (((int)(a + i) + 1) * (int)N - 1) / (int)U;
}

// ---------------------------------------------------------------------------------------
// balanced split
// ---------------------------------------------------------------------------------------
// A position in the unit order: tile b of stream c of sequence s (nb tiles, ctx tokens).
struct Cursor {
    int s, c, b, nb, ctx;
};

// the same cursor, asserted wave-uniform (so that the compiler keeps it in scalar registers)
__device__ __forceinline__ Cursor uniform_cursor(const Cursor& x) {
    return Cursor{uniform(x.s), uniform(x.c), uniform(x.b), uniform(x.nb), uniform(x.ctx)};
}

// Range [lo, hi) of the U units taken by split piece w of the N launched (a wave, or
// a cooperative workgroup), Nw = working_waves(U, N): [w U / Nw, (w+1) U / Nw), empty
// for w >= Nw; cur locates unit lo.  With `writer` (one wave per piece) also the
// merge note of piece w, and in small batches starts[] (piece 0) and the zero
// outputs of empty sequences s with s mod N = w.  Returns false for an empty range.
template <int EB>
__device__ __forceinline__ bool split_range(const DecodeParams& p, long long w, long long N_launched, int lane,
                                            bool writer, long long& U_out, long long& lo_out, long long& hi_out,
                                            Cursor& cur) {
    const int NS = p.Hkv * p.chunks;
    const bool small = p.S <= kInWaveSeqs;
    // small batches: lane l holds sequences 4 l .. 4 l + 3, their contexts and first
    // units in registers (one wave-wide scan over the lanes' tile sums)
    int ctxr[4];
    long long first[4];
    long long tiles = 0, lane_tiles = 0;
    if (small) {
        int nbv[4];
        bool decv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = 4 * lane + j;
            decv[j] = s < p.S && is_decode(p, s);
            ctxr[j] = decv[j] ? p.context_lens[s] : 0;
            nbv[j] = ntiles(ctxr[j]);
            lane_tiles += nbv[j];
        }
        const long long incl = wave_incl_scan(lane_tiles, lane);
        long long run = incl - lane_tiles;  // tiles of the sequences before 4 lane
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            first[j] = (long long)NS * run;
            run += nbv[j];
        }
        tiles = uniform(read_lane64(incl, 63));
        // zero outputs of the empty decode sequences s with s mod N = w
        const int nl = (int)N_launched, wi = (int)w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = 4 * lane + j;
            for (unsigned long long e = __ballot(writer && decv[j] && nbv[j] == 0 && s % nl == wi); e; e &= e - 1) {
                const int se = 4 * __builtin_ctzll(e) + j;
                const size_t n16 = (size_t)p.Hq * p.D * EB / 16;
                uint4* row = (uint4*)((char*)p.out + row_of_uniform(p, se) * p.Hq * p.D * EB);
                for (size_t i = lane; i < n16; i += 64) row[i] = make_uint4(0, 0, 0, 0);
            }
        }
        if (writer && w == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * lane + j < p.S) p.starts[4 * lane + j] = first[j];
            if (lane == 0) p.starts[p.S] = (long long)NS * tiles;
        }
    }
    // The unit count and the range bounds (64-bit divisions, which run on the vector
    // unit) are asserted wave-uniform, so that the counts and cursors derived from
    // them, and the branches on those, are scalar.
    const long long U = uniform(small ? (long long)NS * tiles : p.starts[p.S]);
    const long long N = uniform(working_waves(U, N_launched));
    const long long lo = w < N ? uniform(w * U / N) : U, hi = w < N ? uniform((w + 1) * U / N) : U;
    U_out = U;
    lo_out = lo;
    hi_out = hi;
    if (lo >= hi) {
        if (writer && lane == 0) p.notes[w] = MergeNote{0, U, -1, 0, 0, 0};
        return false;
    }

    // locate unit lo: its sequence, then its stream and tile inside the sequence
    {
        long long a0 = 0;  // first unit of sequence cur.s
        if (small) {
            // the lane whose sequences hold unit lo, then the sequence among its four
            const unsigned long long h =
                __ballot(first[0] <= lo && lo < first[0] + (long long)NS * lane_tiles);
            const int t = (int)__builtin_ctzll(h);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const long long fj = read_lane64(first[j], t);
                const int cj = read_lane(ctxr[j], t);
                if (fj <= lo && lo < fj + (long long)NS * ntiles(cj)) {
                    cur.s = 4 * t + j;
                    cur.ctx = cj;
                    a0 = fj;
                    break;
                }
            }
        } else {
            cur.s = sequence_of_unit(p.starts, p.S, lo, lane);
            cur.ctx = dec_ctx_uniform(p, cur.s);
            a0 = p.starts[cur.s];
        }
        cur.s = uniform(cur.s);
        cur.ctx = uniform(cur.ctx);
        cur.nb = ntiles(cur.ctx);
        const long long r = lo - uniform(a0);
        cur.c = (int)(r / cur.nb);
        cur.b = (int)(r - (long long)cur.c * cur.nb);
    }
    // merge note: this piece merges the stream it starts in when that stream began in
    // an earlier piece and ends in this one
    if (writer && lane == 0) {
        const long long a = lo - cur.b;
        const bool own = cur.b > 0 && a + cur.nb <= hi;
        p.notes[w] = MergeNote{a, U, own ? cur.s : -1, cur.c, cur.nb, 0};
    }
    return true;
}

// Results of finished stream segments staged in LDS (a workgroup of one wave) and
// written out after the wave's last tile load.  On gfx9 stores count on the same
// vector-memory counter as loads, in issue order: a store issued between tile loads
// makes the wave's wait for every later tile wait for the store as well.  `data`
// holds the items back to back (8-byte multiples), `dst`/`bytes` say where each goes.
template <int kBytes> struct SegmentStage {
    static constexpr int kItems = 16;
    alignas(16) char data[kBytes];
    char* dst[kItems];
    int bytes[kItems];
};
// waves with fewer tiles than this store their results directly
constexpr int kStageMinTiles = 64;
// sized so that the LDS does not cut the waves per SIMD the launch asks for (the
// two-tile ring runs up to four); a result that does not fit is stored directly
template <class Loop, int R> constexpr int stage_bytes() {
    return R == 2 ? 8192 : Loop::kWaves == 1 ? 24576 : 12288;
}

// Wave w of the N launched (wave-uniform) takes the units of split_range.  With
// kStage the segment results go through a SegmentStage in LDS.
template <class Loop, int R, bool kStage = false>
__device__ __forceinline__ void decode_split_wave(const DecodeParams& p, long long w, long long N_launched) {
    constexpr int HT = Loop::HT;
    constexpr int SB = kStage ? stage_bytes<Loop, R>() : 16;
    __shared__ SegmentStage<SB> stage;
    int staged_items = 0, staged_bytes = 0;  // wave-uniform
    const int lane = lane_id();
    const int NS = p.Hkv * p.chunks;
    long long U, lo, hi;
    Cursor cur;
    if (!split_range<Loop::kElemBytes>(p, w, N_launched, lane, true, U, lo, hi, cur)) return;
    lo = uniform(lo);
    hi = uniform(hi);
    cur = uniform_cursor(cur);
    auto advance = [&](Cursor& x) {
        if (++x.b < x.nb) return;
        x.b = 0;
        if (++x.c < NS) return;
        x.c = 0;
        do {
            ++x.s;
            x.ctx = x.s < p.S ? dec_ctx_uniform(p, uniform(x.s)) : kTileTokens;
            x.nb = ntiles(x.ctx);
        } while (x.nb == 0);
    };

    Loop L;
    L.init_lane(lane);
    typename Loop::State st;
    const long long cnt = hi - lo;
    // short ranges store directly: there the deferred stores cost more at the end than
    // they save (256 sequences of 64-512 tokens, ~36 tiles a wave: 62.5 us direct,
    // 63.0 us staged; 190 tiles a wave: 258.5 -> 253.0 us staged)
    const bool stage_on = kStage && cnt >= kStageMinTiles;
    long long issued = 0, done = 0;
    Cursor ac = cur, cc = cur;
    const int cap = min(p.G, HT);
    const size_t rec = (size_t)cap * (p.D + 2);
    int seg_b0 = cur.b;
    bool first_seg = true;
    Heads hd = stream_heads<HT>(p, cur.c);

    // every call issues the loads of one tile -- a real one while units remain,
    // else an empty one -- so the wait before each fold covers exactly its own tile
    auto issue = [&](typename Loop::Tile& t) {
        const bool live = issued < cnt;
        L.load(t, p.kc, p.vc, tile_src<Loop::kBS>(p, ac.s, ac.b, ac.c / p.chunks, ac.ctx, live));
        if (live) {
            advance(ac);
            ++issued;
        }
    };
    // the staged items go out, 8 bytes a lane (records are 8-byte aligned)
    auto flush = [&]() {
        int off = 0;
        for (int i = 0; i < staged_items; ++i) {
            char* dst = stage.dst[i];
            const int n = stage.bytes[i];
            for (int o = lane * 8; o < n; o += 512) *(uint2*)(dst + o) = *(const uint2*)(stage.data + off + o);
            off += n;
        }
        staged_items = 0;
        staged_bytes = 0;
    };
    auto compute = [&](typename Loop::Tile& t) {
        L.block(st, t, cc.ctx - cc.b * kTileTokens, p.scale_log2);
        if (done + 1 == cnt || cc.b + 1 == cc.nb) {
            L.finish(st);
            const bool whole = seg_b0 == 0 && cc.b + 1 == cc.nb;
            const size_t orow = row_of_uniform(p, uniform(cc.s));
            float* const rp = p.ws + ((size_t)w * 2 + (first_seg ? 0 : 1)) * rec;
            // to LDS while the stage has room, unless it is the wave's last segment
            const int n = whole ? hd.nh * p.D * Loop::kElemBytes : (int)(rec * sizeof(float));
            if (stage_on && done + 1 < cnt && staged_items < SegmentStage<SB>::kItems && staged_bytes + n <= SB) {
                char* l = stage.data + staged_bytes;
                if (whole)
                    L.store_out(st, l, 0, hd.nh, 0, hd.nh);
                else
                    L.store_partial(st, (float*)l, cap, hd.nh);
                if (lane == 0) {
                    stage.dst[staged_items] =
                        whole ? (char*)p.out + (orow * p.Hq + hd.head0) * p.D * Loop::kElemBytes : (char*)rp;
                    stage.bytes[staged_items] = n;
                }
                staged_items = uniform(staged_items + 1);
                staged_bytes = uniform(staged_bytes + n);
            } else {
                if (whole)
                    L.store_out(st, p.out, orow, p.Hq, hd.head0, hd.nh);
                else
                    L.store_partial(st, rp, cap, hd.nh);
            }
            first_seg = false;
        }
        advance(cc);
        ++done;
    };
    // Issue tile `tn`, then fold tile `tc`.  When tc opens a stream segment its
    // queries are loaded before tn's tiles, and waited for right there, with tn's
    // loads left in flight: the state of the previous segment is already stored.
    auto step = [&](typename Loop::Tile& tn, typename Loop::Tile& tc) {
        if (done == 0 || cc.b == 0) {
            seg_b0 = cc.b;
            hd = stream_heads<HT>(p, cc.c);
            L.start(st, p.q, row_of_uniform(p, uniform(cc.s)), p.Hq, hd.head0, hd.nh);
            issue(tn);
            vm_wait_le<Loop::kTileLoads>();
        } else {
            issue(tn);
        }
        compute(tc);
    };

    // ring of R tiles: R - 1 blocks in flight while one is folded
    typename Loop::Tile ring[R];
#pragma unroll
    for (int j = 0; j + 1 < R; ++j) issue(ring[j]);
    while (done < cnt) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            step(ring[(j + R - 1) % R], ring[j]);
            if (done >= cnt) break;
        }
    }
    if (staged_items > 0) flush();
}

template <class Loop, int R>
__global__ __launch_bounds__(64, Loop::kWaves) void decode_split(DecodeParams p) {
    if (contract_broken(p.guard)) return;
    decode_split_wave<Loop, R, true>(p, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------------------
// cooperative balanced split (loops with 32 heads per stream): piece w is a workgroup
// of kCoopWaves waves, one per SIMD, sharing one unit range [lo, hi); wave k folds
// units lo + k, lo + k + kCoopWaves, ... into its own state, so that the four waves
// stream neighbouring tiles of the same stream at the same time.  At the end of every
// stream segment of the range the waves join their (m, l, acc) states through LDS
// -- o = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k, a wave without tiles in the
// segment contributing nothing -- and each wave writes its quarter of the heads: the
// output when the segment is a whole stream, else the piece's record.  A stream is
// then cut into a quarter as many pieces as with one wave per piece: fewer, smaller
// records for the merge, and none when streams and ranges line up.
// ---------------------------------------------------------------------------------------
constexpr int kCoopWaves = 4;
// ring of each cooperative wave: two tiles in flight while one is folded.  Four waves
// a compute unit with the loop's own six-tile ring kept more bytes in flight than
// streaming reads gain from (one 131072-token MQA sequence: 30.1 -> 28.3 us with three)
constexpr int kCoopRing = 3;

// barrier over the workgroup's LDS traffic only: waits for this wave's LDS accesses,
// not for its global loads still in flight (a release fence would wait for those too)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <class Loop, int R>
__global__ __launch_bounds__(64 * kCoopWaves, 1) void decode_split_coop(DecodeParams p) {
    constexpr int HT = Loop::HT;
    constexpr int D = Loop::kD;
    constexpr int kSlot = HT * D + 2 * HT;  // acc[HT][D], m[HT], l[HT] of one wave
    __shared__ float slot[kCoopWaves][kSlot];
    __shared__ int used[kCoopWaves];
    if (contract_broken(p.guard)) return;
    const int lane = lane_id();
    const int k = uniform((int)(threadIdx.x >> 6));
    const long long w = blockIdx.x;
    const int NS = p.Hkv * p.chunks;
    long long U, lo, hi;
    Cursor cur;
    // the range depends on w alone: every wave of the workgroup returns here or none
    if (!split_range<Loop::kElemBytes>(p, w, gridDim.x, lane, k == 0, U, lo, hi, cur)) return;
    lo = uniform(lo);
    hi = uniform(hi);
    cur = uniform_cursor(cur);
    auto advance = [&](Cursor& x) {
        if (++x.b < x.nb) return;
        x.b = 0;
        if (++x.c < NS) return;
        x.c = 0;
        do {
            ++x.s;
            x.ctx = x.s < p.S ? dec_ctx_uniform(p, uniform(x.s)) : kTileTokens;
            x.nb = ntiles(x.ctx);
        } while (x.nb == 0);
    };
    auto next_stream = [&](Cursor& x) {
        x.b = x.nb - 1;
        advance(x);
    };
    // kCoopWaves units on: within the stream when it is long enough (the common case)
    auto advance_coop = [&](Cursor& x) {
        if (x.b + kCoopWaves < x.nb) {
            x.b += kCoopWaves;
            return;
        }
#pragma unroll
        for (int i = 0; i < kCoopWaves; ++i) advance(x);
    };

    Loop L;
    L.init_lane(lane);
    typename Loop::State st;
    // this wave's units: lo + k + kCoopWaves i, i < cnt
    const long long cnt = lo + k < hi ? (hi - lo - k + kCoopWaves - 1) / kCoopWaves : 0;
    long long issued = 0, done = 0;
    Cursor ac = cur;
    for (int i = 0; i < k; ++i) advance(ac);
    Cursor cc = ac;
    // the segment being accumulated: stream of sg, from unit su of the range
    Cursor sg = cur;
    long long su = lo;
    bool have = false;  // this wave has folded a tile of the segment
    const int cap = min(p.G, HT);
    const size_t rec = (size_t)cap * (D + 2);

    // close segment sg (every wave, in the same order), then move to the next stream
    auto close = [&]() {
        const long long sa = su - sg.b, send = min(hi, sa + sg.nb);
        const bool whole = sg.b == 0 && sa + sg.nb <= hi;
        const Heads hs = stream_heads<HT>(p, sg.c);
        if (have) {
            L.finish(st);
            L.store_partial(st, slot[k], HT, hs.nh);
        }
        if (lane == 0) used[k] = have;
        lds_barrier();
        // wave k joins heads k HW .. k HW + HW - 1; a lane takes E head_dim elements
        constexpr int HW = HT / kCoopWaves, LPH = 64 / HW, E = D / LPH;
        const int h = k * HW + lane / LPH, d0 = (lane % LPH) * E;
        if (h < hs.nh) {
            float M = kNegInf;
#pragma unroll
            for (int j = 0; j < kCoopWaves; ++j)
                if (used[j]) M = fmaxf(M, slot[j][HT * D + h]);
            float Ls = 0.f, O[E];
#pragma unroll
            for (int e = 0; e < E; ++e) O[e] = 0.f;
#pragma unroll
            for (int j = 0; j < kCoopWaves; ++j) {
                if (!used[j]) continue;
                const float wt = fast_exp2(slot[j][HT * D + h] - M);
                Ls += wt * slot[j][HT * D + HT + h];
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    const f32x4 a = *(const f32x4*)&slot[j][h * D + d0 + e];
                    O[e] += wt * a[0];
                    O[e + 1] += wt * a[1];
                    O[e + 2] += wt * a[2];
                    O[e + 3] += wt * a[3];
                }
            }
            if (whole) {
                const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
                uint16_t* o = (uint16_t*)p.out + (row_of_uniform(p, sg.s) * p.Hq + hs.head0 + h) * D + d0;
#pragma unroll
                for (int e = 0; e < E; e += 4)
                    *(uint2*)(o + e) = pack4<Loop::kKind>(O[e] * inv, O[e + 1] * inv, O[e + 2] * inv, O[e + 3] * inv);
            } else {
                // slot 0: the range's first segment; slot 1: its last, when that is another
                float* r = p.ws + ((size_t)w * 2 + (su == lo ? 0 : 1)) * rec;
#pragma unroll
                for (int e = 0; e < E; e += 4) *(f32x4*)(r + h * D + d0 + e) = f32x4{O[e], O[e + 1], O[e + 2], O[e + 3]};
                if (lane % LPH == 0) {
                    r[cap * D + h] = M;
                    r[cap * D + cap + h] = Ls;
                }
            }
        }
        lds_barrier();  // the slots are rewritten by the next segment
        su = send;
        next_stream(sg);
        have = false;
    };

    auto issue = [&](typename Loop::Tile& t) {
        const bool live = issued < cnt;
        L.load(t, p.kc, p.vc, tile_src<Loop::kBS>(p, ac.s, ac.b, ac.c / p.chunks, ac.ctx, live));
        if (live) {
            advance_coop(ac);
            ++issued;
        }
    };
    // Issue tile `tn`, then fold tile `tc` (unit cc): first close the segments before
    // cc's stream; when tc opens this wave's part of a segment its queries are loaded
    // before tn's tiles and waited for right there, with tn's loads left in flight.
    auto step = [&](typename Loop::Tile& tn, typename Loop::Tile& tc) {
        while (sg.s != cc.s || sg.c != cc.c) close();
        if (!have) {
            const Heads hd = stream_heads<HT>(p, cc.c);
            L.start(st, p.q, row_of_uniform(p, uniform(cc.s)), p.Hq, hd.head0, hd.nh);
            have = true;
            issue(tn);
            vm_wait_le<Loop::kTileLoads>();
        } else {
            issue(tn);
        }
        L.block(st, tc, cc.ctx - cc.b * kTileTokens, p.scale_log2);
        advance_coop(cc);
        ++done;
    };

    // ring of R tiles: R - 1 blocks in flight while one is folded
    typename Loop::Tile ring[R];
#pragma unroll
    for (int j = 0; j + 1 < R; ++j) issue(ring[j]);
    while (done < cnt) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            step(ring[(j + R - 1) % R], ring[j]);
            if (done >= cnt) break;
        }
    }
    while (su < hi) close();
}

// ---------------------------------------------------------------------------------------
// fixed partitions (plain batches only: cu_q is NULL)
// ---------------------------------------------------------------------------------------
template <class Loop>
__global__ __launch_bounds__(64, Loop::kWaves) void decode_fixed(DecodeParams p) {
    if (contract_broken(p.guard)) return;
    constexpr int HT = Loop::HT;
    const int NS = p.Hkv * p.chunks;
    int idx = blockIdx.x;
    const int part = idx % p.max_parts;
    idx /= p.max_parts;
    const int c = idx % NS;
    const int s = idx / NS;
    const int ctx = p.context_lens[s];
    const int nparts = ctx > 0 ? (ctx + p.part_tokens - 1) / p.part_tokens : 1;
    if (part >= nparts) return;
    const int t0 = part * p.part_tokens;
    const int t1 = min(ctx, t0 + p.part_tokens);
    const int b0 = t0 / kTileTokens;  // partitions are whole tiles
    const int nb = t1 > t0 ? (t1 - t0 + kTileTokens - 1) / kTileTokens : 0;
    const Heads hd = stream_heads<HT>(p, c);

    Loop L;
    L.init_lane(lane_id());
    typename Loop::State st;
    L.start(st, p.q, s, p.Hq, hd.head0, hd.nh);
    // ring of R tiles, R - 1 blocks in flight while one is folded; past the end
    // the loads are empty
    constexpr int R = Loop::kRing;
    typename Loop::Tile ring[R];
    auto issue = [&](int i, typename Loop::Tile& t) {
        L.load(t, p.kc, p.vc, tile_src<Loop::kBS>(p, s, b0 + i, hd.kvh, ctx, i < nb));
    };
#pragma unroll
    for (int j = 0; j + 1 < R; ++j) issue(j, ring[j]);
    for (int i = 0; i < nb; i += R) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            issue(i + j + R - 1, ring[(j + R - 1) % R]);
            L.block(st, ring[j], t1 - (b0 + i + j) * kTileTokens, p.scale_log2);
            if (i + j + 1 >= nb) break;
        }
    }
    L.finish(st);
    if (nparts == 1) {
        L.store_out(st, p.out, s, p.Hq, hd.head0, hd.nh);
    } else {
        const int cap = min(p.G, HT);
        const size_t rec = (size_t)cap * (p.D + 2);
        L.store_partial(st, p.ws + ((size_t)(s * NS + c) * p.max_parts + part) * rec, cap, hd.nh);
    }
}

// ---------------------------------------------------------------------------------------
// balanced split, many short streams: a workgroup merges all heads of one stream,
//   o = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i:
// with kByStream false, workgroup w takes the stream whose merge note wave w left
// (see MergeNote), if any; with kByStream true, workgroup b takes stream b (sequence
// b / NS, stream b % NS), its units found through starts[] (nothing to do when one
// wave holds the whole stream: that wave wrote its output).
// Its pieces are the waves w0 .. w whose unit ranges cut the stream (w0's last
// record, then slot 0 of the others); when U < N each unit sits alone in its wave.
// A thread takes four consecutive head_dim elements of one head, eight pieces at a
// time with all their loads in flight; the workgroup has
// as many threads as the stream has such quads (up to kMergeStreamThreads; 1024 for
// the 32 heads of an MQA stream at head_dim 128), so that one round of loads merges
// a stream of up to eight pieces.
// ---------------------------------------------------------------------------------------
constexpr int kMergeStreamThreads = 1024;

template <int K, int HT, bool kByStream>
__global__ __launch_bounds__(kMergeStreamThreads) void decode_merge_stream(DecodeParams p, int split_waves) {
    if (contract_broken(p.guard)) return;
    int ns, nc, nnb;
    long long a, U, N, w1;
    if constexpr (kByStream) {
        const int NS = p.Hkv * p.chunks;
        ns = blockIdx.x / NS;
        nc = blockIdx.x - ns * NS;
        if (!is_decode(p, ns)) return;
        nnb = ntiles(p.context_lens[ns]);
        if (nnb == 0) return;  // empty context: its zero output comes from the split kernel
        U = p.starts[p.S];
        N = working_waves(U, split_waves);
        a = p.starts[ns] + (long long)nc * nnb;
        w1 = wave_of(a + nnb - 1, U, N);
        if (wave_of(a, U, N) == w1) return;  // written whole by one wave
    } else {
        // the note, through scalar loads (fields: a, U as int64, then s, c, nb)
        const int32_t* nt = (const int32_t*)(p.notes + blockIdx.x);
        ns = scalar_load(nt, 4);
        if (ns < 0) return;
        a = scalar_load64(nt, 0);
        U = scalar_load64(nt, 2);
        N = working_waves(U, split_waves);
        nc = scalar_load(nt, 5);
        nnb = scalar_load(nt, 6);
        w1 = blockIdx.x;
    }
    const Heads hd = stream_heads<HT>(p, nc);
    const int cap = min(p.G, HT);
    const int D = p.D;
    const size_t rec = (size_t)cap * (D + 2);
    const size_t orow = row_of_uniform(p, ns);
    const long long w0 = wave_of(a, U, N);
    const float* first_rec = p.ws + ((size_t)w0 * 2 + (w0 * U / N == a ? 0 : 1)) * rec;  // w0's last segment
    const long long count = U >= N ? w1 - w0 + 1 : nnb;
    // record of piece i
    auto record = [&](long long i) -> const float* {
        if (i == 0) return first_rec;
        return p.ws + (size_t)piece_wave(w0, i, a, U, N) * 2 * rec;  // slot 0: that wave's first segment
    };
    // one online pass over the pieces, eight at a time: (M, L, O) rescaled by
    // 2^(M_old - M_new)
    constexpr int CH = 8;
    const int quads = D / 4;
    const int n = hd.nh * quads;
    for (int u = threadIdx.x; u < n; u += blockDim.x) {
        const int h = u / quads, d = (u - h * quads) * 4;
        float M = kNegInf, L = 0.f;
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
        for (long long i0 = 0; i0 < count; i0 += CH) {
            float mv[CH], lv[CH];
            f32x4 av[CH];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                mv[j] = kNegInf;
                lv[j] = 0.f;
                av[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (i0 + j < count) {
                    const float* r = record(i0 + j);
                    mv[j] = r[cap * D + h];
                    lv[j] = r[cap * D + cap + h];
                    // records are 8-byte aligned (cap (D + 2) floats each)
                    const f32x2 a0 = *(const f32x2*)(r + h * D + d), a1 = *(const f32x2*)(r + h * D + d + 2);
                    av[j] = f32x4{a0[0], a0[1], a1[0], a1[1]};
                }
            }
            float mn = M;
#pragma unroll
            for (int j = 0; j < CH; ++j) mn = fmaxf(mn, mv[j]);
            const float sc = fast_exp2(M - mn);
            L *= sc;
            O *= sc;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const float wt = fast_exp2(mv[j] - mn);
                L += wt * lv[j];
                O += wt * av[j];
            }
            M = mn;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const size_t e = (orow * p.Hq + hd.head0 + h) * D + d;
#pragma unroll
        for (int k = 0; k < 4; ++k) store_elem<K>(p.out, e + k, O[k] * inv);
    }
}

// ---------------------------------------------------------------------------------------
// merge of the pieces of a stream, one query head (or a 1/DS share of its head_dim)
// per workgroup:
//   o = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
// Pieces: the fixed partitions 0 .. nparts-1 of the stream, or, for the balanced
// split, the waves w0 .. w1 whose unit ranges cut the stream (w0's last record,
// then slot 0 of the others; when U < N each unit sits alone in its own wave).
// NG groups x (128 / DS) head_dim lanes; group g folds pieces g, g+NG, ... in one
// online pass, kChunk pieces at a time with all their loads in flight, (M, L, O)
// rescaled by 2^(M_old - M_new); the groups are joined through LDS at the end.
// (NG, DS) = (2, 1) for streams of tens of pieces, (8, 1) for hundreds, (32, 4) for
// hundreds of pieces of fewer than 64 (stream, head) pairs (see merge_choice).
// ---------------------------------------------------------------------------------------
template <int K, int HT, int NG, int DS>
__global__ __launch_bounds__(NG * 128 / DS) void decode_merge_head(DecodeParams p, int split_waves) {
    constexpr int kChunk = NG >= 8 ? 8 : 16;  // pieces per group in flight at once
    constexpr int GL = 128 / DS;   // head_dim lanes of a group
    __shared__ float other[NG - 1][GL + 2];
    if (contract_broken(p.guard)) return;
    const int NS = p.Hkv * p.chunks;
    const int cap = min(p.G, HT);
    int idx = blockIdx.x;
    const int part = idx % DS;
    idx /= DS;
    const int h = idx % cap;
    idx /= cap;
    const int c = idx % NS;
    const int s = idx / NS;
    const Heads hd = stream_heads<HT>(p, c);
    if (h >= hd.nh || !is_decode(p, s)) return;
    const int ctx = p.context_lens[s];
    const size_t orow = row_of(p, s);
    const int D = p.D;
    const size_t rec = (size_t)cap * (D + 2);
    const int tid = threadIdx.x;

    long long count, w0 = 0, U = 0, a = 0;
    long long N = split_waves;
    const float* first;
    if (split_waves == 0) {
        count = ctx > 0 ? (ctx + p.part_tokens - 1) / p.part_tokens : 1;
        if (count <= 1) return;
        first = p.ws + (size_t)(s * NS + c) * p.max_parts * rec;
    } else {
        const int nb = ntiles(ctx);
        if (nb == 0) return;  // empty context: its zero output comes from the split kernel
        U = p.starts[p.S];
        N = working_waves(U, split_waves);
        a = p.starts[s] + (long long)c * nb;
        w0 = wave_of(a, U, N);
        const long long w1 = wave_of(a + nb - 1, U, N);
        if (w0 == w1) return;  // written whole by one wave
        first = p.ws + ((size_t)w0 * 2 + (w0 * U / N == a ? 0 : 1)) * rec;  // w0's last segment
        count = U >= N ? w1 - w0 + 1 : nb;
    }
    auto record = [&](long long i) -> const float* {
        if (split_waves == 0) return first + i * rec;
        if (i == 0) return first;
        return p.ws + (size_t)piece_wave(w0, i, a, U, N) * 2 * rec;
    };
    const int g = tid / GL, lane = tid - g * GL;
    const int dn = D / DS;             // head_dim elements of this workgroup
    const int d = part * dn + lane;
    const bool dlive = lane < dn;
    const int dd = dlive ? d : 0;      // lanes past this share read element 0 and store nothing
    float M = kNegInf, L = 0.f, O = 0.f;
    for (long long i0 = g; i0 < count; i0 += (long long)NG * kChunk) {
        float mv[kChunk], lv[kChunk], av[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            mv[j] = kNegInf;
            lv[j] = av[j] = 0.f;
            const long long i = i0 + (long long)NG * j;
            if (i < count) {
                const float* r = record(i);
                mv[j] = r[cap * D + h];
                lv[j] = r[cap * D + cap + h];
                av[j] = r[h * D + dd];
            }
        }
        float mn = M;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) mn = fmaxf(mn, mv[j]);
        const float sc = fast_exp2(M - mn);  // M = -inf on the first chunk: sc = 0 and L = O = 0 anyway
        L *= sc;
        O *= sc;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const float wt = fast_exp2(mv[j] - mn);
            L += wt * lv[j];
            O += wt * av[j];
        }
        M = mn;
    }
    // join groups 1 .. NG-1 into group 0 (every piece has a finite m, so a group's M is
    // finite whenever it had a piece; a group without pieces keeps M = -inf, L = O = 0)
    if (g > 0) {
        other[g - 1][lane] = O;
        if (lane == 0) {
            other[g - 1][GL] = M;
            other[g - 1][GL + 1] = L;
        }
    }
    __syncthreads();
    if (g == 0 && dlive) {
        float mn = M;
#pragma unroll 8
        for (int k = 0; k < NG - 1; ++k) mn = fmaxf(mn, other[k][GL]);
        const float s0 = M == kNegInf ? 0.f : fast_exp2(M - mn);
        float Lt = L * s0, Ot = O * s0;
#pragma unroll 8
        for (int k = 0; k < NG - 1; ++k) {
            const float Mk = other[k][GL];
            const float sk = Mk == kNegInf ? 0.f : fast_exp2(Mk - mn);
            Lt += other[k][GL + 1] * sk;
            Ot += other[k][lane] * sk;
        }
        store_elem<K>(p.out, (orow * p.Hq + hd.head0 + h) * D + d, Lt > 0.f ? Ot / Lt : 0.f);
    }
}

// ---------------------------------------------------------------------------------------
// fixed partitions: merge of one query head of one stream per workgroup (streams
// can have hundreds of partitions).  256 threads = 2 groups x 128 head_dim lanes;
// group g folds partitions g, g+2, ...; the weights 2^(m_i - M) come from LDS.
// ---------------------------------------------------------------------------------------
template <int K, int HT>
__global__ __launch_bounds__(256) void decode_merge_fixed(DecodeParams p) {
    constexpr int kRound = 1024;  // partitions folded per round
    __shared__ float wts[kRound];
    __shared__ float red[8];
    __shared__ float part_o[128];
    if (contract_broken(p.guard)) return;
    const int NS = p.Hkv * p.chunks;
    const int cap = min(p.G, HT);
    int idx = blockIdx.x;
    const int h = idx % cap;
    idx /= cap;
    const int c = idx % NS;
    const int s = idx / NS;
    const Heads hd = stream_heads<HT>(p, c);
    if (h >= hd.nh) return;
    const int ctx = p.context_lens[s];
    const int nparts = ctx > 0 ? (ctx + p.part_tokens - 1) / p.part_tokens : 1;
    if (nparts <= 1) return;
    const int D = p.D;
    const size_t rec = (size_t)cap * (D + 2);
    const float* base = p.ws + (size_t)(s * NS + c) * p.max_parts * rec;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    float M = kNegInf;
    for (int i = tid; i < nparts; i += 256) M = fmaxf(M, base[i * rec + cap * D + h]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    if (lane == 0) red[wv] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float L = 0.f, O = 0.f;
    const int g = tid >> 7, d = tid & 127;
    for (int r0 = 0; r0 < nparts; r0 += kRound) {
        const int n = min(kRound, nparts - r0);
        __syncthreads();
        for (int i = tid; i < n; i += 256) {
            const float* r = base + (size_t)(r0 + i) * rec;
            const float w = fast_exp2(r[cap * D + h] - M);
            wts[i] = w;
            L += w * r[cap * D + cap + h];
        }
        __syncthreads();
        if (d < D) {
#pragma unroll 16
            for (int i = g; i < n; i += 2) O += wts[i] * base[(size_t)(r0 + i) * rec + h * D + d];
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) L += __shfl_xor(L, m, 64);
    if (lane == 0) red[4 + wv] = L;
    if (g == 1) part_o[d] = O;
    __syncthreads();
    L = red[4] + red[5] + red[6] + red[7];
    if (g == 0 && d < D)
        store_elem<K>(p.out, ((size_t)s * p.Hq + hd.head0 + h) * D + d, L > 0.f ? (O + part_o[d]) / L : 0.f);
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------

// one-wave workgroups of kernel f that fit on the current device at once, at most
// per_simd per SIMD (a loop sized for one wave per SIMD keeps that shape even when
// it happens to need fewer registers) (cached)
inline int resident_waves(const void* f, int slot, int per_simd) {
    static std::atomic<int> cache[64][128];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev][slot].load(std::memory_order_relaxed);
    if (v > 0) return v;
    const int cus = device_compute_units();
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, 64, 0) != hipSuccess || per_cu <= 0) per_cu = 4;
    if (per_cu > kSimdsPerCu * per_simd) per_cu = kSimdsPerCu * per_simd;
    v = cus * per_cu;
    if (v > kMaxSplitWaves) v = kMaxSplitWaves;
    cache[dev][slot].store(v, std::memory_order_relaxed);
    return v;
}

// the waves per SIMD the balanced split allows a loop (see run below)
template <class Loop> constexpr int split_per_simd() { return Loop::kWaves == 1 ? 1 : 4; }


// merge of the balanced split's pieces (see merge_choice)
template <int K, int HT>
void launch_split_merge(const DecodeParams& p, int NS, int cap, int waves, hipStream_t st) {
    const long long streams = (long long)p.S * NS;
    const unsigned per_head = (unsigned)(streams * cap);
    switch (merge_choice(streams, cap, waves).kind) {
    case 0:
    case 4: {
        // one thread per four head_dim elements of the stream's heads (a multiple of 64)
        const int quads = cap * p.D / 4;
        const int threads = quads >= kMergeStreamThreads ? kMergeStreamThreads : (quads + 63) / 64 * 64;
        if (merge_choice(streams, cap, waves).kind == 0)
            hipLaunchKernelGGL((decode_merge_stream<K, HT, false>), dim3((unsigned)waves), dim3(threads), 0, st, p,
                               waves);
        else
            hipLaunchKernelGGL((decode_merge_stream<K, HT, true>), dim3((unsigned)streams), dim3(threads), 0, st, p,
                               waves);
        break;
    }
    case 1: hipLaunchKernelGGL((decode_merge_head<K, HT, 2, 1>), dim3(per_head), dim3(256), 0, st, p, waves); break;
    case 2: hipLaunchKernelGGL((decode_merge_head<K, HT, 8, 1>), dim3(per_head), dim3(1024), 0, st, p, waves); break;
    default:
        hipLaunchKernelGGL((decode_merge_head<K, HT, 32, 4>), dim3(per_head * 4), dim3(1024), 0, st, p, waves);
        break;
    }
}

// shallow: the balanced split with a two-tile ring (one block in flight) instead of
// the inner loop's own depth (a test and measurement variant; both pipelines stay
// tested)
template <class Loop, int K>
hipError_t run(const DecodeParams& p0, bool split, bool shallow, int slot, hipStream_t st) {
    DecodeParams p = p0;
    p.chunks = (p.G + Loop::HT - 1) / Loop::HT;
    const int NS = p.Hkv * p.chunks;
    int waves = 0;
    if (split) {
        if (p.S > kInWaveSeqs)
            hipLaunchKernelGGL((decode_split_prologue<Loop::kElemBytes>), dim3(1), dim3(kPrologueThreads), 0, st, p,
                               NS);
        if (!shallow) {
            if constexpr (Loop::kCoop) {
                // one cooperative workgroup (a wave per SIMD) per compute unit
                waves = (int)std::min<long long>(device_compute_units(), kMaxSplitWaves);
                hipLaunchKernelGGL((decode_split_coop<Loop, kCoopRing>), dim3(waves), dim3(64 * kCoopWaves), 0,
                                   st, p);
            } else {
                // deep-ring loops are built for one wave per SIMD; the others take what fits
                waves = resident_waves((const void*)decode_split<Loop, Loop::kRing>, slot * 2 + 1,
                                       split_per_simd<Loop>());
                hipLaunchKernelGGL((decode_split<Loop, Loop::kRing>), dim3(waves), dim3(64), 0, st, p);
            }
        } else {
            waves = resident_waves((const void*)decode_split<Loop, 2>, slot * 2, 4);
            hipLaunchKernelGGL((decode_split<Loop, 2>), dim3(waves), dim3(64), 0, st, p);
        }
    } else {
        const long long grid = (long long)p.max_parts * NS * p.S;
        hipLaunchKernelGGL(decode_fixed<Loop>, dim3((unsigned)grid), dim3(64), 0, st, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (!split && p.max_parts <= 1)) return e;
    const int cap = p.G < Loop::HT ? p.G : Loop::HT;
    const unsigned per_head = (unsigned)((long long)p.S * NS * cap);
    if (!split && cap > 8)  // many heads, hundreds of partitions: the online per-head merge
        hipLaunchKernelGGL((decode_merge_head<K, Loop::HT, 2, 1>), dim3(per_head), dim3(256), 0, st, p, 0);
    else if (!split)
        hipLaunchKernelGGL((decode_merge_fixed<K, Loop::HT>), dim3(per_head), dim3(256), 0, st, p);
    else
        launch_split_merge<K, Loop::HT>(p, NS, cap, waves, st);
    return hipGetLastError();
}

template <int K, int D, int BS>
hipError_t dispatch(const DecodeParams& p, bool mfma, bool split, bool shallow, hipStream_t st) {
    const int base = (K * 2 + (D == 128)) * 5;
    if constexpr (K != KF32) {
        if (mfma) {
            if (p.G <= 16) return run<MfmaLoop<K, D, 1, BS>, K>(p, split, shallow, base + 0, st);
            return run<MfmaWideLoop<K, D, BS>, K>(p, split, shallow, base + 1, st);
        }
    }
    if (p.G == 1) return run<ValuLoop<K, D, 1, BS>, K>(p, split, shallow, base + 2, st);
    if (p.G == 2) return run<ValuLoop<K, D, 2, BS>, K>(p, split, shallow, base + 3, st);
    return run<ValuLoop<K, D, 4, BS>, K>(p, split, shallow, base + 4, st);
}

// waves per SIMD of the balanced split for the loop dispatch() picks (block size
// does not change it)
template <int K, int D>
int per_simd_of(int G, bool mfma) {
    if constexpr (K != KF32) {
        if (mfma) return G <= 16 ? split_per_simd<MfmaLoop<K, D, 1, 16>>() : split_per_simd<MfmaWideLoop<K, D, 16>>();
    }
    if (G == 1) return split_per_simd<ValuLoop<K, D, 1, 16>>();
    if (G == 2) return split_per_simd<ValuLoop<K, D, 2, 16>>();
    return split_per_simd<ValuLoop<K, D, 4, 16>>();
}

// path: 0 automatic, 1 vector ALU inner loop, 2 matrix-core inner loop (16-bit types);
// ring: 0 the loop's own prefetch depth, 2 a two-tile ring (balanced split only)
template <int BS>
hipError_t launch_decode_block_size(const DecodeParams& p, int kind, int path, int ring, hipStream_t st) {
    const bool mfma = kind != KF32 && (path == 2 || (path == 0 && p.G >= 4));
    const bool split = p.part_tokens == 0;
    const bool sh = ring == 2;
    switch (kind * 1000 + p.D) {
    case KF32 * 1000 + 64: return dispatch<KF32, 64, BS>(p, false, split, sh, st);
    case KF32 * 1000 + 128: return dispatch<KF32, 128, BS>(p, false, split, sh, st);
    case KF16 * 1000 + 64: return dispatch<KF16, 64, BS>(p, mfma, split, sh, st);
    case KF16 * 1000 + 128: return dispatch<KF16, 128, BS>(p, mfma, split, sh, st);
    case KBF16 * 1000 + 64: return dispatch<KBF16, 64, BS>(p, mfma, split, sh, st);
    case KBF16 * 1000 + 128: return dispatch<KBF16, 128, BS>(p, mfma, split, sh, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace pkv
