// mixed.hip -- one launch over a flattened batch of decode sequences and chunked-
// prefill segments, gfx950.
//
// The batch is the pages' mixed step: prefill chunks and decode tokens of many
// requests flattened into one pass ("现代 LLM 推理引擎剖析", sections 1.4 and 2.1).  A
// segment with one query row is a decode sequence; the others are prefill chunks.
// What is computed is exactly paged_attention_chunked's result for every segment;
// only the schedule differs:
//  * the first decode_wgs workgroups are decode workgroups: each of their four waves
//    is one wave of the balanced split over the decode sequences' 16-token tiles
//    (decode_split_wave), so long decode contexts are cut across many waves;
//  * the remaining workgroups are the chunked-prefill tiles of the other segments
//    (chunked_tile); tiles of one-row segments return at once.
// Decode workgroups come first in the grid, so they start first and stream K/V
// from HBM while prefill tiles keep the matrix cores busy beside them; when the
// decode waves are done their slots go to the remaining prefill tiles.  The merge
// of split decode streams runs as a second, small launch.
//
// The whole kernel is sized for two workgroups (two waves per SIMD) per compute
// unit, the chunked tiles' budget; the decode waves run a two-tile ring.
#include "chunked_kernels.h"
#include "decode_kernels.h"

namespace pkv {

namespace {

// the decode waves' ring: one tile in flight while one is folded.  Fewer decode loads in
// flight per CU leave the memory pipeline to the prefill tiles' K/V loads beside them
// (two 512-row chunks beside long MQA decode: 275 -> 266 us; one chunk beside the GQA
// batch: 336 -> 328 us; a four-tile ring was slower)
constexpr int kMixedRing = 2;

template <class Loop, int K, int D, int BS>
__global__ __launch_bounds__(NW * 64, 2) void mixed_kernel(DecodeParams dp, ChunkedParams cp, int decode_wgs,
                                                            int by_pair) {
    __shared__ __attribute__((aligned(16))) char st0[ChunkLds<D>::STAGE];
    __shared__ __attribute__((aligned(16))) char st1[ChunkLds<D>::STAGE];
    __shared__ __attribute__((aligned(16))) char st2[ChunkLds<D>::STAGE];
    if (contract_broken(dp.guard)) return;
    if ((int)blockIdx.x < decode_wgs) {
        const long long w = (long long)blockIdx.x * NW + uniform((int)(threadIdx.x >> 6));
        decode_split_wave<Loop, kMixedRing>(dp, w, (long long)decode_wgs * NW);
    } else {
        // with decode_wgs a multiple of 8 (one per CU) prefill workgroup i sits on XCD
        // i mod 8, as chunk_item assumes; otherwise only the L2 sharing suffers
        const int i = (int)blockIdx.x - decode_wgs;
        chunked_tile<K, D, BS>(cp, by_pair ? chunk_item(i, chunk_tiles(cp), cp.Hkv * cp.num_segs) : i, st0, st1, st2,
                               true);
    }
}

template <class Loop, int K, int D, int BS>
hipError_t go(const DecodeParams& dp0, const ChunkedParams& cp, long long prefill_rows, hipStream_t st) {
    DecodeParams dp = dp0;
    dp.chunks = (dp.G + Loop::HT - 1) / Loop::HT;
    const int NS = dp.Hkv * dp.chunks;
    // one decode workgroup (four waves: one per SIMD) per compute unit -- per two compute
    // units for the 32-head loop when the prefill tiles with rows (about prefill_rows x
    // Hq / ROWS_PER_WG) alone fill a slot on every unit: those decode waves keep the SIMDs
    // busier than the 16-head loop's, and the prefill tiles beside them get more room
    // (long MQA batch with eight 512-row chunks: 0.455 -> 0.443 ms; the GQA batch with
    // eight chunks, where the 16-head loop decodes, lost 4 % the same way)
    int decode_wgs = device_compute_units();
    if (Loop::kCoop && prefill_rows * cp.Hq >= (long long)decode_wgs * ROWS_PER_WG && decode_wgs >= 16)
        decode_wgs = decode_wgs / 16 * 8;
    if (decode_wgs * NW > kMaxSplitWaves) decode_wgs = kMaxSplitWaves / NW;
    const long long tiles = ((long long)cp.max_q_len * cp.G + ROWS_PER_WG - 1) / ROWS_PER_WG;
    const long long grid = decode_wgs + tiles * cp.Hkv * cp.num_segs;
    // Whole (segment, kv head) pairs per XCD (chunk_item) only when there are surely at
    // least as many prefill pairs as XCDs: a chunk holds at most max_q_len - 1 of the
    // prefill_rows, so there are at least prefill_rows / (max_q_len - 1) chunks.  With
    // fewer, whole pairs would leave XCDs without prefill work (two 512-row chunks beside
    // long MQA decode: 0.44 ms against 0.26 ms with every pair's tiles spread over all
    // XCDs in launch order), so the tiles go in launch order instead.
    const long long min_chunks = cp.max_q_len > 1 ? (prefill_rows + cp.max_q_len - 2) / (cp.max_q_len - 1) : 0;
    const int by_pair = min_chunks * cp.Hkv >= kXcds ? 1 : 0;
    if (dp.S > kInWaveSeqs)
        hipLaunchKernelGGL((decode_split_prologue<Loop::kElemBytes>), dim3(1), dim3(kPrologueThreads), 0, st, dp, NS);
    hipLaunchKernelGGL((mixed_kernel<Loop, K, D, BS>), dim3((unsigned)grid), dim3(NW * 64), 0, st, dp, cp,
                       decode_wgs, by_pair);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int waves = decode_wgs * NW;
    const int cap = dp.G < Loop::HT ? dp.G : Loop::HT;
    launch_split_merge<K, Loop::HT>(dp, NS, cap, waves, st);
    return hipGetLastError();
}

// decode inner loop as in paged_attention_decode: the vector ALU for one or two
// query heads per kv head, the matrix cores otherwise
template <int K, int D, int BS>
hipError_t pick(const DecodeParams& dp, const ChunkedParams& cp, long long prefill_rows, hipStream_t st) {
    if (dp.G == 1) return go<ValuLoop<K, D, 1, BS>, K, D, BS>(dp, cp, prefill_rows, st);
    if (dp.G == 2) return go<ValuLoop<K, D, 2, BS>, K, D, BS>(dp, cp, prefill_rows, st);
    if (dp.G <= 16) return go<MfmaLoop<K, D, 1, BS>, K, D, BS>(dp, cp, prefill_rows, st);
    return go<MfmaWideLoop<K, D, BS>, K, D, BS>(dp, cp, prefill_rows, st);
}

template <int K, int D>
hipError_t by_block_size(const DecodeParams& dp, const ChunkedParams& cp, long long prefill_rows, hipStream_t st) {
    switch (dp.BS) {
    case 8: return pick<K, D, 8>(dp, cp, prefill_rows, st);
    case 16: return pick<K, D, 16>(dp, cp, prefill_rows, st);
    case 32: return pick<K, D, 32>(dp, cp, prefill_rows, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_mixed(const DecodeParams& dp, const ChunkedParams& cp, int kind, long long prefill_rows,
                        hipStream_t st) {
    switch (kind * 1000 + dp.D) {
    case KF16 * 1000 + 64: return by_block_size<KF16, 64>(dp, cp, prefill_rows, st);
    case KF16 * 1000 + 128: return by_block_size<KF16, 128>(dp, cp, prefill_rows, st);
    case KBF16 * 1000 + 64: return by_block_size<KBF16, 64>(dp, cp, prefill_rows, st);
    case KBF16 * 1000 + 128: return by_block_size<KBF16, 128>(dp, cp, prefill_rows, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
