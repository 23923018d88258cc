// chunked.hip -- launcher of the chunked-prefill kernel (chunked_kernels.h).
#include "chunked_kernels.h"

namespace pkv {

namespace {

template <int K, int D>
hipError_t run(const ChunkedParams& p, hipStream_t st) {
    const long long tiles = ((long long)p.max_q_len * p.G + ROWS_PER_WG - 1) / ROWS_PER_WG;
    const long long grid = tiles * p.Hkv * p.num_segs;
    if (grid == 0) return hipSuccess;
    switch (p.BS) {
    case 8: hipLaunchKernelGGL((chunked_fa<K, D, 8>), dim3((unsigned)grid), dim3(NW * 64), 0, st, p); break;
    case 16: hipLaunchKernelGGL((chunked_fa<K, D, 16>), dim3((unsigned)grid), dim3(NW * 64), 0, st, p); break;
    case 32: hipLaunchKernelGGL((chunked_fa<K, D, 32>), dim3((unsigned)grid), dim3(NW * 64), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
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
