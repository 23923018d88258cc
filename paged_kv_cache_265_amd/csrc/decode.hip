// decode.hip -- paged-attention decode for KV blocks of 16 tokens, and the entry
// that picks the instantiation for the block size (8 and 32 live in decode_bs8.hip
// and decode_bs32.hip, compiled separately).
#include "decode_kernels.h"

namespace pkv {

hipError_t launch_decode_bs16(const DecodeParams& p, int kind, int path, int ring, hipStream_t st) {
    return launch_decode_block_size<16>(p, kind, path, ring, st);
}

hipError_t launch_decode_path(const DecodeParams& p, int kind, int path, int ring, hipStream_t st) {
    switch (p.BS) {
    case 8: return launch_decode_bs8(p, kind, path, ring, st);
    case 16: return launch_decode_bs16(p, kind, path, ring, st);
    case 32: return launch_decode_bs32(p, kind, path, ring, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeParams& p, int kind, hipStream_t st) {
    return launch_decode_path(p, kind, 0, 0, st);
}

int device_compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

int split_waves_per_simd(int kind, int G, int D, int path, int ring) {
    const bool mfma = kind != KF32 && (path == 2 || (path == 0 && G >= 4));
    if (ring == 2) return 4;
    switch (kind * 1000 + D) {
    case KF32 * 1000 + 64: return per_simd_of<KF32, 64>(G, false);
    case KF32 * 1000 + 128: return per_simd_of<KF32, 128>(G, false);
    case KF16 * 1000 + 64: return per_simd_of<KF16, 64>(G, mfma);
    case KF16 * 1000 + 128: return per_simd_of<KF16, 128>(G, mfma);
    case KBF16 * 1000 + 64: return per_simd_of<KBF16, 64>(G, mfma);
    case KBF16 * 1000 + 128: return per_simd_of<KBF16, 128>(G, mfma);
    default: return 4;
    }
}

}  // namespace pkv
