// decode.hip -- paged-attention decode for KV blocks of 16 tokens, and the entry
// that picks the instantiation for the block size (8 and 32 live in decode_bs8.hip
// and decode_bs32.hip, compiled separately).
#include "decode_kernels.h"

namespace pkv {

hipError_t launch_decode_bs16(const DecodeParams& p, int kind, int path, hipStream_t st) {
    return launch_decode_block_size<16>(p, kind, path, st);
}

hipError_t launch_decode_path(const DecodeParams& p, int kind, int path, hipStream_t st) {
    switch (p.BS) {
    case 8: return launch_decode_bs8(p, kind, path, st);
    case 16: return launch_decode_bs16(p, kind, path, st);
    case 32: return launch_decode_bs32(p, kind, path, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeParams& p, int kind, hipStream_t st) {
    return launch_decode_path(p, kind, 0, st);
}

}  // namespace pkv
