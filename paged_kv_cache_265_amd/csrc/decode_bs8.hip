// decode_bs8.hip -- paged-attention decode for KV blocks of 8 tokens.
#include "decode_kernels.h"

namespace pkv {

hipError_t launch_decode_bs8(const DecodeParams& p, int kind, int path, int ring, hipStream_t st) {
    return launch_decode_block_size<8>(p, kind, path, ring, st);
}

}  // namespace pkv
