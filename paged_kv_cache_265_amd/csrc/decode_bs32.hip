// decode_bs32.hip -- paged-attention decode for KV blocks of 32 tokens.
#include "decode_kernels.h"

namespace pkv {

hipError_t launch_decode_bs32(const DecodeParams& p, int kind, int path, int ring, hipStream_t st) {
    return launch_decode_block_size<32>(p, kind, path, ring, st);
}

}  // namespace pkv
