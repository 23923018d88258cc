// cache_ops.hip -- the two companion writes of paged attention on gfx950.
//
// reshape_and_cache: new K/V rows go to the slots that slot_mapping names
// ("现代 LLM 推理引擎剖析", section 1.6; "LLM 推理优化的系统视角", section 3.1: a decode
// step appends the new token's K/V).  K rows land contiguously in the token-major
// K tile; V rows are spread over the head_dim-major V tile (stride block_size).
//
// copy_blocks: whole blocks are duplicated for copy-on-write of a block shared
// by several sequences ("每生成一个字都要把全部权重读一遍", copy-on-write paragraph).
// Both are bit copies: no conversion happens.
#include "device.h"
#include "internal.h"

namespace pkv {

namespace {

constexpr int BS = kBlockSize;

// One workgroup per token; each thread moves 16-byte pieces of a (head, row).
template <int EB>
__global__ __launch_bounds__(128) void reshape_and_cache_kernel(CacheParams p) {
    constexpr int VE = 16 / EB;  // elements per 16-byte piece
    const int i = blockIdx.x;
    const int64_t slot = p.slots[i];
    if (slot < 0) return;
    const int64_t blk = slot / BS;
    const int off = (int)(slot - blk * BS);
    const int per_row = p.D / VE;
    const int n = p.Hkv * per_row;
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
        const int h = c / per_row;
        const int e0 = (c - h * per_row) * VE;  // first head_dim element of this piece
        const size_t src = (((size_t)i * p.Hkv + h) * p.D + e0) * EB;
        const uint4 kv = *(const uint4*)((const char*)p.key + src);
        const uint4 vv = *(const uint4*)((const char*)p.value + src);
        const size_t tile = ((size_t)blk * p.Hkv + h) * BS * p.D;  // elements
        *(uint4*)((char*)p.kc + (tile + (size_t)off * p.D + e0) * EB) = kv;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
        if constexpr (EB == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ((uint32_t*)p.vc)[tile + (size_t)(e0 + e) * BS + off] = w[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ((uint16_t*)p.vc)[tile + (size_t)(e0 + e) * BS + off] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// One workgroup per (pair, layer): copy block src to block dst in K and in V.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
    const int pair = blockIdx.x;
    const int layer = blockIdx.y;
    const int64_t src = p.mapping[2 * pair];
    const int64_t dst = p.mapping[2 * pair + 1];
    const size_t n = p.block_bytes / 16;
    const uint4* ks = (const uint4*)((const char*)p.k[layer] + (size_t)src * p.block_bytes);
    const uint4* vs = (const uint4*)((const char*)p.v[layer] + (size_t)src * p.block_bytes);
    uint4* kd = (uint4*)((char*)p.k[layer] + (size_t)dst * p.block_bytes);
    uint4* vd = (uint4*)((char*)p.v[layer] + (size_t)dst * p.block_bytes);
    for (size_t i = threadIdx.x; i < n; i += blockDim.x) {
        const uint4 a = ks[i];
        const uint4 b = vs[i];
        kd[i] = a;
        vd[i] = b;
    }
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheParams& p, int kind, hipStream_t st) {
    if (p.num_tokens == 0) return hipSuccess;
    if (kind == KF32)
        hipLaunchKernelGGL(reshape_and_cache_kernel<4>, dim3(p.num_tokens), dim3(128), 0, st, p);
    else
        hipLaunchKernelGGL(reshape_and_cache_kernel<2>, dim3(p.num_tokens), dim3(128), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyParams& p, int num_layers, hipStream_t st) {
    if (p.num_pairs == 0 || num_layers == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(p.num_pairs, num_layers), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace pkv
