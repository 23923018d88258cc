// cache_ops.hip -- the two companion writes of paged attention on gfx950.
//
// reshape_and_cache: new K/V rows go to the slots that slot_mapping names
// ("现代 LLM 推理引擎剖析", section 1.6; "LLM 推理优化的系统视角", section 3.1: a decode
// step appends the new token's K/V).  K rows land contiguously in the token-major
// K tile; a V row is spread over the head_dim-major V tile (stride block_size).
//
// copy_blocks: whole blocks are duplicated for copy-on-write of a block shared
// by several sequences ("每生成一个字都要把全部权重读一遍", copy-on-write paragraph).
// Both are bit copies: no conversion happens.
#include "device.h"
#include "internal.h"

namespace pkv {

namespace {

// reshape_and_cache: one workgroup per (group of 16 consecutive tokens, kv head).
// K rows go straight to their slots (16-byte pieces; a row is contiguous in the
// token-major tile).  V rows are staged in LDS and written out transposed: 16
// lanes take the 16 tokens of the group for one head_dim row, so tokens that fill
// consecutive offsets of one block write that row's slots as one contiguous run
// instead of one element every block_size elements.
// Both writes are non-temporal (streaming) stores.  The next kernel is usually the
// decode, which reads exactly these tiles (a sequence's last block) from workgroups
// on every XCD; with ordinary stores the written lines stayed behind in the
// writing XCD's L2, and reading them back cost the following GQA decode call of
// 256 sequences ~15 us (282 vs 268 us per write + decode), with streaming stores
// ~1 us.
constexpr int kTokGroup = 16;
constexpr int kCacheThreads = 128;

template <int EB>
__global__ __launch_bounds__(kCacheThreads) void reshape_and_cache_kernel(CacheParams p) {
    constexpr int VE = 16 / EB;                            // elements per 16-byte piece
    constexpr int kMaxRow = 128 * EB + 16;                 // LDS bytes per token row (D <= 128), padded
    __shared__ __attribute__((aligned(16))) char vrow[kTokGroup * kMaxRow];
    if (contract_broken(p.guard)) return;
    const int g = blockIdx.x;
    const int h = blockIdx.y;
    const int i0 = g * kTokGroup;
    const int nt = min(kTokGroup, p.num_tokens - i0);
    const int D = p.D;
    const int BS = p.BS;
    const int row = D * EB + 16;
    const int per_row = D / VE;

    // K to the cache, V rows to LDS
    for (int c = threadIdx.x; c < nt * per_row; c += kCacheThreads) {
        const int j = c / per_row;
        const int e0 = (c - j * per_row) * VE;
        const int64_t slot = p.slots[i0 + j];
        const size_t src = (((size_t)(i0 + j) * p.Hkv + h) * D + e0) * EB;
        const uint4 vv = *(const uint4*)((const char*)p.value + src);
        *(uint4*)(vrow + j * row + e0 * EB) = vv;
        if (slot < 0) continue;
        const int64_t blk = slot / BS;
        const int off = (int)(slot - blk * BS);
        const size_t tile = ((size_t)blk * p.Hkv + h) * BS * D;  // elements
        const uint4 kv = *(const uint4*)((const char*)p.key + src);
        __builtin_nontemporal_store(u32x4{kv.x, kv.y, kv.z, kv.w},
                                    (u32x4*)((char*)p.kc + (tile + (size_t)off * D + e0) * EB));
    }
    __syncthreads();
    // V from LDS: lane group of 16 = the group's tokens, one head_dim row each
    const int j = threadIdx.x % kTokGroup;
    if (j >= nt) return;
    const int64_t slot = p.slots[i0 + j];
    if (slot < 0) return;
    const int64_t blk = slot / BS;
    const int off = (int)(slot - blk * BS);
    const size_t tile = ((size_t)blk * p.Hkv + h) * BS * D;
    for (int d = threadIdx.x / kTokGroup; d < D; d += kCacheThreads / kTokGroup) {
        if constexpr (EB == 4)
            __builtin_nontemporal_store(*(const uint32_t*)(vrow + j * row + d * 4),
                                        (uint32_t*)p.vc + tile + (size_t)d * BS + off);
        else
            __builtin_nontemporal_store(*(const uint16_t*)(vrow + j * row + d * 2),
                                        (uint16_t*)p.vc + tile + (size_t)d * BS + off);
    }
}

// copy_blocks: workgroup (piece, pair, layer) copies 1/kCopySplit of block src to
// block dst in K and in V, every load issued before the stores (streaming stores,
// as in reshape_and_cache: the copies are read next by the decode).
constexpr int kCopySplit = 8;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
    if (contract_broken(p.guard)) return;
    const int piece = blockIdx.x % kCopySplit;
    const int pair = blockIdx.x / kCopySplit;
    const int layer = blockIdx.y;
    const int64_t src = p.mapping[2 * pair];
    const int64_t dst = p.mapping[2 * pair + 1];
    const size_t n = p.block_bytes / 16;  // 16-byte pieces per block
    const size_t per = (n + kCopySplit - 1) / kCopySplit;
    const size_t lo = piece * per, hi = min(n, lo + per);
    const uint4* ks = (const uint4*)((const char*)p.k[layer] + (size_t)src * p.block_bytes);
    const uint4* vs = (const uint4*)((const char*)p.v[layer] + (size_t)src * p.block_bytes);
    uint4* kd = (uint4*)((char*)p.k[layer] + (size_t)dst * p.block_bytes);
    uint4* vd = (uint4*)((char*)p.v[layer] + (size_t)dst * p.block_bytes);
    for (size_t i0 = lo + threadIdx.x; i0 < hi; i0 += (size_t)blockDim.x * kCopyUnroll) {
        uint4 a[kCopyUnroll], b[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = i0 + (size_t)u * blockDim.x;
            if (i < hi) {
                a[u] = ks[i];
                b[u] = vs[i];
            }
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = i0 + (size_t)u * blockDim.x;
            if (i < hi) {
                __builtin_nontemporal_store(u32x4{a[u].x, a[u].y, a[u].z, a[u].w}, (u32x4*)(kd + i));
                __builtin_nontemporal_store(u32x4{b[u].x, b[u].y, b[u].z, b[u].w}, (u32x4*)(vd + i));
            }
        }
    }
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheParams& p, int kind, hipStream_t st) {
    if (p.num_tokens == 0) return hipSuccess;
    const dim3 grid((unsigned)((p.num_tokens + kTokGroup - 1) / kTokGroup), (unsigned)p.Hkv);
    if (kind == KF32)
        hipLaunchKernelGGL(reshape_and_cache_kernel<4>, grid, dim3(kCacheThreads), 0, st, p);
    else
        hipLaunchKernelGGL(reshape_and_cache_kernel<2>, grid, dim3(kCacheThreads), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyParams& p, int num_layers, hipStream_t st) {
    if (p.num_pairs == 0 || num_layers == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)p.num_pairs * kCopySplit, num_layers), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace pkv
