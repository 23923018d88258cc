// probe.hip -- streaming read of a device buffer: a measurement utility that
// gives the practical HBM read ceiling next to the decode kernels (it is not part
// of the attention path).  Each wave reads 4 KiB tiles w, w + W, ... with the
// same non-temporal 16-byte loads the decode kernels use.  Its shape is the
// fastest of a sweep on MI355X (1-8 workgroups of 4 waves per compute unit, 1-8
// tiles in flight per wave, with and without the non-temporal hint): one
// workgroup per compute unit with two tiles in flight per wave reads ~7.2 TB/s;
// more bytes in flight read less (four tiles 6.8-6.9, eight 5.0 TB/s).
#include "device.h"
#include "internal.h"

namespace pkv {

namespace {

constexpr int kInFlight = 2;

__global__ __launch_bounds__(256) void read_probe_kernel(const char* p, size_t tiles, unsigned* sink) {
    const int lane = lane_id();
    const size_t w = (blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6;
    const size_t W = (gridDim.x * (size_t)blockDim.x) >> 6;
    unsigned acc = 0;
    for (size_t t = w; t < tiles; t += W * kInFlight) {
        uint4 v[kInFlight][4];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const size_t ti = t + j * W;
            const bool live = ti < tiles;
            const rsrc_t r = tile_rsrc(p + (live ? ti : 0) * 4096, live ? 4096u : 0u);
#pragma unroll
            for (int c = 0; c < 4; ++c) v[j][c] = stream_load16(r, (uint32_t)(c * 64 + lane) * 16);
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc ^= v[j][c].x ^ v[j][c].y ^ v[j][c].z ^ v[j][c].w;
    }
    // keeps the loads alive; taken only if the XOR of everything read hits this value
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, void* sink, hipStream_t st) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)cus), dim3(256), 0, st, (const char*)buf, bytes / 4096,
                       (unsigned*)sink);
    return hipGetLastError();
}

}  // namespace pkv
