// Streaming read of a device buffer with the same non-temporal 16-byte
// loads that the expert GEMMs use for their weights: the read rate that
// this device reaches, measured beside the kernels, for reading their
// HBM fractions against the device as well as against the data sheet.
//
// Each lane keeps 8 loads in flight per pass (grid-stride over the buffer)
// and folds every 32-bit word it reads into an XOR.  A lane whose fold
// equals MOE_STREAM_READ_MARK stores it to *sink; nothing else is written,
// so the loads cannot be elided and no write traffic is added.  (An atomic
// fold of every wave into *sink cost 10-15% of the read rate.)  For a buffer
// of zeros holding the mark in one word, *sink receives the mark exactly
// when that word is read.
#include <algorithm>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src,
                                                          size_t n16, uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * 256 * kReadUnroll;
    for (size_t i = (size_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; i < n16; i += stride) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            v[u] = i + (size_t)u * 256 < n16 ? load_nt(src + i + (size_t)u * 256)
                                             : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == MOE_STREAM_READ_MARK)
        *sink = acc;
}

} // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0)
        return hipSuccess;
    // 2048 workgroups (8 per CU) measured at the plateau of a sweep over
    // 1024..4096; fewer when the buffer is small
    const size_t per_block = (size_t)256 * kReadUnroll;
    const unsigned blocks = (unsigned)std::min<size_t>(2048, (n16 + per_block - 1) / per_block);
    stream_read_kernel<<<blocks, 256, 0, st>>>(static_cast<const uint4 *>(src), n16, sink);
    return hipGetLastError();
}

} // namespace moe
