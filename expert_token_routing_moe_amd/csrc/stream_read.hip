// Streaming read of a device buffer with the same non-temporal 16-byte
// loads that the expert GEMMs use for their weights: the read rate that
// this device reaches, measured beside the kernels, for reading their
// HBM fractions against the device as well as against the data sheet.
// Its mirror, a streaming fill with the non-temporal 16-byte stores that
// the permute and the GEMM epilogues write with, gives the store rate, and
// a gather with the combine's access and none of its arithmetic gives the
// rate of that access itself.
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

// Every lane stores 8 pieces of 16 bytes per pass (grid-stride), the same
// value in every 32-bit word.
__global__ __launch_bounds__(256) void stream_write_kernel(uint4 *__restrict__ dst, size_t n16,
                                                           uint32_t value)
{
    const uint4 v = make_uint4(value, value, value, value);
    const size_t stride = (size_t)gridDim.x * 256 * kReadUnroll;
    for (size_t i = (size_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; i < n16; i += stride) {
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            if (i + (size_t)u * 256 < n16)
                store_nt(dst + i + (size_t)u * 256, v);
    }
}

// The combine's memory traffic without its arithmetic: out[t] = XOR over
// s < k of rows[slot[t, s]] (16-byte pieces; a slot outside [0, nrows)
// adds nothing).  As in the combine: W wavefronts per token, each over its
// contiguous share of the row's pieces, the slots read once into scalar
// registers, every gather of a piece issued before any is used (KM an upper
// bound on k; larger k one gather at a time), non-temporal gathers, 16-byte
// stores.
template <int KM>
__global__ __launch_bounds__(256) void stream_gather_kernel(const uint4 *__restrict__ rows,
                                                            const int32_t *__restrict__ slot,
                                                            int T, int k, int d16,
                                                            long long nrows,
                                                            uint4 *__restrict__ out, int W)
{
    const int lane = threadIdx.x & 63;
    const int gwave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = gwave / W, h = gwave % W;
    if (t >= T)
        return;
    const int c_lo = (int)((long long)h * d16 / W), c_hi = (int)((long long)(h + 1) * d16 / W);
    uint4 *dst = out + (size_t)t * d16;
    if (k > KM) {
        for (int c = c_lo + lane; c < c_hi; c += 64) {
            uint4 x = make_uint4(0, 0, 0, 0);
            for (int s = 0; s < k; ++s) {
                const int r = slot[(size_t)t * k + s];
                if (r < 0 || r >= nrows)
                    continue;
                const uint4 v = load_nt(rows + (size_t)r * d16 + c);
                x = make_uint4(x.x ^ v.x, x.y ^ v.y, x.z ^ v.z, x.w ^ v.w);
            }
            dst[c] = x;
        }
        return;
    }
    int rr[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        const int r = s < k ? __builtin_amdgcn_readfirstlane(slot[(size_t)t * k + s]) : -1;
        rr[s] = r >= 0 && r < nrows ? r : -1;
    }
    for (int c = c_lo + lane; c < c_hi; c += 64) {
        uint4 v[KM];
#pragma unroll
        for (int s = 0; s < KM; ++s)
            v[s] = rr[s] >= 0 ? load_nt(rows + (size_t)rr[s] * d16 + c) : make_uint4(0, 0, 0, 0);
        uint4 x = v[0];
#pragma unroll
        for (int s = 1; s < KM; ++s)
            x = make_uint4(x.x ^ v[s].x, x.y ^ v[s].y, x.z ^ v[s].z, x.w ^ v[s].w);
        dst[c] = x;
    }
}

} // namespace

hipError_t launch_stream_gather(const void *rows, long long nrows, int d, const int32_t *slot,
                                int T, int k, void *out, hipStream_t st)
{
    if (T == 0)
        return hipSuccess;
    const int W = combine_waves_per_token(T, d);
    const unsigned blocks = (unsigned)(((long long)T * W + 3) / 4);
    const int d16 = d / 8; // bf16 rows: 8 values per 16-byte piece
    const uint4 *r = static_cast<const uint4 *>(rows);
    uint4 *o = static_cast<uint4 *>(out);
    if (k <= 2)
        stream_gather_kernel<2><<<blocks, 256, 0, st>>>(r, slot, T, k, d16, nrows, o, W);
    else if (k <= 4)
        stream_gather_kernel<4><<<blocks, 256, 0, st>>>(r, slot, T, k, d16, nrows, o, W);
    else
        stream_gather_kernel<8><<<blocks, 256, 0, st>>>(r, slot, T, k, d16, nrows, o, W);
    return hipGetLastError();
}

hipError_t launch_stream_write(void *dst, size_t bytes, uint32_t value, hipStream_t st)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0)
        return hipSuccess;
    const size_t per_block = (size_t)256 * kReadUnroll;
    const unsigned blocks = (unsigned)std::min<size_t>(2048, (n16 + per_block - 1) / per_block);
    stream_write_kernel<<<blocks, 256, 0, st>>>(static_cast<uint4 *>(dst), n16, value);
    return hipGetLastError();
}

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
