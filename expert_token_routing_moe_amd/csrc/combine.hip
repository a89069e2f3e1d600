// Combine: y[t] = sum over kept s of G[t,s] * Expert_{idx[t,s]}(x[t]), formed
// at the token's home device ("Mixture-of-Experts (MoE) Architecture and
// Expert Parallelism", section 2; "EP Math -- Expert Parallelism (MoE)",
// "The combine all-to-all").  A dropped assignment (slot -1) adds nothing
// ("Token drop").  A wavefront per token gathers its k expert rows with
// 16-byte loads, accumulates G * row in fp32 in rank order, and stores the
// bf16 result (round to nearest even) with 16-byte stores.
#include "moe_internal.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ expert_out,
                                                      const int32_t *__restrict__ slot,
                                                      const float *__restrict__ topk_w,
                                                      uint16_t *__restrict__ y, int T, int d,
                                                      int k)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T)
        return;
    const int nvec = d / 8;
    const int32_t *sl = slot + (size_t)t * k;
    const float *gw = topk_w + (size_t)t * k;
    uint4 *dst = reinterpret_cast<uint4 *>(y + (size_t)t * d);
    for (int c = lane; c < nvec; c += 64) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < k; ++s) {
            const int r = sl[s];
            if (r < 0)
                continue;
            const float g = gw[s];
            const uint4 v = reinterpret_cast<const uint4 *>(expert_out + (size_t)r * d)[c];
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(g, bf16_to_f32(p[q] & 0xffffu), acc[2 * q]);
                acc[2 * q + 1] = fmaf(g, bf16_to_f32(p[q] >> 16), acc[2 * q + 1]);
            }
        }
        dst[c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
}

} // namespace

hipError_t launch_combine(const Dims &dm, const uint16_t *expert_out, const int32_t *slot,
                          const float *topk_w, uint16_t *y, hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    combine_kernel<<<(dm.T + 3) / 4, 256, 0, st>>>(expert_out, slot, topk_w, y, dm.T, dm.d, dm.k);
    return hipGetLastError();
}

} // namespace moe
