// Combine: y[t] = sum over kept s of G[t,s] * Expert_{idx[t,s]}(x[t]), formed
// at the token's home device ("Mixture-of-Experts (MoE) Architecture and
// Expert Parallelism", section 2; "EP Math -- Expert Parallelism (MoE)",
// "The combine all-to-all").  A dropped assignment (slot -1) adds nothing
// ("Token drop"), and so does a slot past the send buffer's rows (a
// caller's slot array that moe_dispatch did not write).  With a shared
// expert (replicated on every rank, "MoE Expert Parallelism Sizing: Traffic,
// Capacity, Fabric", token-assignment worksheet) its bf16 output row is
// added last, with weight 1.
//
// A wavefront per token, or W of them when there are few tokens (fewer than
// 4096: DeepSeek-V3 decode has 64), wave h of a token then owning the
// contiguous pieces [h n / W, (h+1) n / W) of its row (n 16-byte pieces).
// The token's slots and gates are read once into scalar registers; for
// every piece the lane issues all k gathers before using any of them,
// accumulates G * row in fp32 in rank order, and stores the bf16 result
// (round to nearest even).  The gathers are non-temporal loads: every
// expert_out row is read once.  (Splitting the rows of 4096 or more tokens
// measured no faster at DeepSeek-V3 prefill shape and slower on the
// Mixtral-shaped and skewed layers; at 64 tokens one wave each leaves the
// chip all but idle.)
#include "moe_internal.hpp"

namespace moe {
namespace {

// acc[0..7] += the 8 bf16 values of one 16-byte row piece
__device__ __forceinline__ void add_row_piece(float *acc, uint4 v)
{
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(p[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(p[q] >> 16);
    }
}

template <int KM> // upper bound on k (compile time), so the gathers unroll
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ expert_out,
                                                      const int32_t *__restrict__ slot,
                                                      const float *__restrict__ topk_w,
                                                      const uint16_t *__restrict__ shared_out,
                                                      uint16_t *__restrict__ y, int T, int d,
                                                      int k, long long rows_max, int W)
{
    const int lane = threadIdx.x & 63;
    const int gwave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = gwave / W, h = gwave % W;
    if (t >= T)
        return;
    const int nvec = d / 8;
    const int c_lo = (int)((long long)h * nvec / W), c_hi = (int)((long long)(h + 1) * nvec / W);
    int rows[KM];
    float g[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        const int r = s < k ? __builtin_amdgcn_readfirstlane(slot[(size_t)t * k + s]) : -1;
        rows[s] = r >= 0 && r < rows_max ? r : -1; // a slot past the rows adds nothing
        g[s] = s < k ? __int_as_float(__builtin_amdgcn_readfirstlane(
                               __float_as_int(topk_w[(size_t)t * k + s])))
                         : 0.f;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(y + (size_t)t * d);
    for (int c = c_lo + lane; c < c_hi; c += 64) {
        uint4 v[KM];
#pragma unroll
        for (int s = 0; s < KM; ++s)
            v[s] = rows[s] >= 0
                       ? load_nt(reinterpret_cast<const uint4 *>(expert_out + (size_t)rows[s] * d) + c)
                       : make_uint4(0, 0, 0, 0);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KM; ++s) {
            if (rows[s] < 0)
                continue;
            const uint32_t p[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(g[s], bf16_to_f32(p[q] & 0xffffu), acc[2 * q]);
                acc[2 * q + 1] = fmaf(g[s], bf16_to_f32(p[q] >> 16), acc[2 * q + 1]);
            }
        }
        if (shared_out)
            add_row_piece(acc, reinterpret_cast<const uint4 *>(shared_out + (size_t)t * d)[c]);
        dst[c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
}

// Any k: the slots are walked in rank order, one gather at a time.
__global__ __launch_bounds__(256) void combine_kernel_any_k(
    const uint16_t *__restrict__ expert_out, const int32_t *__restrict__ slot,
    const float *__restrict__ topk_w, const uint16_t *__restrict__ shared_out,
    uint16_t *__restrict__ y, int T, int d, int k, long long rows_max, int W)
{
    const int lane = threadIdx.x & 63;
    const int gwave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = gwave / W, h = gwave % W;
    if (t >= T)
        return;
    const int nvec = d / 8;
    const int c_lo = (int)((long long)h * nvec / W), c_hi = (int)((long long)(h + 1) * nvec / W);
    const int32_t *sl = slot + (size_t)t * k;
    const float *gw = topk_w + (size_t)t * k;
    uint4 *dst = reinterpret_cast<uint4 *>(y + (size_t)t * d);
    for (int c = c_lo + lane; c < c_hi; c += 64) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < k; ++s) {
            const int r = sl[s];
            if (r < 0 || r >= rows_max)
                continue;
            const float g = gw[s];
            const uint4 v = load_nt(reinterpret_cast<const uint4 *>(expert_out + (size_t)r * d) + c);
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(g, bf16_to_f32(p[q] & 0xffffu), acc[2 * q]);
                acc[2 * q + 1] = fmaf(g, bf16_to_f32(p[q] >> 16), acc[2 * q + 1]);
            }
        }
        if (shared_out)
            add_row_piece(acc, reinterpret_cast<const uint4 *>(shared_out + (size_t)t * d)[c]);
        dst[c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
}

} // namespace

hipError_t launch_combine(const Dims &dm, const uint16_t *expert_out, const int32_t *slot,
                          const float *topk_w, const uint16_t *shared_out, uint16_t *y,
                          hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    const int W = combine_waves_per_token(dm.T, dm.d);
    const long long waves = (long long)dm.T * W;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
#define MOE_COMBINE(KERNEL)                                                                 \
    KERNEL<<<blocks, 256, 0, st>>>(expert_out, slot, topk_w, shared_out, y, dm.T, dm.d, dm.k, \
                                   dm.send_rows, W)
    if (dm.k <= 2)
        MOE_COMBINE(combine_kernel<2>);
    else if (dm.k <= 4)
        MOE_COMBINE(combine_kernel<4>);
    else if (dm.k <= 8)
        MOE_COMBINE(combine_kernel<8>);
    else
        MOE_COMBINE(combine_kernel_any_k);
#undef MOE_COMBINE
    return hipGetLastError();
}

} // namespace moe
