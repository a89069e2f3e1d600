// Router: logits H = x W_g (+ b) on bf16 matrix cores, then KeepTopK and a
// softmax over the kept logits ("Mixture-of-Experts (MoE) Architecture and
// Expert Parallelism", section 2 "The Gating Network Formulation"; the noise
// term is zero at inference).
//
// The logit GEMM (M = T tokens, N = E experts, K = d) uses
// v_mfma_f32_16x16x32_bf16: bf16 products are exact in fp32 and accumulate
// in fp32.  A workgroup of 4 waves computes a BT x BE tile; x and W_g tiles
// are staged through LDS, W_g transposed on the way in so that both MFMA
// operands are read K-contiguous.  KeepTopK runs one wavefront per token on
// order-preserving 64-bit keys (value bits, then E-1-e, so a tie goes to the
// lower expert index).
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int RBK = 64;          // K step of the logit GEMM
constexpr int RLD = RBK + 8;     // padded LDS row (elements): conflict-free 16 B reads

template <int BT, int BE, int WT, int WE>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int d, int E,
    int n_et, int total_tiles)
{
    static_assert(WT * WE == 4, "4 waves");
    constexpr int WTT = BT / WT; // tokens per wave
    constexpr int WTE = BE / WE; // experts per wave
    constexpr int RT = WTT / 16, CT = WTE / 16;
    static_assert(RT >= 1 && CT >= 1, "wave tile must be a multiple of 16");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BT * RLD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BE * RLD];

    const int w = xcd_remap(blockIdx.x, total_tiles);
    if (w < 0)
        return;
    const int t0 = (w / n_et) * BT;
    const int e0 = (w % n_et) * BE;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wt = wave / WE, we = wave % WE;
    const bool vec_b = (E % 8) == 0;

    // --- global -> register staging -------------------------------------
    constexpr int A_CH = BT * RBK / 8;         // 16-byte chunks of the x tile
    constexpr int A_PT = (A_CH + 255) / 256;
    constexpr int B_CH = RBK * BE / 8;         // 16-byte chunks of the W_g tile
    constexpr int B_PT = (B_CH + 255) / 256;
    uint4 ra[A_PT], rb[B_PT];

    auto load = [&](int k0) {
#pragma unroll
        for (int j = 0; j < A_PT; ++j) {
            const int c = tid + 256 * j;
            const int r = c / (RBK / 8), kc = c % (RBK / 8);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < A_CH && t0 + r < T)
                v = *reinterpret_cast<const uint4 *>(x + (size_t)(t0 + r) * d + k0 + kc * 8);
            ra[j] = v;
        }
#pragma unroll
        for (int j = 0; j < B_PT; ++j) {
            const int c = tid + 256 * j;
            const int kr = c / (BE / 8), ec = c % (BE / 8);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < B_CH) {
                const int e = e0 + ec * 8;
                const uint16_t *src = wg + (size_t)(k0 + kr) * E + e;
                if (vec_b && e + 8 <= E) {
                    v = *reinterpret_cast<const uint4 *>(src);
                } else {
                    uint16_t tmp[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        tmp[q] = (e + q < E) ? src[q] : (uint16_t)0;
                    v = make_uint4(tmp[0] | (tmp[1] << 16), tmp[2] | (tmp[3] << 16),
                                   tmp[4] | (tmp[5] << 16), tmp[6] | (tmp[7] << 16));
                }
            }
            rb[j] = v;
        }
    };
    auto store = [&](int s) {
#pragma unroll
        for (int j = 0; j < A_PT; ++j) {
            const int c = tid + 256 * j;
            if (c < A_CH) {
                const int r = c / (RBK / 8), kc = c % (RBK / 8);
                *reinterpret_cast<uint4 *>(&As[s][r * RLD + kc * 8]) = ra[j];
            }
        }
#pragma unroll
        for (int j = 0; j < B_PT; ++j) {
            const int c = tid + 256 * j;
            if (c < B_CH) {
                const int kr = c / (BE / 8), ec = c % (BE / 8);
                const uint32_t wv[4] = {rb[j].x, rb[j].y, rb[j].z, rb[j].w};
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    Bs[s][(ec * 8 + q) * RLD + kr] = (uint16_t)(wv[q >> 1] >> (16 * (q & 1)));
            }
        }
    };

    floatx4 acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = d / RBK;
    load(0);
    store(0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int s = step & 1;
        if (step + 1 < nsteps)
            load((step + 1) * RBK);
#pragma unroll
        for (int kk = 0; kk < RBK; kk += 32) {
            bf16x8 af[RT], bfr[CT];
#pragma unroll
            for (int i = 0; i < RT; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(
                    &As[s][(wt * WTT + i * 16 + (lane & 15)) * RLD + kk + 8 * (lane >> 4)]);
#pragma unroll
            for (int j = 0; j < CT; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(
                    &Bs[s][(we * WTE + j * 16 + (lane & 15)) * RLD + kk + 8 * (lane >> 4)]);
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < CT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j],
                                                                         0, 0, 0);
        }
        if (step + 1 < nsteps)
            store(s ^ 1);
        __syncthreads();
    }

    // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16)+q, column lane%16.
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int e = e0 + we * WTE + j * 16 + (lane & 15);
        if (e >= E)
            continue;
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = t0 + wt * WTT + i * 16 + 4 * (lane >> 4) + q;
                if (t < T)
                    logits[(size_t)t * E + e] = acc[i][j][q] + b;
            }
    }
}

// Order-preserving key of a finite fp32 logit and its expert index: larger
// key = larger logit; equal logits -> the lower index has the larger key.
__device__ __forceinline__ uint64_t topk_key(float v, int e, int E)
{
    uint32_t u = __float_as_uint(v == 0.f ? 0.f : v); // -0 and +0 compare equal
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(E - 1 - e);
}

__device__ __forceinline__ float key_value(uint64_t key)
{
    uint32_t u = (uint32_t)(key >> 32);
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((unsigned)(v & 0xffffffffu), off, 64);
        const uint32_t hi = __shfl_xor((unsigned)(v >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// One wavefront per token; lane l holds logits l, l+64, ... (V per lane).
template <int V>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float *__restrict__ logits,
                                                           int32_t *__restrict__ topk_idx,
                                                           float *__restrict__ topk_w, int T,
                                                           int E, int k)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T)
        return;
    const float *h = logits + (size_t)t * E;
    uint64_t key[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = lane + 64 * j;
        key[j] = e < E ? topk_key(h[e], e, E) : 0ull; // 0 sorts below every real key
    }
    float hmax = 0.f, denom = 0.f;
    // k rounds of a wave-wide arg-max; the winner's key is retired.  Lane
    // (s % 64) stores rank s's index and its unnormalised weight.
    for (int s = 0; s < k; ++s) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < V; ++j)
            best = key[j] > best ? key[j] : best;
        const uint64_t win = wave_max_u64(best);
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (key[j] == win)
                key[j] = 0;
        const int e = E - 1 - (int)(uint32_t)(win & 0xffffffffu);
        const float v = key_value(win);
        if (s == 0)
            hmax = v;
        const float p = expf(v - hmax);
        denom += p; // same order in every lane
        if (lane == (s & 63)) {
            topk_idx[(size_t)t * k + s] = e;
            topk_w[(size_t)t * k + s] = p;
        }
    }
    // normalise; each lane rereads only what it wrote itself
    for (int s = lane; s < k; s += 64) {
        const size_t o = (size_t)t * k + s;
        topk_w[o] = topk_w[o] / denom;
    }
}

} // namespace

hipError_t launch_router_logits(const Dims &dm, const uint16_t *x, const uint16_t *w_gate,
                                const float *bias, float *logits, hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    const int T = dm.T, E = dm.E, d = dm.d;
    if (E <= 16) {
        constexpr int BT = 64, BE = 16;
        const int n_tt = (T + BT - 1) / BT, n_et = (E + BE - 1) / BE, tiles = n_tt * n_et;
        router_logits_kernel<BT, BE, 4, 1><<<xcd_grid(tiles), 256, 0, st>>>(
            x, w_gate, bias, logits, T, d, E, n_et, tiles);
    } else if (E <= 32) {
        constexpr int BT = 64, BE = 32;
        const int n_tt = (T + BT - 1) / BT, n_et = (E + BE - 1) / BE, tiles = n_tt * n_et;
        router_logits_kernel<BT, BE, 2, 2><<<xcd_grid(tiles), 256, 0, st>>>(
            x, w_gate, bias, logits, T, d, E, n_et, tiles);
    } else {
        const int n_et = (E + 63) / 64;
        if ((long)((T + 63) / 64) * n_et >= 256) {
            constexpr int BT = 64, BE = 64;
            const int n_tt = (T + BT - 1) / BT, tiles = n_tt * n_et;
            router_logits_kernel<BT, BE, 2, 2><<<xcd_grid(tiles), 256, 0, st>>>(
                x, w_gate, bias, logits, T, d, E, n_et, tiles);
        } else {
            constexpr int BT = 32, BE = 64;
            const int n_tt = (T + BT - 1) / BT, tiles = n_tt * n_et;
            router_logits_kernel<BT, BE, 2, 2><<<xcd_grid(tiles), 256, 0, st>>>(
                x, w_gate, bias, logits, T, d, E, n_et, tiles);
        }
    }
    return hipGetLastError();
}

hipError_t launch_topk_softmax(const Dims &dm, const float *logits, int32_t *topk_idx,
                               float *topk_w, hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    const int blocks = (dm.T + 3) / 4;
    const int V = (dm.E + 63) / 64;
#define MOE_TOPK(VV)                                                                       \
    topk_softmax_kernel<VV><<<blocks, 256, 0, st>>>(logits, topk_idx, topk_w, dm.T, dm.E, dm.k)
    if (V <= 1)
        MOE_TOPK(1);
    else if (V <= 2)
        MOE_TOPK(2);
    else if (V <= 4)
        MOE_TOPK(4);
    else if (V <= 8)
        MOE_TOPK(8);
    else
        MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

} // namespace moe
