// Router: logits H = x W_g (+ b) on bf16 matrix cores, then KeepTopK and a
// softmax over the kept logits ("Mixture-of-Experts (MoE) Architecture and
// Expert Parallelism", section 2 "The Gating Network Formulation"; the noise
// term is zero at inference).
//
// Three launches:
//  1. W_g [d, E] is transposed into the workspace as W_g^T [E_pad, d]
//     (E_pad = E rounded up to 64, zero rows past E), so both operands of the
//     logit GEMM are K-contiguous.
//  2. The logit GEMM (M = T tokens, N = E_pad, K = d) on
//     v_mfma_f32_16x16x32_bf16: bf16 products are exact in fp32 and
//     accumulate in fp32.  A workgroup owns a 64-token x BE-expert tile and
//     one of SK slices of K, fed through an LDS ring by direct-to-LDS loads;
//     it writes fp32 partial logits [SK][T][E].  Splitting K fills the chip
//     when T*E is small.
//  3. KeepTopK + softmax, one wavefront per token: the SK partials are summed
//     in slice order and the bias added (the logits), then k rounds of a
//     wave-wide arg-max on order-preserving 64-bit keys (value bits, then
//     E-1-e, so a tie goes to the lower expert index).
#include <type_traits>

#include "moe_internal.hpp"
#include "ring.hpp"

namespace moe {

int router_epad(int E) { return (E + 63) / 64 * 64; }

// Experts per logit tile: all 256 of a multiple of 256 (one workgroup per
// CU, so x is read once per expert group of 256), else 128 or 64 (two
// workgroups per CU).
static int router_be(int E)
{
    const int epad = router_epad(E);
    return epad % 256 == 0 ? 256 : epad % 128 == 0 ? 128 : 64;
}

// Split of K for the logit GEMM: enough workgroups to cover the chip (one
// or two per CU), at least four K steps per slice.  Shared by the workspace
// layout.
int router_ksplit(int T, int E, int d)
{
    const int be = router_be(E);
    const int tiles = ((T + 63) / 64) * (router_epad(E) / be);
    const int steps = d / 64;
    if (tiles == 0)
        return 1; // T = 0: nothing to split
    const int target = be == 256 ? 256 : 512;
    int sk = (target + tiles - 1) / tiles;
    sk = std::min(sk, std::max(1, steps / 4));
    return std::max(1, sk);
}

namespace {

// W_g [d, E] -> W_g^T [E_pad, d], 64 x 64 tiles through LDS.  E % 8 == 0:
// 16-byte loads of 8 experts and 16-byte stores of 8 K values.
__global__ __launch_bounds__(256) void transpose_wg_vec_kernel(const uint16_t *__restrict__ wg,
                                                               uint16_t *__restrict__ wgt,
                                                               int d, int E)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72]; // [k][e], 144-byte rows
    const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    for (int c = threadIdx.x; c < 512; c += 256) {
        const int kr = c >> 3, ec = (c & 7) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (e0 + ec < E) // E % 8 == 0: all 8 experts are in range or none
            v = *reinterpret_cast<const uint4 *>(wg + (size_t)(k0 + kr) * E + e0 + ec);
        *reinterpret_cast<uint4 *>(&tile[kr][ec]) = v;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
        const int er = c & 63, kc = (c >> 6) * 8; // neighbouring lanes read neighbouring columns
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)tile[kc + 2 * j][er] | ((uint32_t)tile[kc + 2 * j + 1][er] << 16);
        *reinterpret_cast<uint4 *>(wgt + (size_t)(e0 + er) * d + k0 + kc) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Any E: element by element.
__global__ __launch_bounds__(256) void transpose_wg_kernel(const uint16_t *__restrict__ wg,
                                                           uint16_t *__restrict__ wgt, int d,
                                                           int E)
{
    __shared__ uint16_t tile[64][65];
    const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int kr = i / 64, ec = i % 64;
        const int e = e0 + ec;
        tile[kr][ec] = (e < E) ? wg[(size_t)(k0 + kr) * E + e] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int er = i / 64, kc = i % 64;
        wgt[(size_t)(e0 + er) * d + k0 + kc] = tile[kc][er];
    }
}

#ifndef MOE_ROUTER_WN
#define MOE_ROUTER_WN 4 // wave columns of a 256-expert logit tile (2 x WN waves)
#endif
constexpr int RBT = 64;   // tokens per tile
constexpr int RBK = 64;   // K step

template <int BE, int RRING, int MINB, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, MINB) void router_logits_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wgt,
    float *__restrict__ partial, int T, int d, int E, int n_et, int sk_count, int total)
{
    constexpr int NW = WM * WN;                    // waves per workgroup
    constexpr int RC = RBK / 8, RPI = 64 / RC;     // 8 pieces per row, 8 rows per load
    constexpr int A_PW = RBT / RPI / NW;           // x loads per wave per stage
    constexpr int B_PW = BE / RPI / NW;            // W_g^T loads per wave per stage
    static_assert(A_PW * RPI * NW == RBT && B_PW * RPI * NW == BE, "whole loads per wave");
    constexpr int A_BYTES = RBT * RBK * 2, STAGE = (RBT + BE) * RBK * 2;
    constexpr int S = RRING / STAGE < 8 ? RRING / STAGE : 8;
    static_assert(S >= 2, "two stages fit");
    constexpr int WTT = RBT / WM, WTE = BE / WN;   // WM x WN waves
    constexpr int RT = WTT / 16, CT = WTE / 16;
    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int w = xcd_remap(blockIdx.x, total);
    if (w < 0)
        return;
    // work order: K slice, then token tile, then expert tile.  The XCD remap
    // gives each XCD a contiguous range, so the workgroups of one XCD share
    // one slice of W_g^T in their L2 while each streams its own x rows.
    const int n_tt = total / (n_et * sk_count);
    const int et = w % n_et;
    const int tt = (w / n_et) % n_tt;
    const int sk = w / (n_et * n_tt);
    const int t0 = tt * RBT, e0 = et * BE;
    const int steps = d / RBK;
    const int s_lo = steps * sk / sk_count, s_hi = steps * (sk + 1) / sk_count;
    const int nsteps = s_hi - s_lo;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave / WN, we = wave % WN;

    const uint16_t *asrc[A_PW];
    const uint16_t *bsrc[B_PW];
#pragma unroll
    for (int j = 0; j < A_PW; ++j) {
        const int r = (NW * j + wave) * RPI + lane / RC;
        const int piece = (lane % RC) ^ swz<RC>(r);
        const int t = (t0 + r < T) ? t0 + r : t0; // rows past T read row t0 (never stored)
        asrc[j] = x + (size_t)t * d + (size_t)s_lo * RBK + piece * 8;
    }
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
        const int r = (NW * j + wave) * RPI + lane / RC;
        const int piece = (lane % RC) ^ swz<RC>(r);
        bsrc[j] = wgt + (size_t)(e0 + r) * d + (size_t)s_lo * RBK + piece * 8;
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS char *)smem;
    auto issue = [&](int step, int slot) {
        const uint32_t st = lds_base + slot * STAGE;
        const int k0 = step * RBK;
#pragma unroll
        for (int j = 0; j < A_PW; ++j)
            dma16(asrc[j] + k0, st + (NW * j + wave) * 1024);
#pragma unroll
        for (int j = 0; j < B_PW; ++j)
            dma16(bsrc[j] + k0, st + A_BYTES + (NW * j + wave) * 1024);
    };

    floatx4 acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int u = 0; u < S - 1 && u < nsteps; ++u)
        issue(u, u);
    for (int st = 0; st < nsteps; ++st) {
        const int ahead = min(S - 2, nsteps - 1 - st);
        wait_vmcnt(ahead * (A_PW + B_PW));
        ring_barrier();
        if (st + S - 1 < nsteps)
            issue(st + S - 1, (st + S - 1) % S);
        const char *As = smem + (st % S) * STAGE;
        const char *Bs = As + A_BYTES;
#pragma unroll
        for (int kc = 0; kc < RC; kc += 4) {
            const int piece = kc + (lane >> 4);
            bf16x8 a[RT], b[CT];
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const int r = wt * WTT + i * 16 + (lane & 15);
                a[i] = *reinterpret_cast<const bf16x8 *>(As + r * (RBK * 2) +
                                                         ((piece ^ swz<RC>(r)) << 4));
            }
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                const int n = we * WTE + j * 16 + (lane & 15);
                b[j] = *reinterpret_cast<const bf16x8 *>(Bs + n * (RBK * 2) +
                                                         ((piece ^ swz<RC>(n)) << 4));
            }
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < CT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j],
                                                                         0, 0, 0);
        }
    }

    // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16)+q, column lane%16.
    float *out = partial + (size_t)sk * T * E;
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int e = e0 + we * WTE + j * 16 + (lane & 15);
        if (e >= E)
            continue;
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = t0 + wt * WTT + i * 16 + 4 * (lane >> 4) + q;
                if (t < T)
                    out[(size_t)t * E + e] = acc[i][j][q];
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

// v = max(v, v of the lane that DPP control CTRL selects), for the rows in
// ROW_MASK; a lane without a source keeps its own value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t max_dpp(uint64_t v)
{
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, 0xF, false);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, 0xF, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}

// Maximum over the wavefront, returned in every lane: within each 16-lane row
// by quad permutes and the half-row / row mirrors, across rows by the row
// broadcasts of lanes 15 and 31 (lane 63 then holds the total).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    v = max_dpp<0xB1, 0xF>(v);  // quad_perm [1, 0, 3, 2]
    v = max_dpp<0x4E, 0xF>(v);  // quad_perm [2, 3, 0, 1]
    v = max_dpp<0x141, 0xF>(v); // row_half_mirror
    v = max_dpp<0x140, 0xF>(v); // row_mirror
    v = max_dpp<0x142, 0xA>(v); // row_bcast:15 into rows 1 and 3
    v = max_dpp<0x143, 0xC>(v); // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// The wave's own LDS operations have completed (lgkmcnt(0)); the compiler
// keeps memory accesses on their side.
__device__ __forceinline__ void lds_wait()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
}

// One wavefront per token; lane l holds logits l, l+64, ... (V per lane).
// The logit of (t, e) is the sum, in slice order, of the sk_count partials
// plus the bias; it is written to logits_out when that is non-null.
// Group limit ("MoE Expert Parallelism Sizing: Traffic, Capacity, Fabric":
// at most M nodes per token, Megatron's group-limited routing), when
// G > 1 and M < G: the E experts form G contiguous groups; each group's
// score is its best logit (LDS atomic max of the order-preserving key), the
// M best groups are picked by M wave arg-max rounds (ties to the lower
// group), and the other groups' experts are retired before KeepTopK.
template <int V>
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float *__restrict__ partial, int sk_count, const float *__restrict__ bias,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int T, int E, int k, int G, int M)
{
    __shared__ uint32_t s_gscore[4][kMaxExperts];
    __shared__ uint8_t s_allow[4][kMaxExperts];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T)
        return;
    // The lane's partial sums are loaded in batches of SKB slices, all
    // loads of a batch issued before any is added (one memory round trip per
    // batch instead of one per slice), then summed in slice order.
    constexpr int SKB = 8;
    float h[V], bv[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = lane + 64 * j;
        h[j] = 0.f;
        bv[j] = (bias && e < E) ? bias[e] : 0.f;
    }
    for (int s0 = 0; s0 < sk_count; s0 += SKB) {
        float pv[V][SKB];
#pragma unroll
        for (int j = 0; j < V; ++j)
#pragma unroll
            for (int u = 0; u < SKB; ++u) {
                const int e = lane + 64 * j, s = s0 + u;
                pv[j][u] = (e < E && s < sk_count) ? partial[((size_t)s * T + t) * E + e] : 0.f;
            }
#pragma unroll
        for (int j = 0; j < V; ++j)
#pragma unroll
            for (int u = 0; u < SKB; ++u)
                if (s0 + u < sk_count)
                    h[j] = s0 + u == 0 ? pv[j][u] : h[j] + pv[j][u];
    }
    uint64_t key[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = lane + 64 * j;
        key[j] = 0ull; // sorts below every real key
        if (e < E) {
            if (bias)
                h[j] += bv[j];
            if (logits_out)
                logits_out[(size_t)t * E + e] = h[j];
            key[j] = topk_key(h[j], e, E);
        }
    }
    if (G > 1 && M < G) {
        uint32_t *gs = s_gscore[wave];
        uint8_t *allow = s_allow[wave];
        const int per = E / G;
        for (int g = lane; g < G; g += 64) {
            gs[g] = 0u; // below every real score
            allow[g] = 0;
        }
        lds_wait();
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int e = lane + 64 * j;
            if (e < E)
                atomicMax(&gs[e / per], (uint32_t)(key[j] >> 32));
        }
        lds_wait();
        for (int r = 0; r < M; ++r) {
            uint64_t best = 0;
            for (int g = lane; g < G; g += 64) {
                const uint64_t gk = ((uint64_t)gs[g] << 32) | (uint32_t)(G - 1 - g);
                best = (gs[g] != 0u && gk > best) ? gk : best;
            }
            const int gw = G - 1 - (int)(uint32_t)(wave_max_u64(best) & 0xffffffffu);
            if (lane == 0) {
                gs[gw] = 0u; // retired
                allow[gw] = 1;
            }
            lds_wait();
        }
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !allow[e / per])
                key[j] = 0;
        }
    }
    float hmax = 0.f, denom = 0.f;
    // k rounds of a wave-wide arg-max; the winner's key is retired.  Lane s
    // keeps rank s's index and unnormalised weight (ranks past 64: lane
    // s % 64 stores them and rereads them to normalise).
    int my_e = 0;
    float my_p = 0.f;
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
            if (s < 64) {
                my_e = e;
                my_p = p;
            } else {
                topk_idx[(size_t)t * k + s] = e;
                topk_w[(size_t)t * k + s] = p;
            }
        }
    }
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = my_e;
        topk_w[(size_t)t * k + lane] = my_p / denom;
    }
    for (int s = lane + 64; s < k; s += 64) {
        const size_t o = (size_t)t * k + s;
        topk_w[o] = topk_w[o] / denom;
    }
}

hipError_t launch_topk(const Dims &dm, const float *partial, int sk, const float *bias,
                       float *logits_out, int32_t *topk_idx, float *topk_w, hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    const int blocks = (dm.T + 3) / 4;
    const int V = (dm.E + 63) / 64;
#define MOE_TOPK(VV)                                                                       \
    topk_softmax_kernel<VV><<<blocks, 256, 0, st>>>(partial, sk, bias, logits_out, topk_idx,  \
                                                   topk_w, dm.T, dm.E, dm.k, dm.n_groups,    \
                                                   dm.group_limit)
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

} // namespace

hipError_t launch_route(const Dims &dm, const uint16_t *x, const uint16_t *w_gate,
                        const float *bias, float *logits_out, int32_t *topk_idx, float *topk_w,
                        char *ws, const Workspace &wl, hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    const int T = dm.T, E = dm.E, d = dm.d;
    const int epad = router_epad(E);
    uint16_t *wgt = reinterpret_cast<uint16_t *>(ws + wl.wg_t);
    float *partial = reinterpret_cast<float *>(ws + wl.logits);
    if (E % 8 == 0)
        transpose_wg_vec_kernel<<<dim3(d / 64, epad / 64), 256, 0, st>>>(w_gate, wgt, d, E);
    else
        transpose_wg_kernel<<<dim3(d / 64, epad / 64), 256, 0, st>>>(w_gate, wgt, d, E);
    const int sk = router_ksplit(T, E, d);
    const int n_tt = (T + RBT - 1) / RBT;
    const int be = router_be(E), n_et = epad / be, total = n_tt * n_et * sk;
    if (be == 256)
        router_logits_kernel<256, 156 * 1024, 1, 2, MOE_ROUTER_WN>
            <<<xcd_grid(total), 2 * MOE_ROUTER_WN * 64, 0, st>>>(
            x, wgt, partial, T, d, E, n_et, sk, total);
    else if (be == 128)
        router_logits_kernel<128, 78 * 1024, 2, 2, 2><<<xcd_grid(total), 256, 0, st>>>(
            x, wgt, partial, T, d, E, n_et, sk, total);
    else
        router_logits_kernel<64, 78 * 1024, 2, 2, 2><<<xcd_grid(total), 256, 0, st>>>(
            x, wgt, partial, T, d, E, n_et, sk, total);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_topk(dm, partial, sk, bias, logits_out, topk_idx, topk_w, st);
}

hipError_t launch_topk_softmax(const Dims &dm, const float *logits, int32_t *topk_idx,
                               float *topk_w, hipStream_t st)
{
    return launch_topk(dm, logits, 1, nullptr, nullptr, topk_idx, topk_w, st);
}

} // namespace moe
