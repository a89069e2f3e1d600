// Expert FFN: every expert's SwiGLU block on its rows of the send buffer, as
// two grouped GEMMs on bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation).  The expert is the gated three-matrix FFN ("MoE Expert
// Parallelism Sizing: Traffic, Capacity, Fabric", "Memory residency for the
// same shape"): h = SiLU(X W1^T) * (X W3^T), out = h W2^T.
//
//  gate/up GEMM  A = send_buf rows of expert e [M_e, d], B = W1_e and W3_e
//                [H, d] side by side; epilogue applies SiLU(g) * u and stores
//                h as bf16.
//  down GEMM     A = h [M_e, H], B = W2_e [d, H]; epilogue stores bf16.
//
// Both operands are K-contiguous ("NT"), so tiles go global -> registers ->
// LDS with 16-byte accesses and MFMA fragments are read from LDS rows padded
// by 16 bytes (no bank conflicts).  Ragged M: each workgroup scans the
// device-resident kept counts (one wavefront, E values) into a prefix of tile
// work per expert and finds its own (expert, N tile, M tile), so nothing waits
// on the host and no planning launch is needed.  The work order is expert-major, then N tile, then M
// tile: the M tiles that share a weight tile run side by side, and an XCD
// walks a contiguous range of experts (its L2 sees each expert's rows).
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int GBK = 64;         // K step
constexpr int GLD = GBK + 8;    // padded LDS row (elements)

struct GemmArgs {
    const uint16_t *A;          // [rows, K]
    const int32_t *row_offset;  // [E + 1] first row of each expert
    const int32_t *row_count;   // [E] rows of each expert
    const uint16_t *B0;         // [E, N, K]
    const uint16_t *B1;         // [E, N, K] (gate/up GEMM: W3) or null
    uint16_t *out;              // [rows, N]
    int E, N, K;
};

// Tile work of expert e is ceil(rows_e / BM) * (N / BN) tiles.  Wave 0 of the
// workgroup scans all experts (lane l owns experts [l*V, (l+1)*V)), maps the
// block to a work index with the XCD remap, and publishes (expert, local
// index) in LDS; e = -1 marks a surplus block.
template <int BM>
__device__ __forceinline__ void decode_work(const int32_t *__restrict__ rows, int E, int nN,
                                            int *s_e, int *s_local)
{
    const int lane = threadIdx.x & 63;
    const int V = (E + 63) >> 6;
    int sum = 0;
    for (int j = 0; j < V; ++j) {
        const int e = lane * V + j;
        if (e < E)
            sum += (rows[e] + BM - 1) / BM * nN;
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += o;
    }
    const int W = __shfl(incl, 63, 64);
    const int w = xcd_remap(blockIdx.x, W);
    if (lane == 0)
        *s_e = -1;
    if (w >= 0 && w >= incl - sum && w < incl) {
        int acc = incl - sum;
        for (int j = 0; j < V; ++j) {
            const int e = lane * V + j;
            if (e >= E)
                break;
            const int t = (rows[e] + BM - 1) / BM * nN;
            if (w < acc + t) {
                *s_e = e;
                *s_local = w - acc;
                break;
            }
            acc += t;
        }
    }
}

// Global -> register staging of one K step.  Every thread owns the same
// 16-byte chunks at every step (chunk c = tid + 256*j covers row c/8, column
// piece c%8), so its source rows are fixed and set up once.
template <int A_PT, int B_PT>
struct StageRegs {
    uint4 a[A_PT];
    uint4 b[B_PT];
};

template <int A_PT, int B_PT>
__device__ __forceinline__ void stage_load(StageRegs<A_PT, B_PT> &r,
                                           const uint16_t *const (&asrc)[A_PT],
                                           const uint16_t *const (&bsrc)[B_PT], int k0)
{
#pragma unroll
    for (int j = 0; j < A_PT; ++j)
        r.a[j] = asrc[j] ? *reinterpret_cast<const uint4 *>(asrc[j] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < B_PT; ++j)
        r.b[j] = *reinterpret_cast<const uint4 *>(bsrc[j] + k0);
}

template <int A_PT, int B_PT>
__device__ __forceinline__ void stage_store(const StageRegs<A_PT, B_PT> &r, uint16_t *As,
                                            uint16_t *Bs, int tid)
{
#pragma unroll
    for (int j = 0; j < A_PT; ++j) {
        const int c = tid + 256 * j;
        *reinterpret_cast<uint4 *>(As + (c >> 3) * GLD + (c & 7) * 8) = r.a[j];
    }
#pragma unroll
    for (int j = 0; j < B_PT; ++j) {
        const int c = tid + 256 * j;
        *reinterpret_cast<uint4 *>(Bs + (c >> 3) * GLD + (c & 7) * 8) = r.b[j];
    }
}

template <int BM, int BN, int WM, int WN, bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs g)
{
    static_assert(WM * WN == 4, "4 waves");
    constexpr int NB = DUAL ? 2 * BN : BN;            // B rows staged per step
    constexpr int WTM = BM / WM, WTN = BN / WN;       // wave tile
    constexpr int RT = WTM / 16, CT = WTN / 16;       // 16x16 MFMA tiles per wave
    constexpr int A_CH = BM * GBK / 8, B_CH = NB * GBK / 8;
    static_assert(A_CH % 256 == 0 && B_CH % 256 == 0, "whole chunks per thread");
    constexpr int A_PT = A_CH / 256, B_PT = B_CH / 256;
    constexpr int STAGE = (BM + NB) * GLD;
    constexpr int LDC = BN + 8;
    static_assert(BM * LDC <= 2 * STAGE, "epilogue tile fits in the staging LDS");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    __shared__ int s_e, s_local;
    if (threadIdx.x < 64)
        decode_work<BM>(g.row_count, g.E, g.N / BN, &s_e, &s_local);
    __syncthreads();
    const int e = s_e;
    if (e < 0)
        return;
    const int local = s_local;
    const int cnt = g.row_count[e];
    const int mt = (cnt + BM - 1) / BM;
    const int n_tile = local / mt, m_tile = local % mt;
    const int m0 = m_tile * BM;
    const int rows_valid = min(BM, cnt - m0);
    const size_t row0 = (size_t)g.row_offset[e] + m0;
    const int n0 = n_tile * BN;
    const int N = g.N, K = g.K;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // per-thread source rows (A rows past the expert's last row read as zero)
    const uint16_t *asrc[A_PT];
    const uint16_t *bsrc[B_PT];
#pragma unroll
    for (int j = 0; j < A_PT; ++j) {
        const int c = tid + 256 * j, r = c >> 3;
        asrc[j] = (r < rows_valid) ? g.A + (row0 + r) * K + (c & 7) * 8 : nullptr;
    }
#pragma unroll
    for (int j = 0; j < B_PT; ++j) {
        const int c = tid + 256 * j, r = c >> 3;
        const uint16_t *base = (DUAL && r >= BN) ? g.B1 : g.B0;
        const int rr = (DUAL && r >= BN) ? r - BN : r;
        bsrc[j] = base + ((size_t)e * N + n0 + rr) * K + (c & 7) * 8;
    }

    floatx4 acc0[RT][CT], acc1[DUAL ? RT : 1][DUAL ? CT : 1];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            acc0[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
            if constexpr (DUAL)
                acc1[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        }

    auto compute = [&](const uint16_t *As, const uint16_t *Bs) {
#pragma unroll
        for (int kk = 0; kk < GBK; kk += 32) {
            const int koff = kk + 8 * (lane >> 4);
            bf16x8 b0[CT], b1[DUAL ? CT : 1];
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                const int col = wn * WTN + j * 16 + (lane & 15);
                b0[j] = *reinterpret_cast<const bf16x8 *>(Bs + col * GLD + koff);
                if constexpr (DUAL)
                    b1[j] = *reinterpret_cast<const bf16x8 *>(Bs + (BN + col) * GLD + koff);
            }
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                if (wm * WTM + i * 16 >= rows_valid)
                    continue; // this 16-row slice is past the expert's last row
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    As + (wm * WTM + i * 16 + (lane & 15)) * GLD + koff);
#pragma unroll
                for (int j = 0; j < CT; ++j) {
                    acc0[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0[j], acc0[i][j], 0, 0, 0);
                    if constexpr (DUAL)
                        acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1[j], acc1[i][j], 0, 0, 0);
                }
            }
        }
    };

    // Pipeline: LDS holds steps i (being multiplied) and i+1 (being filled);
    // two register sets hold the loads of steps i+1 and i+2 in flight.
    const int nsteps = K / GBK;
    StageRegs<A_PT, B_PT> r0, r1;
    stage_load(r0, asrc, bsrc, 0);
    if (nsteps > 1)
        stage_load(r1, asrc, bsrc, GBK);
    stage_store(r0, lds, lds + BM * GLD, tid);
    __syncthreads();
    if (nsteps > 2)
        stage_load(r0, asrc, bsrc, 2 * GBK);
    for (int i = 0; i < nsteps; i += 2) {
        // step i: its tile is in buffer 0; step i+1 arrives in r1
        compute(lds, lds + BM * GLD);
        if (i + 1 < nsteps)
            stage_store(r1, lds + STAGE, lds + STAGE + BM * GLD, tid);
        __syncthreads();
        if (i + 3 < nsteps)
            stage_load(r1, asrc, bsrc, (i + 3) * GBK);
        if (i + 1 >= nsteps)
            break;
        // step i+1: buffer 1; step i+2 arrives in r0
        compute(lds + STAGE, lds + STAGE + BM * GLD);
        if (i + 2 < nsteps)
            stage_store(r0, lds, lds + BM * GLD, tid);
        __syncthreads();
        if (i + 4 < nsteps)
            stage_load(r0, asrc, bsrc, (i + 4) * GBK);
    }

    // Epilogue through LDS so that global stores are whole 16-byte row pieces.
    // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16)+q, column lane%16.
    uint16_t *Cs = lds;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = wm * WTM + i * 16 + 4 * (lane >> 4) + q;
                const int n = wn * WTN + j * 16 + (lane & 15);
                float v = acc0[i][j][q];
                if constexpr (DUAL) {
                    const float gt = v, up = acc1[i][j][q];
                    v = gt / (1.f + expf(-gt)) * up; // SiLU(g) * u
                }
                Cs[m * LDC + n] = (uint16_t)f32_to_bf16_rne(v);
            }
    __syncthreads();
    constexpr int CPR = BN / 8; // 16-byte pieces per output row
    for (int c = tid; c < BM * CPR; c += 256) {
        const int r = c / CPR, cc = c % CPR;
        if (r < rows_valid)
            *reinterpret_cast<uint4 *>(g.out + (row0 + r) * N + n0 + cc * 8) =
                *reinterpret_cast<const uint4 *>(Cs + r * LDC + cc * 8);
    }
}

constexpr int kBM = 128;  // M tile of both GEMMs
constexpr int kBN1 = 64;  // h columns per gate/up tile (x2 for W1 and W3)

} // namespace

hipError_t launch_gate_up(const Dims &dm, const uint16_t *send_buf, const int32_t *expert_offset,
                          const int32_t *expert_kept, const uint16_t *w1, const uint16_t *w3,
                          uint16_t *h, hipStream_t st)
{
    if (dm.send_rows == 0)
        return hipSuccess;
    const int nn = dm.H / kBN1;
    const long long mtiles_max = (dm.send_rows + kBM - 1) / kBM + dm.E;
    GemmArgs a{send_buf, expert_offset, expert_kept, w1, w3, h, dm.E, dm.H, dm.d};
    grouped_gemm_kernel<kBM, kBN1, 2, 2, true><<<xcd_grid((int)(mtiles_max * nn)), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_down(const Dims &dm, const uint16_t *h, const int32_t *expert_offset,
                       const int32_t *expert_kept, const uint16_t *w2, uint16_t *expert_out,
                       hipStream_t st)
{
    if (dm.send_rows == 0)
        return hipSuccess;
    const long long mtiles_max = (dm.send_rows + kBM - 1) / kBM + dm.E;
    GemmArgs a{h, expert_offset, expert_kept, w2, nullptr, expert_out, dm.E, dm.d, dm.H};
    if (dm.d % 128 == 0)
        grouped_gemm_kernel<kBM, 128, 2, 2, false>
            <<<xcd_grid((int)(mtiles_max * (dm.d / 128))), 256, 0, st>>>(a);
    else
        grouped_gemm_kernel<kBM, 64, 2, 2, false>
            <<<xcd_grid((int)(mtiles_max * (dm.d / 64))), 256, 0, st>>>(a);
    return hipGetLastError();
}

} // namespace moe
