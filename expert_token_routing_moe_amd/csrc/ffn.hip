// Expert FFN: every expert's SwiGLU block on its rows of the send buffer, as
// two grouped GEMMs on bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation).  The expert is the gated three-matrix FFN ("MoE Expert
// Parallelism Sizing: Traffic, Capacity, Fabric", "Memory residency for the
// same shape"): h = SiLU(X W1^T) * (X W3^T), out = h W2^T.
//
//  gate/up GEMM  A = send_buf rows of expert e [M_e, d], B = W1_e and W3_e
//                [H, d] side by side; the epilogue applies SiLU(g) * u and
//                stores h as bf16.
//  down GEMM     A = h [M_e, H], B = W2_e [d, H]; the epilogue stores bf16.
//
// Memory path.  Both operands are K-contiguous ("NT").  Tiles move global ->
// LDS with direct-to-LDS loads (global_load_lds_dwordx4): no staging
// registers, no LDS write instructions.  LDS is a ring of S stages, S chosen
// per tile from its row count (fewer rows, more stages); a stage is
// issued S-1 steps before it is multiplied, and each wave waits on its own
// load counter (s_waitcnt vmcnt) for exactly the stages it needs, then one
// workgroup barrier per step publishes the stage.  Rows are stored unpadded
// with an XOR swizzle of their 16-byte pieces, so the MFMA fragment reads are
// free of bank conflicts.  Weight loads are non-temporal (each weight byte is
// read once per M tile), A loads are not (every N tile re-reads them).
//
// Tiles.  An M tile holds up to 256 rows (an expert's rows are split into
// equal tiles), so every expert with at most 256 rows streams each weight
// tile from HBM exactly once; the 16-row slices of
// the tile are interleaved across the waves and empty slices are skipped
// (neither loaded nor multiplied).  Ragged M: each workgroup scans the
// device-resident kept counts (one wavefront, E values) into a prefix of tile
// work per expert and finds its own (expert, N tile, M tile), so nothing waits
// on the host.  The work order is expert-major, then N tile, then M tile, and
// the XCD remap gives each XCD a contiguous range of it: the N tiles of one
// expert run side by side and share that expert's rows in one L2.
//
// Epilogue.  A 4x4 transpose inside each lane quad (DPP) turns the MFMA
// layout into 8-byte row pieces, converted to bf16 by v_cvt_pk_bf16_f32; they
// are gathered in LDS (the ring is free by then) and leave as 16-byte
// non-temporal stores (the next kernel is the only reader).
//
// Shapes bound by the matrix cores (experts of hundreds of rows) take a
// second kernel with the same tiles and the same bits, whose two wave groups
// alternate between fragment reads and MFMAs (grouped_gemm_pp_kernel below).
#include <algorithm>
#include <type_traits>

#include "moe_internal.hpp"
#include "ring.hpp"

namespace moe {
namespace {


struct GemmArgs {
    const void *A;              // [rows, K] bf16, or E4M3 codes (A8)
    const float *a_scale;       // [rows] fp32 row scales (E4M3 rows; else null)
    const int32_t *row_offset;  // [E + 1] first row of each expert
    const int32_t *row_count;   // [E] rows of each expert
    const uint16_t *B0;         // [E, N, K]
    const uint16_t *B1;         // [E, N, K] (gate/up GEMM: W3) or null
    uint16_t *out;              // [rows, N]
    int E, N, K;
    int rot;                    // 1: each N tile starts its K walk at its own offset
    long long rows;             // rows of A and out: no tile reaches past them
};


// Inclusive prefix sum over the wavefront: within each 16-lane row by DPP
// row shifts of 1, 2, 4 and 8 (a lane without a source adds 0), then the
// totals of rows 0 and 2 into rows 1 and 3 (row broadcast of lane 15) and
// the total of rows 0-1 into rows 2 and 3 (row broadcast of lane 31).
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true); // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true); // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true); // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true); // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31
    return v;
}

// Tile work of expert e is ceil(rows_e / BM) * (N / BN) tiles.  Wave 0 of the
// workgroup scans all experts (lane l owns the V = ceil(E / 64) experts
// [l*V, (l+1)*V), their counts loaded together: E <= 1024, so V <= 16), maps
// the block to a work index with the XCD remap, and publishes (expert, local
// index) in LDS; e = -1 marks a surplus block.
template <int BM>
__device__ __forceinline__ void decode_work(const GemmArgs &g, int nN, int *s_e, int *s_local)
{
    const int lane = threadIdx.x & 63;
    const int E = g.E;
    const int V = (E + 63) >> 6;
    // every load in bounds (clamped to expert E-1), none under a branch, so
    // that all sixteen are in flight together; the ones past the lane's
    // experts are discarded
    int t[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        t[j] = g.row_count[min(lane * V + j, E - 1)];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = lane * V + j;
        t[j] = (j < V && e < E) ? (max(t[j], 0) + BM - 1) / BM * nN : 0;
        sum += t[j];
    }
    const int incl = wave_incl_scan(sum);
    const int W = __builtin_amdgcn_readlane(incl, 63);
    const int w = xcd_remap(blockIdx.x, W);
    if (lane == 0)
        *s_e = -1;
    if (w >= 0 && w >= incl - sum && w < incl) {
        int acc = incl - sum;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            // the tile ranges are disjoint: exactly one (lane, j) holds w
            if (w >= acc && w < acc + t[j]) {
                *s_e = lane * V + j;
                *s_local = w - acc;
            }
            acc += t[j];
        }
    }
}

// Exchange with the lane of the quad that CTRL (a quad_perm) names.
template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// 4x4 transpose inside a lane quad.  On entry lane c (= lane % 4) holds
// v[q] = M[q][c]; returns row c of M, columns 0..3, as four bf16 (RNE),
// lowest column first.  Every lane of the wave must take part.
__device__ __forceinline__ uint2 quad_transpose_bf16(const float v[4], int c)
{
    // with lane c^2: keep rows rb, rb+1 (rb = 2 for c >= 2, else 0)
    const bool hi = c & 2;
    const float r0 = quad_dpp<0x4E>(hi ? v[0] : v[2]); // M[rb][c^2]
    const float r1 = quad_dpp<0x4E>(hi ? v[1] : v[3]); // M[rb+1][c^2]
    const float x0 = hi ? v[2] : v[0], x1 = hi ? v[3] : v[1]; // M[rb][c], M[rb+1][c]
    // with lane c^1: keep row R = rb + (c & 1)
    const bool odd = c & 1;
    const float u0 = quad_dpp<0xB1>(odd ? x0 : x1); // M[R][c^1]
    const float u1 = quad_dpp<0xB1>(odd ? r0 : r1); // M[R][c^3]
    const float k0 = odd ? x1 : x0, k1 = odd ? r1 : r0; // M[R][c], M[R][c^2]
    float o[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        const int dlt = cc ^ c;
        o[cc] = dlt == 0 ? k0 : dlt == 1 ? u0 : dlt == 2 ? k1 : u1;
    }
    return make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
}

// SiLU(g) * u ("MoE Expert Parallelism Sizing: Traffic, Capacity, Fabric",
// the gated three-matrix expert) with the hardware base-2 exponential and
// reciprocal: g * u / (1 + 2^(-g log2 e)).  Each is within about one unit in
// the last place of fp32, far below the bf16 rounding of h that follows; the
// IEEE division and range-reduced exponential took about half of the gate/up
// epilogue.  Large negative g gives 2^(+inf) = inf and a product of 0, as the
// exact function does.
__device__ __forceinline__ float silu_mul(float g, float u)
{
    const float t = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.f + t) * u;
}

// A8: the A operand is E4M3 codes with one fp32 scale per row (FP8
// dispatch); its fragments are widened to bf16 (exact) before the MFMA and
// the row scale multiplies the fp32 sums in the epilogue.
// MINB: workgroups per CU the register budget must allow (RING * MINB fits
// the CU's 160 KB of LDS).
template <int BM, int BN, int BK, int RING, int MINB, int WM, int WN, bool DUAL, bool A8>
__global__ __launch_bounds__(WM * WN * 64, MINB) void grouped_gemm_kernel(GemmArgs g)
{
    constexpr int NW = WM * WN; // waves per workgroup
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static_assert(!A8 || BK == 64, "the E4M3 A path reads both 32-deep halves of a 64-deep step");
    constexpr int RC = BK / 8;                        // 16-byte B pieces per row and step
    constexpr int RPI = 64 / RC;                      // B rows filled by one wave-wide load
    constexpr int A_EB = A8 ? 1 : 2;                  // bytes per A element
    constexpr int RC_A = BK * A_EB / 16;              // 16-byte A pieces per row and step
    constexpr int RPI_A = 64 / RC_A;                  // A rows filled by one wave-wide load
    constexpr int NB = DUAL ? 2 * BN : BN;            // B rows per stage
    constexpr int A_PW = BM / RPI_A / NW, B_PW = NB / RPI / NW; // loads per wave per stage
    static_assert(A_PW * RPI_A * NW == BM && B_PW * RPI * NW == NB, "whole loads per wave");
    constexpr int B_BYTES = NB * BK * 2;
    constexpr int WTN = BN / WN;                      // wave tile columns
    constexpr int RT = BM / 16 / WM, CT = WTN / 16;   // 16x16 MFMA tiles per wave
    static_assert(2 * (BM * BK * A_EB + B_BYTES) <= RING, "two full stages fit in the ring");
    // Wave (wm, wn) owns the 16-row slices wm, wm+WM, wm+2*WM, ... of the tile
    // (interleaved, so a partly filled tile keeps every wave busy) and the
    // columns [wn*WTN, (wn+1)*WTN).
    __shared__ __attribute__((aligned(1024))) char smem[RING];
    __shared__ int s_e, s_local;

    if (threadIdx.x < 64)
        decode_work<BM>(g, g.N / BN, &s_e, &s_local);
    __syncthreads();
    // tile facts are wave-uniform; readfirstlane lets the compiler keep them in
    // scalar registers and branch on them without exec masking
    const int e = __builtin_amdgcn_readfirstlane(s_e);
    if (e < 0)
        return;
    const int local = __builtin_amdgcn_readfirstlane(s_local);
    const int cnt = __builtin_amdgcn_readfirstlane(max(g.row_count[e], 0));
    // The expert's rows are cut into mt tiles of (nearly) equal size rather
    // than full tiles plus a remainder: the M tiles that share a weight tile
    // run side by side, and equal tiles keep them in step, so the weights
    // they read are still in L2 when the others ask for them.
    const int mt = (cnt + BM - 1) / BM;
    const int n_tile = local / mt, m_tile = local % mt;
    const int tile_rows = (cnt + mt - 1) / mt; // <= BM; the last tile is never empty
    const int m0 = m_tile * tile_rows;
    const int offset = __builtin_amdgcn_readfirstlane(g.row_offset[e]);
    // Offsets and counts come from the caller: a tile's rows are clipped to
    // the buffers' rows (as moe_dispatch writes them nothing is clipped), and
    // a tile left with none, or of an offset below 0, stores nothing.
    const int rows_valid = offset < 0 ? 0
                                      : (int)min((long long)min(tile_rows, cnt - m0),
                                                 g.rows - ((long long)offset + m0));
    if (rows_valid <= 0)
        return;
    const size_t row0 = (size_t)offset + m0;
    const int n0 = n_tile * BN;
    const int N = g.N, K = g.K;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // Load descriptors.  Load j of wave w fills rows [(NW*j + w) * RPI, +RPI) of
    // its region; lane l writes piece l % RC of row l / RC, i.e. it fetches
    // source piece (l % RC) ^ swz(row).  A loads whose rows all lie past the
    // expert's end are skipped (wave-uniform); a row past the end inside a
    // partly valid load reads row 0 of the tile instead (never multiplied
    // into a stored result).
    const char *asrc[A_PW];
    const uint16_t *bsrc[B_PW];
    int a_loads = 0; // loads this wave issues per stage for A
#pragma unroll
    for (int j = 0; j < A_PW; ++j) {
        const int grp = NW * j + wave;
        const int r = grp * RPI_A + lane / RC_A;
        const int piece = (lane % RC_A) ^ swz<RC_A>(r);
        const int rr = r < rows_valid ? r : 0;
        asrc[j] = reinterpret_cast<const char *>(g.A) + ((row0 + rr) * K) * A_EB + piece * 16;
        a_loads += (grp * RPI_A < rows_valid) ? 1 : 0;
    }
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
        const int grp = NW * j + wave;
        const int r = grp * RPI + lane / RC;
        const int piece = (lane % RC) ^ swz<RC>(r);
        const uint16_t *base = (DUAL && r >= BN) ? g.B1 : g.B0;
        const int rr = (DUAL && r >= BN) ? r - BN : r;
        bsrc[j] = base + ((size_t)e * N + n0 + rr) * K + piece * 8;
    }
    const int loads_per_stage = a_loads + B_PW;
    // A stage holds only the A rows that carry data (whole 1 KB loads), then
    // the B rows; the ring takes as many stages as fit (2 .. 8), so a tile
    // with fewer rows keeps more K steps in flight.  A tile of more than 192
    // rows keeps two: its MFMA work per step already covers the load of the
    // next, and a third stage in flight measured slower (E4M3 rows, whose
    // full tiles would fit three: Mixtral gate/up 2.01 -> 1.85 ms).
    const int a_bytes = ((rows_valid + RPI_A - 1) / RPI_A) * 1024;
    const int stage = a_bytes + B_BYTES;
    const int S = min(rows_valid > 192 ? 2 : 8, RING / stage);

    // K walk.  When the B rows lie a multiple of 4 KB apart, workgroups that
    // read the same 128-byte column of every row at the same time load a
    // few HBM channels only; starting each N tile's walk at its own step
    // spreads them.  The M tiles of one N tile keep one start, so they stay
    // in step and share the weight tile in L2.  The sum over K is then
    // taken in the rotated (but fixed) order.
    const int nsteps = K / BK;
    const int krot = g.rot ? (n_tile * 5) % nsteps : 0;
    // Weight tiles are loaded non-temporal, A rows normally: all N tiles of
    // an expert re-read the same A rows from L2, and weight lines would
    // otherwise push those out.  The non-temporal path also streams faster
    // from HBM (a plain read probe: 7.0 against 6.2 TB/s).
    const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS char *)smem;
    auto issue = [&](int step, int slot) {
        const uint32_t st = lds_base + slot * stage;
        const int ks = step + krot;
        const int k0 = (ks < nsteps ? ks : ks - nsteps) * BK;
#pragma unroll
        for (int j = 0; j < A_PW; ++j)
            if ((NW * j + wave) * RPI_A < rows_valid)
                dma16(asrc[j] + k0 * A_EB, st + (NW * j + wave) * 1024);
#pragma unroll
        for (int j = 0; j < B_PW; ++j)
            dma16<true>(bsrc[j] + k0, st + a_bytes + (NW * j + wave) * 1024);
    };

    for (int u = 0; u < S - 1 && u < nsteps; ++u)
        issue(u, u);

    // The main loop and epilogue for a wave that multiplies NA 16-row slices
    // (its first NA slices hold rows; the rest lie past the expert's end).
    // NA is a compile-time constant, so no MFMA sits under a branch.  S2
    // fixes the ring at two stages at compile time (the large tiles, which
    // take two): the load wait and the slot updates are then constants, which
    // took the MFMA-bound Mixtral-shaped gate/up GEMM 2-4% faster.
    auto run = [&](auto na_const, auto s2_const) {
        constexpr int NA = decltype(na_const)::value;
        constexpr bool S2 = decltype(s2_const)::value;
        const int SS = S2 ? 2 : S;
        floatx4 acc0[NA > 0 ? NA : 1][CT], acc1[(DUAL && NA > 0) ? NA : 1][DUAL ? CT : 1];
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                acc0[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
                if constexpr (DUAL)
                    acc1[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        // ring slots of stage st and of stage st + S - 1, advanced without
        // a division (S is a run-time value; a modulo per step cost the
        // MFMA-bound Mixtral gate/up 3.5%)
        int rslot = 0, wslot = SS - 1;
        for (int st = 0; st < nsteps; ++st) {
            // stages st+1 .. st+S-2 may stay in flight; stage st must have landed
            if constexpr (S2) {
                wait_vmcnt(0);
            } else {
                const int ahead = min(SS - 2, nsteps - 1 - st);
                wait_vmcnt(ahead * loads_per_stage);
            }
            ring_barrier();
            if (st + SS - 1 < nsteps)
                issue(st + SS - 1, wslot);
            if constexpr (NA > 0) {
                const char *As = smem + rslot * stage;
                const char *Bs = As + a_bytes;
                // Fragment reads are software-pipelined: the A fragment of the
                // next slice (and, before the last slice of a 32-deep step,
                // the B fragments of the next step) is read while the MFMAs of
                // the current slice run, so LDS latency hides under them.
                constexpr int KC = RC / 4;           // 32-deep MFMA steps per stage
                constexpr int NBF = DUAL ? 2 * CT : CT; // B fragments per MFMA step
                auto read_b = [&](int kc, bf16x8 *dst) {
                    const int piece = 4 * kc + (lane >> 4);
#pragma unroll
                    for (int j = 0; j < CT; ++j) {
                        const int n = wn * WTN + j * 16 + (lane & 15);
                        dst[j] = *reinterpret_cast<const bf16x8 *>(
                            Bs + n * (BK * 2) + ((piece ^ swz<RC>(n)) << 4));
                        if constexpr (DUAL) {
                            const int n1 = BN + n;
                            dst[CT + j] = *reinterpret_cast<const bf16x8 *>(
                                Bs + n1 * (BK * 2) + ((piece ^ swz<RC>(n1)) << 4));
                        }
                    }
                };
                auto read_a = [&](int kc, int i) {
                    const int piece = 4 * kc + (lane >> 4);
                    const int r = (wm + WM * i) * 16 + (lane & 15);
                    return *reinterpret_cast<const bf16x8 *>(As + r * (BK * 2) +
                                                             ((piece ^ swz<RC>(r)) << 4));
                };
                if constexpr (A8) {
                    // E4M3 A: per slice, lane group q = lane/16 reads the 8
                    // codes of each 32-deep MFMA step it needs (k = 8q.. and
                    // 32+8q..) once; the first feed step 0, the second wait
                    // in registers for step 1.  B is read as in the bf16 path.
                    auto read_b8 = [&](int kc, int j) {
                        const int piece = 4 * kc + (lane >> 4);
                        const int n = (j < CT ? 0 : BN - CT * 16) + wn * WTN + j * 16 + (lane & 15);
                        return *reinterpret_cast<const bf16x8 *>(
                            Bs + n * (BK * 2) + ((piece ^ swz<RC>(n)) << 4));
                    };
                    auto read_a8 = [&](int i) {
                        // codes k = 8q .. 8q+7 (step 0) and 32+8q .. 32+8q+7
                        // (step 1): two 8-byte halves of 16-byte pieces
                        const int r = (wm + WM * i) * 16 + (lane & 15);
                        const int q = lane >> 4;
                        const char *row = As + r * (BK * A_EB) + 8 * (q & 1);
                        const uint2 a = *reinterpret_cast<const uint2 *>(
                            row + (((q >> 1) ^ swz<RC_A>(r)) << 4));
                        const uint2 b = *reinterpret_cast<const uint2 *>(
                            row + (((2 + (q >> 1)) ^ swz<RC_A>(r)) << 4));
                        return make_uint4(a.x, a.y, b.x, b.y);
                    };
                    auto widen = [&](uint32_t a, uint32_t b) {
                        const uint2 x = e4m3x4_to_bf16x4(a), y = e4m3x4_to_bf16x4(b);
                        return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, y.x, y.y));
                    };
                    bf16x8 b0[NBF], b1[NBF], hi[NA];
#pragma unroll
                    for (int j = 0; j < NBF; ++j)
                        b0[j] = read_b8(0, j);
                    // A pieces are read two slices ahead and widened one
                    // slice ahead, so neither the LDS latency nor the
                    // conversion sits in front of a slice's MFMAs
                    uint4 raw = read_a8(0), raw_next = raw;
                    if (NA > 1)
                        raw_next = read_a8(1);
                    bf16x8 lo = widen(raw.x, raw.y);
                    hi[0] = widen(raw.z, raw.w);
                    // step 0: per slice, the next reads, the next slice's
                    // widening, then 8 MFMAs on the current low half; the
                    // high halves wait in registers for step 1
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                        uint4 raw2 = raw_next;
                        if (i + 2 < NA)
                            raw2 = read_a8(i + 2);
#pragma unroll
                        for (int j = i * NBF / NA; j < (i + 1) * NBF / NA; ++j)
                            b1[j] = read_b8(1, j);
                        bf16x8 lo_next = lo;
                        if (i + 1 < NA) {
                            lo_next = widen(raw_next.x, raw_next.y);
                            hi[i + 1] = widen(raw_next.z, raw_next.w);
                        }
#pragma unroll
                        for (int j = 0; j < CT; ++j) {
                            acc0[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                lo, b0[j], acc0[i][j], 0, 0, 0);
                            if constexpr (DUAL)
                                acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    lo, b0[CT + j], acc1[i][j], 0, 0, 0);
                        }
                        lo = lo_next;
                        raw_next = raw2;
                    }
                    // step 1: no LDS reads
#pragma unroll
                    for (int i = 0; i < NA; ++i)
#pragma unroll
                        for (int j = 0; j < CT; ++j) {
                            acc0[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                hi[i], b1[j], acc0[i][j], 0, 0, 0);
                            if constexpr (DUAL)
                                acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    hi[i], b1[CT + j], acc1[i][j], 0, 0, 0);
                        }
                    __builtin_amdgcn_sched_group_barrier(0x100, NBF + (NA > 1 ? 4 : 2), 0);
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                        constexpr int lo_n = NBF / (NA > 0 ? NA : 1);
                        const int cnt = (i + 2 < NA ? 2 : 0) + (i + 1) * NBF / NA - i * NBF / NA;
                        if (lo_n > 0 && cnt == lo_n)
                            __builtin_amdgcn_sched_group_barrier(0x100, lo_n, 0);
                        else if (cnt == lo_n + 1)
                            __builtin_amdgcn_sched_group_barrier(0x100, lo_n + 1, 0);
                        else if (cnt == lo_n + 2)
                            __builtin_amdgcn_sched_group_barrier(0x100, lo_n + 2, 0);
                        else if (cnt == lo_n + 3)
                            __builtin_amdgcn_sched_group_barrier(0x100, lo_n + 3, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, NBF, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, NA * NBF, 0);
                } else {
                bf16x8 bf[2][NBF], af[2];
                read_b(0, bf[0]);
                af[0] = read_a(0, 0);
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                        const int cur = (kc * NA + i) & 1;
                        if (i + 1 < NA) {
                            af[cur ^ 1] = read_a(kc, i + 1);
                        } else if (kc + 1 < KC) {
                            read_b(kc + 1, bf[(kc + 1) & 1]);
                            af[cur ^ 1] = read_a(kc + 1, 0);
                        }
                        const bf16x8 *b = bf[kc & 1];
#pragma unroll
                        for (int j = 0; j < CT; ++j) {
                            acc0[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                af[cur], b[j], acc0[i][j], 0, 0, 0);
                            if constexpr (DUAL)
                                acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    af[cur], b[CT + j], acc1[i][j], 0, 0, 0);
                        }
                    }
                }
                // Pin that order for the scheduler, which would otherwise sink
                // every fragment read next to its first use: the first reads,
                // then per slice the prefetch reads followed by its MFMAs.
                __builtin_amdgcn_sched_group_barrier(0x100, NBF + 1, 0);
#pragma unroll
                for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                        if (i + 1 < NA)
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        else if (kc + 1 < KC)
                            __builtin_amdgcn_sched_group_barrier(0x100, NBF + 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, NBF, 0);
                    }
                }
            }
            if constexpr (S2) {
                rslot ^= 1;
                wslot ^= 1;
            } else {
                rslot = rslot + 1 == SS ? 0 : rslot + 1;
                wslot = wslot + 1 == SS ? 0 : wslot + 1;
            }
        }

        // Epilogue through LDS.  D layout of a 16x16 MFMA tile: lane holds
        // rows 4*(lane/16)+q (q = 0..3) of column lane%16.  A 4x4 transpose
        // inside each lane quad (two DPP exchanges) gives lane c of a quad row
        // 4*(lane/16)+c of the quad's four columns, packed to bf16 and written
        // to LDS as one 8-byte piece.  LDS rows are LDC elements apart, 32
        // bytes past a multiple of 256, so the 8 rows one write covers per
        // pass fall in distinct banks.  The tile then leaves in 16-byte
        // pieces, each wave store covering whole rows (a third of the time of
        // 32-byte row pieces straight from the quads).  The stores are
        // non-temporal: h and expert_out are read by the next kernel only.
        constexpr int LDC = BN + 16;
        static_assert(BM * LDC * 2 <= RING, "epilogue tile fits in the ring");
        __syncthreads(); // every wave is done with the ring
        uint16_t *Cs = reinterpret_cast<uint16_t *>(smem);
        const int c4 = lane & 3;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int mq = (wm + WM * i) * 16 + 4 * (lane >> 4); // row of q = 0
            float sr[4] = {1.f, 1.f, 1.f, 1.f};
            if (A8 || g.a_scale) { // the rows' dequantization scales (E4M3 rows,
                                   // in registers or widened beforehand)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sr[q] = mq + q < rows_valid ? g.a_scale[row0 + mq + q] : 0.f;
            }
            const int m = mq + c4;
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float gt = acc0[i][j][q] * sr[q];
                    if constexpr (DUAL) {
                        gt = silu_mul(gt, acc1[i][j][q] * sr[q]);
                    }
                    v[q] = gt;
                }
                const uint2 o = quad_transpose_bf16(v, c4);
                const int n = wn * WTN + j * 16 + 4 * ((lane & 15) >> 2);
                *reinterpret_cast<uint2 *>(Cs + m * LDC + n) = o;
            }
        }
        __syncthreads();
        constexpr int CPR = BN / 8; // 16-byte pieces per output row
        for (int c = tid; c < rows_valid * CPR; c += NW * 64) {
            const int r = c / CPR, cc = c % CPR;
            store_nt(reinterpret_cast<uint4 *>(g.out + (row0 + r) * N + n0 + cc * 8),
                     *reinterpret_cast<const uint4 *>(Cs + r * LDC + cc * 8));
        }
    };

    // active slices of this wave: slices wm, wm+WM, ... below rows_valid
    const int slices = (rows_valid + 15) / 16;
    const int n_act = slices > wm ? min(RT, (slices - wm + WM - 1) / WM) : 0;
    static_assert(RT <= 8, "dispatch covers up to 8 slices per wave");
    // two-stage tiles have at least 161 rows, so 5 or more slices per wave
    using F_ = std::false_type;
    using T_ = std::true_type;
    const bool s2 = S == 2;
    switch (n_act) {
    case 0: run(std::integral_constant<int, 0>{}, F_{}); break;
    case 1: run(std::integral_constant<int, (RT >= 1 ? 1 : 0)>{}, F_{}); break;
    case 2: run(std::integral_constant<int, (RT >= 2 ? 2 : 0)>{}, F_{}); break;
    case 3: run(std::integral_constant<int, (RT >= 3 ? 3 : 0)>{}, F_{}); break;
    case 4: run(std::integral_constant<int, (RT >= 4 ? 4 : 0)>{}, F_{}); break;
    case 5: if (s2) run(std::integral_constant<int, (RT >= 5 ? 5 : 0)>{}, T_{}); else run(std::integral_constant<int, (RT >= 5 ? 5 : 0)>{}, F_{}); break;
    case 6: if (s2) run(std::integral_constant<int, (RT >= 6 ? 6 : 0)>{}, T_{}); else run(std::integral_constant<int, (RT >= 6 ? 6 : 0)>{}, F_{}); break;
    case 7: if (s2) run(std::integral_constant<int, (RT >= 7 ? 7 : 0)>{}, T_{}); else run(std::integral_constant<int, (RT >= 7 ? 7 : 0)>{}, F_{}); break;
    default: if (s2) run(std::integral_constant<int, RT>{}, T_{}); else run(std::integral_constant<int, RT>{}, F_{}); break;
    }
}

// Ping-pong grouped GEMM, for shapes bound by the matrix cores (experts of
// hundreds of rows and more).  The tile is 256 rows x 256 weight rows (gate/up:
// 128 columns of W1 and of W3; down: 256 columns), as in the kernel above, and
// each output's K sum runs in the same order, so the results are the same
// bits.
//
// The eight waves form two groups of four, one wave of each on every SIMD;
// group g owns rows [128g, 128g + 128), and wave q of a group owns the weight
// columns 32q.. of W1 and of W3 (gate/up) or 64q.. (down).  The K walk goes in
// units of 32, each two phases separated by workgroup barriers:
//   X_u: group 0 multiplies unit u, group 1 reads unit u's fragments;
//   Y_u: group 0 reads unit u + 1's fragments, group 1 multiplies unit u.
// So on every SIMD one wave keeps the matrix cores busy while the other reads
// LDS.  The direct-to-LDS loads go out from the reading group only: a load
// issued between a wave's MFMAs held that wave up (a probe of this loop: 0.87
// of the matrix-core peak at the held clock this way, 0.74 with the loads
// spread between the MFMAs, 0.75 for the kernel above).
//
// LDS (all 160 KB): the weights in three 64-deep stages (128-byte row pieces,
// as HBM wants them; 32 KB each), loaded by group 0; the tile's rows in four
// 32-deep units (16 KB each), loaded by group 1.  Each phase then carries 16 KB
// of loads, issued by the group that reads in it (a probe took longer phases
// where 32 KB went out in one).  Weight stage s + 3 goes into stage s's slot,
// half at the start of Y_{2s+1} (once both groups have read unit 2s + 1) and
// half at the start of Y_{2s+2}; row unit u + 3 goes into unit u - 1's slot at
// the start of X_u.
__device__ __forceinline__ void pp_barrier()
{
    // keeps the compiler from moving any instruction across the phase boundary
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int BN, bool DUAL>
__global__ __launch_bounds__(512, 1) void grouped_gemm_pp_kernel(GemmArgs g)
{
    constexpr int BM = 256;
    constexpr int NB = DUAL ? 2 * BN : BN;      // weight rows per tile
    static_assert(NB == 256, "256 weight rows per tile");
    constexpr int B_STAGE = NB * 64 * 2;        // 32 KB: 64-deep weight stage
    constexpr int A_UNIT = BM * 32 * 2;         // 16 KB: 32-deep row unit
    constexpr int A_BASE = 3 * B_STAGE;         // row units after the three weight stages
    constexpr int RING = A_BASE + 4 * A_UNIT;   // 160 KB: the whole LDS
    constexpr int LDC = BN + 16;                // epilogue row pitch (elements)
    constexpr int SMEM = RING > BM * LDC * 2 ? RING : BM * LDC * 2;
    constexpr int CT = DUAL ? 2 : 4;            // 16-column tiles per wave and matrix
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];
    // the decoded tile lives in the ring's first bytes until every wave has it
    int *s_tile = reinterpret_cast<int *>(smem);

    if (threadIdx.x < 64)
        decode_work<BM>(g, g.N / BN, s_tile, s_tile + 1);
    __syncthreads();
    const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
    const int local = __builtin_amdgcn_readfirstlane(s_tile[1]);
    __syncthreads();
    if (e < 0)
        return;
    const int cnt = __builtin_amdgcn_readfirstlane(max(g.row_count[e], 0));
    const int mt = (cnt + BM - 1) / BM;
    const int n_tile = local / mt, m_tile = local % mt;
    const int tile_rows = (cnt + mt - 1) / mt;
    const int m0 = m_tile * tile_rows;
    const int offset = __builtin_amdgcn_readfirstlane(g.row_offset[e]);
    const int rows_valid = offset < 0 ? 0
                                      : (int)min((long long)min(tile_rows, cnt - m0),
                                                 g.rows - ((long long)offset + m0));
    if (rows_valid <= 0)
        return;
    const size_t row0 = (size_t)offset + m0;
    const int n0 = n_tile * BN;
    const int N = g.N, K = g.K;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, q = wave & 3;

    // Loads of wave q of its group, load l: L = 4 l + q.
    //  group 0, weight stage (l < 8): rows [8 L, 8 L + 8), lane i writes piece
    //    i % 8 of row i / 8 (source piece (i % 8) ^ swz<8>(row));
    //  group 1, row unit (l < 4): rows [16 L, 16 L + 16), lane i writes piece
    //    i % 4 of row i / 4 (source piece (i % 4) ^ swz<4>(row)); rows past the
    //    tile's end read row 0 of the tile (never stored).
    const char *src[8];
#pragma unroll
    for (int l = 0; l < 8; ++l) {
        const int L = 4 * l + q;
        if (grp == 0) {
            const int r = 8 * L + lane / 8;
            const int piece = (lane % 8) ^ swz<8>(r);
            const uint16_t *base = (DUAL && r >= BN) ? g.B1 : g.B0;
            const int rr = (DUAL && r >= BN) ? r - BN : r;
            src[l] = reinterpret_cast<const char *>(base + ((size_t)e * N + n0 + rr) * K + piece * 8);
        } else {
            const int r = 16 * (L & 15) + lane / 4;
            const int piece = (lane % 4) ^ swz<4>(r);
            const int rr = r < rows_valid ? r : 0;
            src[l] = reinterpret_cast<const char *>(
                reinterpret_cast<const uint16_t *>(g.A) + (row0 + rr) * K + piece * 8);
        }
    }
    // the K walk, rotated as in the kernel above (in 64-deep steps)
    const int S = K / 64, U = 2 * S;
    const int krot = g.rot ? (n_tile * 5) % S : 0;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS char *)smem;
    auto issue_b = [&](int s, int half) { // group 0: half (0, 1) of weight stage s
        const int ks = s + krot < S ? s + krot : s + krot - S;
        const uint32_t st = lds_base + (s % 3) * B_STAGE;
#pragma unroll
        for (int l = 4 * half; l < 4 * half + 4; ++l)
            dma16<true>(src[l] + (size_t)ks * 128, st + (4 * l + q) * 1024);
    };
    auto issue_a = [&](int u) { // group 1: row unit u
        const int s = u >> 1, ks = s + krot < S ? s + krot : s + krot - S;
        const uint32_t st = lds_base + A_BASE + (u & 3) * A_UNIT;
#pragma unroll
        for (int l = 0; l < 4; ++l)
            dma16(src[l] + (size_t)ks * 128 + (u & 1) * 64, st + (4 * l + q) * 1024);
    };

    // fragments: rows 128 grp + 16 i + (lane & 15) and weight rows nb(j) +
    // (lane & 15); the swizzles depend on the lane only
    const int a_lane = A_BASE + (128 * grp + (lane & 15)) * 64 +
                       (((lane >> 4) ^ swz<4>(lane & 15)) << 4);
    const int b_lane = (lane & 15) * 128;
    auto b_row = [&](int j) { // first weight row of fragment j of this wave
        return DUAL ? (j < 2 ? 32 * q + 16 * j : BN + 32 * q + 16 * (j - 2)) : 64 * q + 16 * j;
    };
    uint16_t *Cs = reinterpret_cast<uint16_t *>(smem); // the epilogue's staging
    // The loop and the epilogue's first half for a wave whose group holds NA
    // non-empty 16-row slices (a compile-time value, so no MFMA or fragment
    // read sits under a branch); slices past NA are neither read nor
    // multiplied.  The sequence of barriers does not depend on NA.
    auto body = [&](auto na_const) {
        constexpr int NA = decltype(na_const)::value;
        bf16x8 af[NA > 0 ? NA : 1], bf[4];
        floatx4 acc[NA > 0 ? NA : 1][4];
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        // read: issue the fragment reads of unit u (waited on with read_wait,
        // so that the phase's loads can go out while they are in flight)
        auto read = [&](int u) {
            if constexpr (NA > 0) {
                const char *As = smem + a_lane + (u & 3) * A_UNIT;
                const char *Bs = smem + b_lane + ((u >> 1) % 3) * B_STAGE +
                                 (((4 * (u & 1) + (lane >> 4)) ^ (lane & 7)) << 4);
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    af[i] = *reinterpret_cast<const bf16x8 *>(As + i * 16 * 64);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bf[j] = *reinterpret_cast<const bf16x8 *>(Bs + b_row(j) * 128);
            }
        };
        auto read_wait = [&]() {
            __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8)); // lgkmcnt(0)
        };
        auto mult = [&]() {
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        };
        // prologue: weight stages 0..2, row units 0..3; unit 0 in place
        if (grp == 0) {
            for (int t = 0; t < 3 && t < S; ++t) {
                issue_b(t, 0);
                issue_b(t, 1);
            }
            wait_vmcnt(8 * (min(S, 3) - 1));
        } else {
            for (int u = 0; u < 4 && u < U; ++u)
                issue_a(u);
            wait_vmcnt(4 * (min(U, 4) - 1));
        }
        pp_barrier();
        if (grp == 0) {
            read(0);
            read_wait();
        }
        pp_barrier();
        // The groups run separate loops with the same sequence of barriers, so
        // that no fragment set is merged across branches.
        if (grp == 0) {
            for (int u = 0; u < U; ++u) {
                mult(); // X_u
                if (u & 1) // weight stage s + 1 = (u + 1) / 2 for unit u + 1; s + 2 may be in flight
                    wait_vmcnt((u >> 1) + 2 < S ? 8 : 0);
                pp_barrier();
                // Y_u: the fragment reads of unit u + 1 go out first, then the
                // loads: first half of stage s + 3 (u = 2s + 1), second half of
                // stage s + 2 (u = 2s, s >= 1)
                if (u + 1 < U)
                    read(u + 1);
                if ((u & 1) && (u >> 1) + 3 < S)
                    issue_b((u >> 1) + 3, 0);
                else if (!(u & 1) && u >= 2 && (u >> 1) + 2 < S)
                    issue_b((u >> 1) + 2, 1);
                read_wait();
                pp_barrier();
            }
        } else {
            for (int u = 0; u < U; ++u) {
                read(u); // X_u, then unit u + 3 into unit u - 1's slot
                if (u >= 1 && u + 3 < U)
                    issue_a(u + 3);
                read_wait();
                const int later = min(U - 1, u + 3) - (u + 1); // row unit u + 1 in place
                if (later >= 2)
                    wait_vmcnt(8);
                else if (later == 1)
                    wait_vmcnt(4);
                else
                    wait_vmcnt(0);
                pp_barrier();
                mult(); // Y_u
                pp_barrier();
            }
        }

        // Epilogue through LDS (the ring is free: every unit has been read), as
        // in the kernel above.
        __syncthreads();
        const int c4 = lane & 3;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int mq = 128 * grp + 16 * i + 4 * (lane >> 4); // row of q = 0
            float sr[4] = {1.f, 1.f, 1.f, 1.f};
            if (g.a_scale) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sr[r] = mq + r < rows_valid ? g.a_scale[row0 + mq + r] : 0.f;
            }
            const int m = mq + c4;
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float gt = acc[i][j][r] * sr[r];
                    if constexpr (DUAL)
                        gt = silu_mul(gt, acc[i][2 + j][r] * sr[r]);
                    v[r] = gt;
                }
                const uint2 o = quad_transpose_bf16(v, c4);
                const int n = (DUAL ? 32 * q : 64 * q) + 16 * j + 4 * ((lane & 15) >> 2);
                *reinterpret_cast<uint2 *>(Cs + m * LDC + n) = o;
            }
        }
    };
    // non-empty slices of this wave's group
    const int g_rows = min(max(rows_valid - 128 * grp, 0), 128);
    switch ((g_rows + 15) / 16) {
    case 0: body(std::integral_constant<int, 0>{}); break;
    case 1: body(std::integral_constant<int, 1>{}); break;
    case 2: body(std::integral_constant<int, 2>{}); break;
    case 3: body(std::integral_constant<int, 3>{}); break;
    case 4: body(std::integral_constant<int, 4>{}); break;
    case 5: body(std::integral_constant<int, 5>{}); break;
    case 6: body(std::integral_constant<int, 6>{}); break;
    case 7: body(std::integral_constant<int, 7>{}); break;
    default: body(std::integral_constant<int, 8>{}); break;
    }
    __syncthreads();
    constexpr int CPR = BN / 8; // 16-byte pieces per output row
    for (int c = tid; c < rows_valid * CPR; c += 512) {
        const int r = c / CPR, cc = c % CPR;
        store_nt(reinterpret_cast<uint4 *>(g.out + (row0 + r) * N + n0 + cc * 8),
                 *reinterpret_cast<const uint4 *>(Cs + r * LDC + cc * 8));
    }
}

#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
#ifndef MOE_GU_RING
#define MOE_GU_RING (156 * 1024)
#endif
#ifndef MOE_GU_MINB
#define MOE_GU_MINB 1
#endif
#ifndef MOE_DN_RING
#define MOE_DN_RING (156 * 1024)
#endif
#ifndef MOE_DN_MINB
#define MOE_DN_MINB 1
#endif
#ifndef MOE_GEMM_BN1
#define MOE_GEMM_BN1 128
#endif
#ifndef MOE_GEMM_BN2
#define MOE_GEMM_BN2 256
#endif
#ifndef MOE_GEMM_ROT_GU
#define MOE_GEMM_ROT_GU 0
#endif
#ifndef MOE_GEMM_ROT_DN
#define MOE_GEMM_ROT_DN 1
#endif
#ifndef MOE_GU_BM
#define MOE_GU_BM 256
#endif
#ifndef MOE_DN_BM
#define MOE_DN_BM 256
#endif
constexpr int kBM1 = MOE_GU_BM;       // M tile of the gate/up GEMM
constexpr int kBM2 = MOE_DN_BM;       // and of the down GEMM
constexpr int kBN1 = MOE_GEMM_BN1;    // h columns per gate/up tile (x2 for W1 and W3)
constexpr int kBN2 = MOE_GEMM_BN2;    // output columns per down tile
constexpr int kBK = MOE_GEMM_BK;      // K step
constexpr int kRing1 = MOE_GU_RING;   // LDS ring bytes of a gate/up workgroup
constexpr int kMinB1 = MOE_GU_MINB;   // gate/up workgroups per CU
constexpr int kRing2 = MOE_DN_RING;   // and of the down GEMM
constexpr int kMinB2 = MOE_DN_MINB;
// Eight waves per workgroup, 2 x 4: every wave then needs at most ~220
// registers, so two share a SIMD and one's MFMAs run while the other waits
// on LDS or on its loads (four waves of twice the tile: one per SIMD, 512
// registers each).  Measured against 2 x 2: DeepSeek-V3 gate/up 2.84 -> 2.74
// ms, Mixtral gate/up 1.68 -> 1.62 ms and down 0.88 -> 0.79 ms; 4 x 2 lands
// in between (its waves read more B fragments from LDS).
#ifndef MOE_GU_WM
#define MOE_GU_WM 2
#endif
#ifndef MOE_GU_WN
#define MOE_GU_WN 4
#endif
#ifndef MOE_DN_WM
#define MOE_DN_WM 2
#endif
#ifndef MOE_DN_WN
#define MOE_DN_WN 4
#endif
constexpr int kWM1 = MOE_GU_WM, kWN1 = MOE_GU_WN; // wave grid of a gate/up workgroup
constexpr int kWM2 = MOE_DN_WM, kWN2 = MOE_DN_WN; // and of a down workgroup

// Rotated K walks for B rows of K bf16 values whose pitch is a power of two
// of at least 4 KB (measured: DeepSeek-V3 down GEMM, K = 2048, 1.64 -> 1.61
// ms).  The gate/up GEMM keeps the plain walk: there the N tiles of an expert
// share its rows in L2 only while they walk K together (Mixtral gate/up,
// K = 4096: 1.81 -> 1.92 ms rotated).
int rotate_k(int K)
{
    const int pitch = K * 2;
    return pitch >= 4096 && (pitch & (pitch - 1)) == 0 ? 1 : 0;
}

} // namespace

// E4M3 send rows -> bf16 code values (exact; the row scales stay apart),
// for the rows [0, min(*row_end, rows_max)) that the experts' groups cover.
// Each lane widens 16 codes per pass (one 16-byte load, two 16-byte
// stores), grid-stride.
__global__ __launch_bounds__(256) void widen_e4m3_kernel(const uint4 *__restrict__ codes,
                                                         const int32_t *__restrict__ row_end,
                                                         long long rows_max, int d,
                                                         uint4 *__restrict__ out)
{
    const long long rows = min((long long)*row_end, rows_max);
    const long long n = rows * (d / 16); // 16-code pieces
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (long long)gridDim.x * 256) {
        const uint4 c = load_nt(codes + i);
        const uint2 a = e4m3x4_to_bf16x4(c.x), b = e4m3x4_to_bf16x4(c.y);
        const uint2 e = e4m3x4_to_bf16x4(c.z), f = e4m3x4_to_bf16x4(c.w);
        out[2 * i] = make_uint4(a.x, a.y, b.x, b.y);
        out[2 * i + 1] = make_uint4(e.x, e.y, f.x, f.y);
    }
}

// Launches of fewer tiles than the chip has CUs (small layers: a few
// experts, narrow d or H) take 64-column tiles, so more workgroups stream
// the weights at once.  The estimate of M tiles is the larger of the
// experts that can hold rows and the full tiles the rows need.  Every
// output's K sum runs in one wave in the same order whatever the tile width,
// so the results are the same bits.
constexpr long long kNarrowBelow = 256;
static bool few_tiles(const Dims &dm, int N, int BN, int BM)
{
    const long long mt = std::max<long long>(std::min<long long>(dm.E, dm.send_rows),
                                             (dm.send_rows + BM - 1) / BM);
    return mt * (N / BN) < kNarrowBelow;
}

#ifndef MOE_GEMM_PP
#define MOE_GEMM_PP 1
#endif
// The ping-pong kernel takes the bf16 launches of shapes bound by the matrix
// cores whose tiles fill the chip.
static bool use_pp(const Dims &dm, int N, int BN)
{
    return MOE_GEMM_PP && dm.mfma_bound && N % BN == 0 && !few_tiles(dm, N, BN, 256);
}

template <bool A8>
static void launch_gate_up_t(const Dims &dm, const GemmArgs &a, long long mtiles_max,
                             hipStream_t st)
{
    constexpr int threads = kWM1 * kWN1 * 64;
    if (!A8 && use_pp(dm, dm.H, 128))
        grouped_gemm_pp_kernel<128, true>
            <<<xcd_grid((int)(mtiles_max * (dm.H / 128))), 512, 0, st>>>(a);
    else if (dm.H % kBN1 == 0 && !few_tiles(dm, dm.H, kBN1, kBM1))
        // H is a multiple of 64; the wide tile needs a multiple of kBN1
        grouped_gemm_kernel<kBM1, kBN1, kBK, kRing1, kMinB1, kWM1, kWN1, true, A8>
            <<<xcd_grid((int)(mtiles_max * (dm.H / kBN1))), threads, 0, st>>>(a);
    else
        grouped_gemm_kernel<kBM1, 64, kBK, kRing1, kMinB1, kWM1, kWN1, true, A8>
            <<<xcd_grid((int)(mtiles_max * (dm.H / 64))), threads, 0, st>>>(a);
}

hipError_t launch_gate_up(const Dims &dm, const void *send_buf, const float *send_scale,
                          const int32_t *expert_offset, const int32_t *expert_kept,
                          const uint16_t *w1, const uint16_t *w3, uint16_t *h, uint16_t *a_wide,
                          hipStream_t st)
{
    if (dm.send_rows == 0)
        return hipSuccess;
    const long long mtiles_max = (dm.send_rows + kBM1 - 1) / kBM1 + dm.E;
    GemmArgs a{send_buf, dm.fp8 ? send_scale : nullptr, expert_offset, expert_kept, w1, w3, h,
               dm.E, dm.H, dm.d, MOE_GEMM_ROT_GU ? rotate_k(dm.d) : 0, dm.send_rows};
    if (dm.fp8 && dm.fp8_widen && a_wide) {
        // E4M3 values widened to bf16 (exact), row scales applied in the
        // epilogue as in the E4M3 loop: the same products in the same
        // order, so the same output bits
        widen_e4m3_kernel<<<2048, 256, 0, st>>>(static_cast<const uint4 *>(send_buf),
                                                 expert_offset + dm.E, dm.send_rows, dm.d,
                                                 reinterpret_cast<uint4 *>(a_wide));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        a.A = a_wide;
        launch_gate_up_t<false>(dm, a, mtiles_max, st);
    } else if (dm.fp8) {
        launch_gate_up_t<true>(dm, a, mtiles_max, st);
    } else {
        launch_gate_up_t<false>(dm, a, mtiles_max, st);
    }
    return hipGetLastError();
}

hipError_t launch_down(const Dims &dm, const uint16_t *h, const int32_t *expert_offset,
                       const int32_t *expert_kept, const uint16_t *w2, uint16_t *expert_out,
                       hipStream_t st)
{
    if (dm.send_rows == 0)
        return hipSuccess;
    const long long mtiles_max = (dm.send_rows + kBM2 - 1) / kBM2 + dm.E;
    GemmArgs a{h, nullptr, expert_offset, expert_kept, w2, nullptr, expert_out, dm.E, dm.d, dm.H,
               MOE_GEMM_ROT_DN ? rotate_k(dm.H) : 0, dm.send_rows};
    constexpr int threads = kWM2 * kWN2 * 64;
    if (use_pp(dm, dm.d, 256))
        grouped_gemm_pp_kernel<256, false>
            <<<xcd_grid((int)(mtiles_max * (dm.d / 256))), 512, 0, st>>>(a);
    else if (dm.d % kBN2 == 0 && !few_tiles(dm, dm.d, kBN2, kBM2))
        grouped_gemm_kernel<kBM2, kBN2, kBK, kRing2, kMinB2, kWM2, kWN2, false, false>
            <<<xcd_grid((int)(mtiles_max * (dm.d / kBN2))), threads, 0, st>>>(a);
    else
        grouped_gemm_kernel<kBM2, 64, kBK, kRing2, kMinB2, kWM2, kWN2, false, false>
            <<<xcd_grid((int)(mtiles_max * (dm.d / 64))), threads, 0, st>>>(a);
    return hipGetLastError();
}

// The shared expert (replicated on every rank, "MoE Expert Parallelism
// Sizing: Traffic, Capacity, Fabric", token-assignment worksheet): the same
// two grouped GEMMs with one group of all T tokens, A = x.
__global__ void shared_rows_kernel(int32_t *rows, int T)
{
    if (threadIdx.x == 0) {
        rows[0] = 0; // row_offset[0]
        rows[1] = T; // row_offset[1]
        rows[2] = T; // row_count[0]
    }
}

hipError_t launch_shared_expert(const Dims &dm, const uint16_t *x, const uint16_t *w1s,
                                const uint16_t *w3s, const uint16_t *w2s, uint16_t *shared_out,
                                char *ws, const Workspace &wl, hipStream_t st)
{
    if (dm.T == 0 || dm.shared_H == 0)
        return hipSuccess;
    int32_t *rows = reinterpret_cast<int32_t *>(ws + wl.shared_rows);
    uint16_t *hs = reinterpret_cast<uint16_t *>(ws + wl.shared_h);
    shared_rows_kernel<<<1, 64, 0, st>>>(rows, dm.T);
    Dims ds = dm;
    ds.E = 1;
    ds.H = dm.shared_H;
    ds.send_rows = dm.T;
    ds.fp8 = 0;
    ds.fp8_widen = false;
    ds.mfma_bound = dm.T >= kMfmaBoundRows;
    hipError_t e = launch_gate_up(ds, x, nullptr, rows, rows + 2, w1s, w3s, hs, nullptr, st);
    if (e == hipSuccess)
        e = launch_down(ds, hs, rows, rows + 2, w2s, shared_out, st);
    return e;
}

} // namespace moe
