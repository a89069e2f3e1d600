// Internal declarations of the gfx950 MoE library: device helpers, the
// workspace layout and the kernel launchers called by the C ABI (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// Vector types and bf16 helpers (device side)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// Pack two fp32 values as two bf16 in one 32-bit word (lo first in memory),
// round to nearest even, NaN kept as a quiet NaN (payload's top bits kept,
// quiet bit set): one v_cvt_pk_bf16_f32.  Measured on gfx950 to agree bit for
// bit with the integer rounding u + 0x7fff + ((u >> 16) & 1) (NaN: (u >> 16)
// | 0x40) over every upper half-word with 32 lower ones each, signed zeros,
// denormals, ties and infinities included.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// fp32 -> bf16 bits, rounded as pack_bf16x2 does.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Non-temporal 16- and 8-byte accesses, for data that one kernel touches once:
// rows a gather reads once, and rows a kernel writes for the next kernel
// (hundreds of MB, far beyond the L2).  They keep such lines from pushing
// out of L2 the lines that a kernel does re-read (the GEMMs' A rows).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt(const uint4 *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v)
{
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(p));
}
__device__ __forceinline__ void store_nt(uint2 *p, uint2 v)
{
    __builtin_nontemporal_store(u32x2_t{v.x, v.y}, reinterpret_cast<u32x2_t *>(p));
}

// ---------------------------------------------------------------------------
// FP8 E4M3 (OCP: sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
// finite 448, no infinities) for the dispatch payload.
// ---------------------------------------------------------------------------
// Nearest E4M3 code to v, ties to even, |v| >= 448 saturating to 448, the
// sign bit kept (so -0 and tiny negatives give 0x80).
__device__ __forceinline__ uint32_t e4m3_from_f32(float v)
{
    const uint32_t sgn = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t c;
    if (!(a < 448.f)) {
        c = 0x7Eu;
    } else if (a < 0.015625f) { // below 2^-6: multiples of 2^-9, rounded to even
        c = (uint32_t)__builtin_rintf(a * 512.f);
    } else { // keep 3 mantissa bits, round to nearest even (carry may bump the exponent)
        uint32_t u = __float_as_uint(a);
        u += 0x7FFFFu + ((u >> 20) & 1u);
        c = (u - (120u << 23)) >> 20; // exponent bias 127 -> 7
    }
    return c | sgn;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Four E4M3 codes (one per byte of w, lowest first) as four bf16 (two
// packed pairs).  The gfx950 packed fp8 -> fp32 conversion decodes two codes
// at a time; every E4M3 value has at most 4 significant bits, so its fp32
// image's upper half is the exact bf16, and one byte permute packs two.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w)
{
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false); // codes 0, 1
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);  // codes 2, 3
    return make_uint2(
        __builtin_amdgcn_perm(__float_as_uint(a.y), __float_as_uint(a.x), 0x07060302u),
        __builtin_amdgcn_perm(__float_as_uint(b.y), __float_as_uint(b.x), 0x07060302u));
}

// ---------------------------------------------------------------------------
// Sizes shared by host and kernels
// ---------------------------------------------------------------------------
constexpr int kChunk = 256;      // tokens per histogram chunk (one per thread)
constexpr int kMaxExperts = 1024; // E limit of the LDS bitmaps and scans

// Derived per-call shape facts (host side).
struct Dims {
    int T, d, E, k, H, D, my_rank;
    int drop_policy;   // 0: token order, 1: by gate value (capacity mode only)
    int fp8;           // dispatch payload: 0 bf16 rows, 1 E4M3 rows + fp32 row scales
    int n_groups;      // expert groups for group-limited routing (<= 1: none)
    int group_limit;   // groups a token may use (routing is limited iff < n_groups)
    int shared_H;      // shared expert's SwiGLU hidden size (0: none)
    int64_t capacity;  // C, or -1 when dropless
    int64_t send_rows; // E*C or T*k
    int nchunks;       // ceil(T / kChunk)
    // An expert is expected to hold at least kMfmaBoundRows rows: the
    // grouped GEMMs are then bound by the matrix cores and take the
    // ping-pong kernel.
    bool mfma_bound;
    // E4M3 rows are widened to bf16 in a separate pass before the gate/up
    // GEMM (given a workspace) on such shapes: the bf16 loop runs faster
    // than the loop that widens in registers.
    bool fp8_widen;
};
constexpr int64_t kMfmaBoundRows = 512;

// Byte offsets of each region inside the caller's workspace.
struct Workspace {
    size_t logits;        // fp32 [SK, T, E_pad] router partial logits (SK = router_ksplit)
    size_t wg_pad;        // bf16 [d, E8]       W_g with rows padded to 8 experts (E % 8 != 0)
    size_t chunk_counts;  // int32 [nchunks, E] per-chunk expert counts
    size_t chunk_base;    // int32 [nchunks, E] exclusive scan of the counts over chunks
    size_t chunk_invalid; // int32 [nchunks]    invalid entries per chunk
    size_t all_offset;    // int32 [E]          exclusive scan of n_e (drop policy 1)
    size_t by_expert;     // int32 [T*k]        assignments grouped by expert (drop policy 1)
    size_t h;             // bf16 [send_rows, H] SwiGLU hidden activations
    size_t a_wide;        // bf16 [send_rows, d] E4M3 send rows widened (fp8_widen only)
    size_t shared_rows;   // int32 [4]          row offsets/count of the shared expert's one group
    size_t shared_h;      // bf16 [T, shared_H] the shared expert's hidden activations
    size_t total;
};

Workspace workspace_layout(const Dims &dm);

// ---------------------------------------------------------------------------
// Launchers (return hipGetLastError() of their launches)
// ---------------------------------------------------------------------------
int router_ksplit(int T, int E, int d); // K slices of the logit GEMM
bool router_partials(int T, int E, int d); // the logit GEMM stores partial sums (S * n_et > 1)
int router_epad(int E);                 // E rounded up to 64
int router_ldw(int E);                  // W_g row length the router reads (E rounded up to 8)
hipError_t launch_route(const Dims &dm, const uint16_t *x, const uint16_t *w_gate,
                        const float *bias, float *logits_out, int32_t *topk_idx, float *topk_w,
                        char *ws, const Workspace &wl, hipStream_t st);
hipError_t launch_topk_softmax(const Dims &dm, const float *logits, int32_t *topk_idx,
                               float *topk_w, hipStream_t st);
hipError_t launch_dispatch(const Dims &dm, const uint16_t *x, const int32_t *topk_idx,
                           const float *topk_w, void *send_buf, float *send_scale, int32_t *slot, int32_t *expert_count,
                           int32_t *expert_kept, int32_t *expert_offset, int32_t *rank_rows,
                           moe_stats *stats, char *ws, const Workspace &wl, hipStream_t st);
// a_wide: NULL, or (with dm.fp8_widen) room for the widened E4M3 rows
hipError_t launch_gate_up(const Dims &dm, const void *send_buf, const float *send_scale,
                          const int32_t *expert_offset,
                          const int32_t *expert_kept, const uint16_t *w1, const uint16_t *w3,
                          uint16_t *h, uint16_t *a_wide, hipStream_t st);
hipError_t launch_down(const Dims &dm, const uint16_t *h, const int32_t *expert_offset,
                       const int32_t *expert_kept, const uint16_t *w2, uint16_t *expert_out,
                       hipStream_t st);
hipError_t launch_combine(const Dims &dm, const uint16_t *expert_out, const int32_t *slot,
                          const float *topk_w, const uint16_t *shared_out, uint16_t *y,
                          hipStream_t st);
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_stream_write(void *dst, size_t bytes, uint32_t value, hipStream_t st);
hipError_t launch_stream_gather(const void *rows, long long nrows, int d, const int32_t *slot,
                                int T, int k, void *out, hipStream_t st);
hipError_t launch_shared_expert(const Dims &dm, const uint16_t *x, const uint16_t *w1s,
                                const uint16_t *w3s, const uint16_t *w2s, uint16_t *shared_out,
                                char *ws, const Workspace &wl, hipStream_t st);
// scales NULL: every row's scale is 1 (the E4M3 values themselves, exact in bf16)
hipError_t launch_fp8_rows_to_bf16(const uint8_t *codes, const float *scales, long long rows,
                                   int d, uint16_t *out, hipStream_t st);

// XCD-aware block remap: the chip dispatches consecutive workgroups to its 8
// XCDs round robin; this turns block b into a logical work index so that each
// XCD walks one contiguous range of the work list (neighbouring tiles, which
// share operands, then meet in the same L2).  Returns -1 for surplus blocks.
// The grid must hold at least 8 * ceil(total / 8) blocks.
__device__ __forceinline__ int xcd_remap(int b, int total)
{
    const int per = (total + 7) >> 3;
    const int idx = b >> 3;
    if (idx >= per)
        return -1;
    const int w = (b & 7) * per + idx;
    return w < total ? w : -1;
}

inline int xcd_grid(int total) { return ((total + 7) / 8) * 8; }

// Wavefronts that share one token's row in the combine (and its gather
// probe): one per token when the tokens alone give the launch 4096
// wavefronts (16 per CU), else enough to reach that, each keeping at least
// 64 of the row's 16-byte pieces (one per lane), at most 16.
inline int combine_waves_per_token(int T, int d)
{
    const int most = d / 8 / 64 < 16 ? d / 8 / 64 : 16;
    const int want = T > 0 ? (4096 + T - 1) / T : 1;
    const int w = want < most ? want : most;
    return w < 1 ? 1 : w;
}

} // namespace moe
